"""Helpers for the GPU parity tests: host<->device copies of seeded inputs and the error metric."""
import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> CUDA tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the parity metric)."""
    got, ref = as64(got) if got.dtype == np.uint16 else got.astype(np.float64), ref.astype(np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


TOL = {"bf16": 1e-2, "f32": 1e-5}
