"""MI355X (gfx950) MoE expert layer with renormalised top-k routing — Python binding.

Thin ctypes marshalling over the C ABI of libmoe_rocm.so (declared in include/moe_rocm.h). Every
step of the layer runs in the library's HIP kernels; PyTorch only provides device memory and the
current stream. There is no fallback: if the library is missing or a call fails, this raises.

The functions carry the ABI's names and take torch tensors on the GPU. Output tensors may be
passed in (they are then written in place) or are allocated here with torch.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZE_LIB=1 loads the host-sanitized build (tests/sanitizers.py); nothing else does
LIB_PATH = os.path.join(_PKG, "libmoe_rocm_san.so" if os.environ.get("MOE_SANITIZE_LIB") == "1" else "libmoe_rocm.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "moe_rocm.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libmoe_rocm.so (built in-tree by build.py). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run mixture_experts_layer_renorm_amd/build.py "
                              "(or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_abi_version": (I, []),
            "moe_router_logits": (I, [P, P, I, I, I, I, P, P]),
            "moe_router_topk": (I, [P, I, I, I, I, P, P, P]),
            "moe_router_stats_workspace_bytes": (Z, [I, I]),
            "moe_router_stats": (I, [P, P, I, I, I, P, P, P, P, Z, P]),
            "moe_permute_workspace_bytes": (Z, [I, I, I]),
            "moe_permute": (I, [P, I, I, I, P, I, I, P, P, P, P, P, P, Z, P]),
            "moe_permute_noalloc": (I, [P, I, I, I, P, I, I, P, P, P, P, P, P]),
            "moe_router_topk_permute": (I, [P, I, I, I, I, P, P, P, I, I, P, P, P, P, P, P, Z, P]),
            "moe_grouped_swiglu_ffn": (I, [P, P, P, I, I, I, I, I, P, P, P, P, P]),
            "moe_grouped_gemm_swiglu": (I, [P, P, I, I, I, I, I, P, P, P, P]),
            "moe_grouped_gemm_down": (I, [P, P, I, I, I, I, I, P, P, P]),
            "moe_grouped_gemm_swiglu_gather": (I, [P, P, I, I, P, I, I, I, I, I, P, P, P, P]),
            "moe_grouped_swiglu_ffn_gather": (I, [P, P, I, I, P, P, I, I, I, I, I, P, P, P, P, P]),
            "moe_unpermute_combine": (I, [P, I, I, I, I, P, P, P, P, P]),
            "moe_unpermute_combine_bwd": (I, [P, P, I, I, I, I, P, P, P, P, P]),
            "moe_grouped_swiglu_ffn_bwd": (I, [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P]),
            "moe_grouped_gemm_down_bwd": (I, [P, P, P, I, I, I, I, I, P, P, P]),
            "moe_grouped_gemm_gate_up_bwd": (I, [P, P, I, I, I, I, I, P, P, P]),
            "moe_grouped_gemm_wgrad": (I, [P, P, I, I, I, I, I, P, P, I, P]),
            "moe_permute_bwd": (I, [P, I, I, I, I, P, P, P, P]),
            "moe_router_topk_bwd": (I, [P, P, P, P, I, I, I, I, P, P]),
            "moe_router_logits_bwd": (I, [P, P, P, I, I, I, I, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/moe_rocm.h."""
    with open(HEADER) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe_\w+)\s*\(", src, re.M)))


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, load_library().moe_last_error().decode() or what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t, what, dtype=None, shape=None):
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# ---- the ABI calls ----------------------------------------------------------------------------
def moe_router_logits(x, w_gate, logits=None, stream=None):
    T, H = x.shape
    E = w_gate.shape[1]
    _need(x, "x"), _need(w_gate, "w_gate", x.dtype, (H, E))
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _need(logits, "logits", torch.float32, (T, E))
    _check(load_library().moe_router_logits(_ptr(x), _ptr(w_gate), _dt(x), T, H, E, _ptr(logits), _stream(stream)),
           "moe_router_logits")
    return logits


def moe_router_topk(logits, k, renorm=True, topk_idx=None, topk_w=None, stream=None):
    T, E = logits.shape
    _need(logits, "logits", torch.float32)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need(topk_idx, "topk_idx", torch.int32, (T, k)), _need(topk_w, "topk_w", torch.float32, (T, k))
    _check(load_library().moe_router_topk(_ptr(logits), T, E, k, int(bool(renorm)), _ptr(topk_idx), _ptr(topk_w),
                                          _stream(stream)), "moe_router_topk")
    return topk_idx, topk_w


def moe_permute_workspace_bytes(T, k, E):
    return int(load_library().moe_permute_workspace_bytes(T, k, E))


class Plan:
    """The permute's layout handle: counts, offsets, row_of_slot, slot_of_row (all int32, device)."""

    def __init__(self, counts, offsets, row_of_slot, slot_of_row):
        self.counts, self.offsets, self.row_of_slot, self.slot_of_row = counts, offsets, row_of_slot, slot_of_row


def moe_router_stats_workspace_bytes(T, E):
    return int(load_library().moe_router_stats_workspace_bytes(T, E))


def moe_router_stats(logits, topk_idx, want_probs=True, probs=None, mean_prob=None, load=None, workspace=None,
                     stream=None):
    """Full softmax per token (optional), its mean over tokens and the per-expert load, for an
    auxiliary load-balance loss. Returns (probs or None, mean_prob [E] fp32, load [E] int32)."""
    T, E = logits.shape
    k = topk_idx.shape[1]
    _need(logits, "logits", torch.float32, (T, E)), _need(topk_idx, "topk_idx", torch.int32, (T, k))
    dev = logits.device
    if want_probs and probs is None:
        probs = torch.empty((T, E), dtype=torch.float32, device=dev)
    if not want_probs:
        probs = None
    if mean_prob is None:
        mean_prob = torch.empty(E, dtype=torch.float32, device=dev)
    if load is None:
        load = torch.empty(E, dtype=torch.int32, device=dev)
    ws = moe_router_stats_workspace_bytes(T, E)
    if workspace is None:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _check(load_library().moe_router_stats(_ptr(logits), _ptr(topk_idx), T, E, k, _ptr(probs), _ptr(mean_prob),
                                           _ptr(load), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_router_stats")
    return probs, mean_prob, load


def moe_permute(x, topk_idx, E, x_perm=None, plan=None, workspace=None, stream=None, rows=True):
    """rows=False computes the plan only (no x_perm; for the gathering FFN) and returns (None, plan)."""
    T, H = x.shape
    k = topk_idx.shape[1]
    _need(x, "x"), _need(topk_idx, "topk_idx", torch.int32, (T, k))
    dev = x.device
    N = T * k
    if not rows:
        x_perm = None
    elif x_perm is None:
        x_perm = torch.empty((N, H), dtype=x.dtype, device=dev)
    if plan is None:
        plan = Plan(torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
                    torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev))
    ws_bytes = moe_permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(load_library().moe_permute(_ptr(x), _dt(x), T, H, _ptr(topk_idx), k, E, _ptr(x_perm) if rows else None,
                                      _ptr(plan.counts),
                                      _ptr(plan.offsets), _ptr(plan.row_of_slot), _ptr(plan.slot_of_row),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_permute")
    return x_perm, plan


def moe_permute_noalloc(x, topk_idx, E, x_perm, plan, stream=None, rows=True):
    """moe_permute with the library's fixed device scratch instead of a workspace: allocates
    nothing, so every output (x_perm unless rows=False, the four plan arrays) is passed in."""
    T, H = x.shape
    k = topk_idx.shape[1]
    _need(x, "x"), _need(topk_idx, "topk_idx", torch.int32, (T, k))
    N = T * k
    if rows:
        _need(x_perm, "x_perm", x.dtype)
        if x_perm.shape[0] < N or x_perm.shape[1] != H:
            raise ValueError("x_perm must hold [T*k, H] rows")
    for t, n in [(plan.counts, E), (plan.offsets, E + 1), (plan.row_of_slot, N), (plan.slot_of_row, N)]:
        _need(t, "plan", torch.int32)
        if t.numel() < n:
            raise ValueError("plan arrays too small")
    _check(load_library().moe_permute_noalloc(_ptr(x), _dt(x), T, H, _ptr(topk_idx), k, E,
                                              _ptr(x_perm) if rows else None, _ptr(plan.counts), _ptr(plan.offsets),
                                              _ptr(plan.row_of_slot), _ptr(plan.slot_of_row), _stream(stream)),
           "moe_permute_noalloc")
    return x_perm if rows else None, plan


def moe_router_topk_permute(logits, k, x, E=None, renorm=True, topk_idx=None, topk_w=None, x_perm=None, plan=None,
                            workspace=None, stream=None, rows=True):
    """moe_router_topk then moe_permute in one call (same results bit for bit); rows=False computes
    the plan only. Returns (topk_idx, topk_w, x_perm or None, plan)."""
    T, E = logits.shape
    H = x.shape[1]
    _need(logits, "logits", torch.float32), _need(x, "x")
    if x.shape[0] != T:
        raise ValueError("x must have the logits' T rows")
    dev = logits.device
    N = T * k
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k)), _need(topk_w, "topk_w", torch.float32, (T, k))
    if not rows:
        x_perm = None
    elif x_perm is None:
        x_perm = torch.empty((N, H), dtype=x.dtype, device=dev)
    if plan is None:
        plan = Plan(torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
                    torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev))
    ws_bytes = moe_permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(load_library().moe_router_topk_permute(_ptr(logits), T, E, k, int(bool(renorm)), _ptr(topk_idx),
                                                  _ptr(topk_w), _ptr(x), _dt(x), H, _ptr(x_perm) if rows else None,
                                                  _ptr(plan.counts), _ptr(plan.offsets), _ptr(plan.row_of_slot),
                                                  _ptr(plan.slot_of_row), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_router_topk_permute")
    return topk_idx, topk_w, x_perm, plan


def moe_grouped_swiglu_ffn(x_perm, gate_up, down, expert_offsets, h=None, y=None, gu_saved=None, stream=None):
    N, H = x_perm.shape
    I = down.shape[0] // (gate_up.shape[0] // H)
    E = gate_up.shape[0] // H
    _need(x_perm, "x_perm"), _need(gate_up, "gate_up", x_perm.dtype, (E * H, 2 * I))
    _need(down, "down", x_perm.dtype, (E * I, H)), _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if h is None:
        h = torch.empty((N, I), dtype=x_perm.dtype, device=x_perm.device)
    if y is None:
        y = torch.empty((N, H), dtype=x_perm.dtype, device=x_perm.device)
    _need(h, "h", x_perm.dtype, (N, I)), _need(y, "y", x_perm.dtype, (N, H))
    if gu_saved is not None:
        _need(gu_saved, "gu_saved", x_perm.dtype, (N, 2 * I))
    _check(load_library().moe_grouped_swiglu_ffn(_ptr(x_perm), _ptr(gate_up), _ptr(down), _dt(x_perm), N, H, I, E,
                                                 _ptr(expert_offsets), _ptr(h), _ptr(gu_saved), _ptr(y),
                                                 _stream(stream)), "moe_grouped_swiglu_ffn")
    return y, h


def moe_grouped_gemm_swiglu_gather(x, slot_of_row, k, gate_up, expert_offsets, N=None, h=None, gu_saved=None,
                                   stream=None):
    """First grouped matmul + SwiGLU with the grouped rows gathered from x: row r is token
    slot_of_row[r] // k. N defaults to T*k."""
    T, H = x.shape
    N = T * k if N is None else N
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    _need(x, "x"), _need(slot_of_row, "slot_of_row", torch.int32)
    _need(gate_up, "gate_up", x.dtype, (E * H, 2 * I)), _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if h is None:
        h = torch.empty((N, I), dtype=x.dtype, device=x.device)
    _need(h, "h", x.dtype, (N, I))
    if gu_saved is not None:
        _need(gu_saved, "gu_saved", x.dtype, (N, 2 * I))
    _check(load_library().moe_grouped_gemm_swiglu_gather(_ptr(x), _ptr(slot_of_row), T, k, _ptr(gate_up), _dt(x), N, H,
                                                         I, E, _ptr(expert_offsets), _ptr(h), _ptr(gu_saved),
                                                         _stream(stream)), "moe_grouped_gemm_swiglu_gather")
    return h


def moe_grouped_swiglu_ffn_gather(x, slot_of_row, k, gate_up, down, expert_offsets, N=None, h=None, y=None,
                                  gu_saved=None, stream=None):
    """The grouped SwiGLU FFN with the grouped rows gathered from x (row r is token slot_of_row[r] // k)."""
    T, H = x.shape
    N = T * k if N is None else N
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    _need(x, "x"), _need(slot_of_row, "slot_of_row", torch.int32), _need(gate_up, "gate_up", x.dtype, (E * H, 2 * I))
    _need(down, "down", x.dtype, (E * I, H)), _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if h is None:
        h = torch.empty((N, I), dtype=x.dtype, device=x.device)
    if y is None:
        y = torch.empty((N, H), dtype=x.dtype, device=x.device)
    _need(h, "h", x.dtype, (N, I)), _need(y, "y", x.dtype, (N, H))
    if gu_saved is not None:
        _need(gu_saved, "gu_saved", x.dtype, (N, 2 * I))
    _check(load_library().moe_grouped_swiglu_ffn_gather(_ptr(x), _ptr(slot_of_row), T, k, _ptr(gate_up), _ptr(down),
                                                        _dt(x), N, H, I, E, _ptr(expert_offsets), _ptr(h),
                                                        _ptr(gu_saved), _ptr(y), _stream(stream)),
           "moe_grouped_swiglu_ffn_gather")
    return y, h


def moe_grouped_gemm_swiglu(x_perm, gate_up, expert_offsets, h=None, gu_saved=None, stream=None):
    N, H = x_perm.shape
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    _need(x_perm, "x_perm"), _need(gate_up, "gate_up", x_perm.dtype, (E * H, 2 * I))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if h is None:
        h = torch.empty((N, I), dtype=x_perm.dtype, device=x_perm.device)
    _need(h, "h", x_perm.dtype, (N, I))
    if gu_saved is not None:
        _need(gu_saved, "gu_saved", x_perm.dtype, (N, 2 * I))
    _check(load_library().moe_grouped_gemm_swiglu(_ptr(x_perm), _ptr(gate_up), _dt(x_perm), N, H, I, E,
                                                  _ptr(expert_offsets), _ptr(h), _ptr(gu_saved), _stream(stream)),
           "moe_grouped_gemm_swiglu")
    return h


def moe_grouped_gemm_down(h, down, expert_offsets, y=None, stream=None):
    N, I = h.shape
    E = expert_offsets.shape[0] - 1
    H = down.shape[1]
    _need(h, "h"), _need(down, "down", h.dtype, (E * I, H)), _need(expert_offsets, "expert_offsets", torch.int32)
    if y is None:
        y = torch.empty((N, H), dtype=h.dtype, device=h.device)
    _need(y, "y", h.dtype, (N, H))
    _check(load_library().moe_grouped_gemm_down(_ptr(h), _ptr(down), _dt(h), N, H, I, E, _ptr(expert_offsets),
                                                _ptr(y), _stream(stream)), "moe_grouped_gemm_down")
    return y


def moe_unpermute_combine(y, row_of_slot, topk_w, residual=None, out=None, stream=None):
    T, k = topk_w.shape
    H = y.shape[1]
    _need(y, "y"), _need(row_of_slot, "row_of_slot", torch.int32), _need(topk_w, "topk_w", torch.float32)
    if row_of_slot.numel() != T * k:
        raise ValueError("row_of_slot must hold T*k entries")
    if residual is not None:
        _need(residual, "residual", y.dtype, (T, H))
    if out is None:
        out = torch.empty((T, H), dtype=y.dtype, device=y.device)
    _need(out, "out", y.dtype, (T, H))
    _check(load_library().moe_unpermute_combine(_ptr(y), _dt(y), T, H, k, _ptr(row_of_slot), _ptr(topk_w),
                                                _ptr(residual), _ptr(out), _stream(stream)), "moe_unpermute_combine")
    return out


# ---- backward ----------------------------------------------------------------------------------
def moe_unpermute_combine_bwd(d_out, y, row_of_slot, topk_w, d_y=None, d_w=None, stream=None):
    T, k = topk_w.shape
    H = y.shape[1]
    _need(d_out, "d_out", y.dtype, (T, H)), _need(y, "y"), _need(row_of_slot, "row_of_slot", torch.int32)
    _need(topk_w, "topk_w", torch.float32)
    if d_y is None:
        d_y = torch.empty_like(y)
    if d_w is None:
        d_w = torch.empty((T, k), dtype=torch.float32, device=y.device)
    _need(d_y, "d_y", y.dtype, tuple(y.shape)), _need(d_w, "d_w", torch.float32, (T, k))
    _check(load_library().moe_unpermute_combine_bwd(_ptr(d_out), _ptr(y), _dt(y), T, H, k, _ptr(row_of_slot),
                                                    _ptr(topk_w), _ptr(d_y), _ptr(d_w), _stream(stream)),
           "moe_unpermute_combine_bwd")
    return d_y, d_w


def moe_grouped_swiglu_ffn_bwd(d_y, x_perm, gu_saved, h, gate_up, down, expert_offsets, d_x_perm=None, d_gate_up=None,
                               d_down=None, d_gu=None, stream=None):
    N, H = x_perm.shape
    E = expert_offsets.shape[0] - 1
    I = h.shape[1]
    for t, nme, shp in [(d_y, "d_y", (N, H)), (x_perm, "x_perm", (N, H)), (gu_saved, "gu_saved", (N, 2 * I)),
                        (h, "h", (N, I)), (gate_up, "gate_up", (E * H, 2 * I)), (down, "down", (E * I, H))]:
        _need(t, nme, x_perm.dtype, shp)
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    dev = x_perm.device
    if d_x_perm is None:
        d_x_perm = torch.empty((N, H), dtype=x_perm.dtype, device=dev)
    if d_gate_up is None:
        d_gate_up = torch.empty_like(gate_up)
    if d_down is None:
        d_down = torch.empty_like(down)
    if d_gu is None:
        d_gu = torch.empty((N, 2 * I), dtype=x_perm.dtype, device=dev)
    _check(load_library().moe_grouped_swiglu_ffn_bwd(_ptr(d_y), _ptr(x_perm), _ptr(gu_saved), _ptr(h), _ptr(gate_up),
                                                     _ptr(down), _dt(x_perm), N, H, I, E, _ptr(expert_offsets),
                                                     _ptr(d_x_perm), _ptr(d_gate_up), _ptr(d_down), _ptr(d_gu),
                                                     _stream(stream)), "moe_grouped_swiglu_ffn_bwd")
    return d_x_perm, d_gate_up, d_down, d_gu


def moe_grouped_gemm_down_bwd(d_y, down, gu_saved, expert_offsets, d_gu=None, stream=None):
    """d_gu = SwiGLU backward of d_y @ down_e^T for every expert's rows (first product of the FFN backward)."""
    N, H = d_y.shape
    E = expert_offsets.shape[0] - 1
    I = gu_saved.shape[1] // 2
    _need(down, "down", d_y.dtype, (E * I, H)), _need(gu_saved, "gu_saved", d_y.dtype, (N, 2 * I))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if d_gu is None:
        d_gu = torch.empty((N, 2 * I), dtype=d_y.dtype, device=d_y.device)
    _check(load_library().moe_grouped_gemm_down_bwd(_ptr(d_y), _ptr(down), _ptr(gu_saved), _dt(d_y), N, H, I, E,
                                                    _ptr(expert_offsets), _ptr(d_gu), _stream(stream)),
           "moe_grouped_gemm_down_bwd")
    return d_gu


def moe_grouped_gemm_gate_up_bwd(d_gu, gate_up, expert_offsets, d_x_perm=None, stream=None):
    """d_x_perm = d_gu @ gate_up_e^T for every expert's rows."""
    N = d_gu.shape[0]
    I = d_gu.shape[1] // 2
    E = expert_offsets.shape[0] - 1
    H = gate_up.shape[0] // E
    _need(gate_up, "gate_up", d_gu.dtype, (E * H, 2 * I)), _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if d_x_perm is None:
        d_x_perm = torch.empty((N, H), dtype=d_gu.dtype, device=d_gu.device)
    _check(load_library().moe_grouped_gemm_gate_up_bwd(_ptr(d_gu), _ptr(gate_up), _dt(d_gu), N, H, I, E,
                                                       _ptr(expert_offsets), _ptr(d_x_perm), _stream(stream)),
           "moe_grouped_gemm_gate_up_bwd")
    return d_x_perm


def moe_grouped_gemm_wgrad(P, Q, expert_offsets, d_w=None, max_workgroups=0, stream=None):
    """d_w[e*M:(e+1)*M] = P_e^T @ Q_e over the rows of expert e (P [N, M], Q [N, Nq], rows grouped by
    expert); max_workgroups > 0 caps the CUs the product holds."""
    N, M = P.shape
    Nq = Q.shape[1]
    E = expert_offsets.shape[0] - 1
    _need(Q, "Q", P.dtype, (N, Nq)), _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    if d_w is None:
        d_w = torch.empty((E * M, Nq), dtype=P.dtype, device=P.device)
    _need(d_w, "d_w", P.dtype, (E * M, Nq))
    _check(load_library().moe_grouped_gemm_wgrad(_ptr(P), _ptr(Q), _dt(P), N, M, Nq, E, _ptr(expert_offsets),
                                                 _ptr(d_w), int(max_workgroups), _stream(stream)),
           "moe_grouped_gemm_wgrad")
    return d_w


def moe_permute_bwd(d_x_perm, row_of_slot, T, k, d_x_add=None, d_x=None, stream=None):
    H = d_x_perm.shape[1]
    _need(d_x_perm, "d_x_perm"), _need(row_of_slot, "row_of_slot", torch.int32)
    if d_x_add is not None:
        _need(d_x_add, "d_x_add", d_x_perm.dtype, (T, H))
    if d_x is None:
        d_x = torch.empty((T, H), dtype=d_x_perm.dtype, device=d_x_perm.device)
    _check(load_library().moe_permute_bwd(_ptr(d_x_perm), _dt(d_x_perm), T, H, k, _ptr(row_of_slot), _ptr(d_x_add),
                                          _ptr(d_x), _stream(stream)), "moe_permute_bwd")
    return d_x


def moe_router_topk_bwd(logits, topk_idx, topk_w, d_w, renorm=True, d_logits=None, stream=None):
    T, k = topk_idx.shape
    E = logits.shape[1] if logits is not None else None
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=torch.float32, device=topk_idx.device)
    E = d_logits.shape[1]
    _check(load_library().moe_router_topk_bwd(_ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(d_w), T, E, k,
                                              int(bool(renorm)), _ptr(d_logits), _stream(stream)),
           "moe_router_topk_bwd")
    return d_logits


def moe_router_logits_bwd(x, w_gate, d_logits, d_w_gate=None, d_x_in=None, d_x=None, want_dw=True, want_dx=True,
                          stream=None):
    T, H = x.shape
    E = w_gate.shape[1]
    _need(d_logits, "d_logits", torch.float32, (T, E))
    if want_dw and d_w_gate is None:
        d_w_gate = torch.empty((H, E), dtype=torch.float32, device=x.device)
    if want_dx and d_x is None:
        d_x = torch.empty((T, H), dtype=x.dtype, device=x.device)
    _check(load_library().moe_router_logits_bwd(_ptr(x), _ptr(w_gate), _ptr(d_logits), _dt(x), T, H, E,
                                                _ptr(d_w_gate if want_dw else None), _ptr(d_x_in),
                                                _ptr(d_x if want_dx else None), _stream(stream)),
           "moe_router_logits_bwd")
    return d_w_gate, d_x


# ---- the layer: the five calls in order on one stream ---------------------------------------------
class LayerBuffers:
    """Device buffers of one layer call, allocated once and reused (no allocation in the timed path).
    gu_saved keeps the expert pre-activations for the backward; I_shared > 0 adds the shared expert's
    buffers (its segment offsets {0, T} are copied to the device here, once)."""

    def __init__(self, T, H, I, E, k, dtype, device, logits=True, gu_saved=False, I_shared=0, x_perm=True):
        N = T * k
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device) if logits else None
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.x_perm = torch.empty((N, H), dtype=dtype, device=device) if x_perm else None
        self.plan = Plan(torch.empty(E, dtype=torch.int32, device=device),
                         torch.empty(E + 1, dtype=torch.int32, device=device),
                         torch.empty(N, dtype=torch.int32, device=device),
                         torch.empty(N, dtype=torch.int32, device=device))
        self.workspace = torch.empty(max(moe_permute_workspace_bytes(T, k, E), 1), dtype=torch.uint8, device=device)
        self.h = torch.empty((N, I), dtype=dtype, device=device)
        self.gu_saved = torch.empty((N, 2 * I), dtype=dtype, device=device) if gu_saved else None
        self.y = torch.empty((N, H), dtype=dtype, device=device)
        self.out = torch.empty((T, H), dtype=dtype, device=device)
        self.shared = None
        if I_shared:
            self.shared = {
                "offsets": torch.tensor([0, T], dtype=torch.int32).to(device),
                "h": torch.empty((T, I_shared), dtype=dtype, device=device),
                "gu_saved": torch.empty((T, 2 * I_shared), dtype=dtype, device=device) if gu_saved else None,
                "y": torch.empty((T, H), dtype=dtype, device=device),
            }


def moe_layer_forward(x, gate_up, down, k, w_gate=None, logits=None, renorm=True, residual=None, bufs=None,
                      shared_gate_up=None, shared_down=None, save_for_backward=False, stream=None, gather=False,
                      ffn_groups=None):
    """Router (logits unless given) -> top-k -> permute -> grouped SwiGLU FFN -> combine.
    With shared_gate_up / shared_down, the shared expert runs on every token as a one-segment grouped
    FFN and its output is the combine's residual (a separate residual is then not accepted).
    gather=True: the permute computes the plan only and the first grouped matmul gathers its rows
    from x (same result, bit for bit; x_perm is never written, so there is no backward from it).
    ffn_groups: an ExpertGroupsFfn; the routed FFN then runs as expert groups on its streams (same
    result, bit for bit)."""
    T, H = x.shape
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    I_sh = 0 if shared_gate_up is None else shared_gate_up.shape[1] // 2
    if I_sh and residual is not None:
        raise ValueError("moe_layer_forward: the shared expert's output is the residual; pass one or the other")
    if gather and save_for_backward:
        raise ValueError("moe_layer_forward: gather=True keeps no x_perm, which the backward needs")
    if bufs is None:
        bufs = LayerBuffers(T, H, I, E, k, x.dtype, x.device, logits=logits is None, gu_saved=save_for_backward,
                            I_shared=I_sh, x_perm=not gather)
    if logits is None:
        logits = moe_router_logits(x, w_gate, bufs.logits, stream)
    moe_router_topk_permute(logits, k, x, E, renorm, bufs.topk_idx, bufs.topk_w, bufs.x_perm, bufs.plan,
                            bufs.workspace, stream, rows=not gather)
    if ffn_groups is not None:
        ffn_groups(gate_up, down, bufs.plan.offsets, bufs.h, bufs.y, x_perm=bufs.x_perm, x=x if gather else None,
                   slot_of_row=bufs.plan.slot_of_row, k=k, gu_saved=bufs.gu_saved, stream=stream)
    elif gather:
        moe_grouped_swiglu_ffn_gather(x, bufs.plan.slot_of_row, k, gate_up, down, bufs.plan.offsets, None, bufs.h,
                                      bufs.y, bufs.gu_saved, stream)
    else:
        moe_grouped_swiglu_ffn(bufs.x_perm, gate_up, down, bufs.plan.offsets, bufs.h, bufs.y, bufs.gu_saved, stream)
    if I_sh:
        sh = bufs.shared
        moe_grouped_swiglu_ffn(x, shared_gate_up, shared_down, sh["offsets"], sh["h"], sh["y"], sh["gu_saved"], stream)
        residual = sh["y"]
    moe_unpermute_combine(bufs.y, bufs.plan.row_of_slot, bufs.topk_w, residual, bufs.out, stream)
    return bufs.out, bufs


class ExpertGroupsFfn:
    """The grouped SwiGLU FFN as G groups of consecutive experts on G streams (default priority):
    group i runs its gate_up matmul then its down matmul on stream i, each group starting after the
    work already queued on the calling stream, and the calling stream waits for all of them. One
    launch leaves the tail of its tile list to a few CUs; here the other groups' tiles (and group i's
    down matmul as soon as its gate_up is done) fill it. The groups are plain sub-ranges of the
    experts (weights and offsets sliced, rows addressed absolutely), so the result is bit-identical
    to the one-stream FFN."""

    def __init__(self, groups=2, device=None):
        if groups < 1:
            raise ValueError("ExpertGroupsFfn: groups must be >= 1")
        self.groups = groups
        self.streams = [torch.cuda.Stream(device=device) for _ in range(groups)]
        self.done = [torch.cuda.Event() for _ in range(groups)]

    def __call__(self, gate_up, down, expert_offsets, h, y, x_perm=None, x=None, slot_of_row=None, k=None,
                 gu_saved=None, stream=None):
        """Rows from x_perm, or gathered from x through slot_of_row (row r = token slot_of_row[r] // k)."""
        main = torch.cuda.current_stream() if stream is None else stream
        E = expert_offsets.shape[0] - 1
        H = gate_up.shape[0] // E
        I = gate_up.shape[1] // 2
        N = h.shape[0]
        bounds = [E * i // self.groups for i in range(self.groups + 1)]
        for s in self.streams:
            s.wait_stream(main)
        for i, s in enumerate(self.streams):   # all gate_up launches first, so that they start together
            e0, e1 = bounds[i], bounds[i + 1]
            if e1 == e0:
                continue
            gu_i, off_i = gate_up[e0 * H:e1 * H], expert_offsets[e0:e1 + 1]
            if x_perm is None:
                moe_grouped_gemm_swiglu_gather(x, slot_of_row, k, gu_i, off_i, N, h, gu_saved, s)
            else:
                moe_grouped_gemm_swiglu(x_perm, gu_i, off_i, h, gu_saved, s)
        for i, s in enumerate(self.streams):
            e0, e1 = bounds[i], bounds[i + 1]
            if e1 > e0:
                moe_grouped_gemm_down(h, down[e0 * I:e1 * I], expert_offsets[e0:e1 + 1], y, s)
            self.done[i].record(s)
            main.wait_event(self.done[i])
        return y, h


class ChunkedForward:
    """Domino-style forward on one GPU: the tokens are split into `chunks` contiguous chunks; the
    routing of each chunk (router logits, top-k, permute plan: the stand-in for its dispatch) runs
    on a side stream, and chunk c's grouped FFN and combine run on the calling stream as soon as
    chunk c is routed, so the routing of chunk c+1 overlaps chunk c's expert matmuls. An event per
    chunk orders the two streams. Every chunk has its own buffers, allocated here once; the output
    rows of chunk c are written straight into out[rows of c]. Per token the result is bit-identical
    to moe_layer_forward (routing and the FFN rows do not depend on the other tokens).
    overlap=False issues the same calls on one stream (for comparison)."""

    def __init__(self, T, H, I, E, k, dtype, device, chunks=2, logits=True, gather=True):
        if chunks < 1 or chunks > T:
            raise ValueError(f"ChunkedForward: chunks={chunks} must be in [1, T={T}]")
        self.T, self.H, self.E, self.k, self.gather = T, H, E, k, gather
        self.bounds = [T * c // chunks for c in range(chunks + 1)]
        self.bufs = [LayerBuffers(self.bounds[c + 1] - self.bounds[c], H, I, E, k, dtype, device, logits=logits,
                                  x_perm=not gather) for c in range(chunks)]
        self.side = torch.cuda.Stream(device=device)          # default priority
        self.routed = [torch.cuda.Event() for _ in range(chunks)]
        self.out = torch.empty((T, H), dtype=dtype, device=device)

    def __call__(self, x, gate_up, down, w_gate=None, logits=None, renorm=True, overlap=True, stream=None):
        main = torch.cuda.current_stream() if stream is None else stream
        side = self.side if overlap else main
        if overlap:
            side.wait_stream(main)   # x ready, and the previous call's chunks done with their buffers
        k, E = self.k, self.E
        for c, b in enumerate(self.bufs):
            t0, t1 = self.bounds[c], self.bounds[c + 1]
            xc = x[t0:t1]
            lg = logits[t0:t1] if logits is not None else moe_router_logits(xc, w_gate, b.logits, side)
            moe_router_topk_permute(lg, k, xc, E, renorm, b.topk_idx, b.topk_w, b.x_perm, b.plan, b.workspace, side,
                                    rows=not self.gather)
            if overlap:
                self.routed[c].record(side)
                main.wait_event(self.routed[c])
            if self.gather:
                moe_grouped_swiglu_ffn_gather(xc, b.plan.slot_of_row, k, gate_up, down, b.plan.offsets, None, b.h,
                                              b.y, None, main)
            else:
                moe_grouped_swiglu_ffn(b.x_perm, gate_up, down, b.plan.offsets, b.h, b.y, None, main)
            moe_unpermute_combine(b.y, b.plan.row_of_slot, b.topk_w, None, self.out[t0:t1], main)
        return self.out


class LayerGrads:
    """Gradient buffers of one layer backward (allocated once, reused)."""

    def __init__(self, T, H, I, E, k, dtype, device, I_shared=0, router=True):
        N = T * k
        self.d_y = torch.empty((N, H), dtype=dtype, device=device)
        self.d_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.d_gu = torch.empty((N, 2 * I), dtype=dtype, device=device)
        self.d_x_perm = torch.empty((N, H), dtype=dtype, device=device)
        self.d_gate_up = torch.empty((E * H, 2 * I), dtype=dtype, device=device)
        self.d_down = torch.empty((E * I, H), dtype=dtype, device=device)
        self.d_logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.d_w_gate = torch.empty((H, E), dtype=torch.float32, device=device) if router else None
        self.d_x_side = torch.empty((T, H), dtype=dtype, device=device)   # shared-expert / router dX
        self.d_x_side2 = torch.empty((T, H), dtype=dtype, device=device) if I_shared and router else None
        self.d_x = torch.empty((T, H), dtype=dtype, device=device)
        self.d_shared_gate_up = self.d_shared_down = self.d_shared_gu = None
        if I_shared:
            self.d_shared_gate_up = torch.empty((H, 2 * I_shared), dtype=dtype, device=device)
            self.d_shared_down = torch.empty((I_shared, H), dtype=dtype, device=device)
            self.d_shared_gu = torch.empty((T, 2 * I_shared), dtype=dtype, device=device)


class OverlappedBackward:
    """moe_layer_backward with its independent products on three streams (default priority):

      main   combine bwd -> dY.down^T + SwiGLU bwd (dGU) -> dGU.gate_up^T (dX) -> join -> permute bwd
      wgrad  after combine bwd: dW_down = h^T dY; after dGU: dW_gate_up = X^T dGU
      aux    after combine bwd: shared-expert backward -> top-k bwd -> router-logits bwd

    The weight gradients are bound by writing their E*3*H*I outputs and the data gradients by the
    matrix cores, so the two share the chip better than they follow each other: the weight-gradient
    products (persistent, one workgroup per CU) are capped to `wgrad_cus` CUs and the data-gradient
    tiles run on the others. Every product is the same kernel on the same inputs as in the one-stream
    backward, so the gradients are bit-identical to moe_layer_backward's."""

    def __init__(self, device=None, wgrad_cus=128):
        self.wgrad_cus = wgrad_cus
        self.wgrad = torch.cuda.Stream(device=device)
        self.aux = torch.cuda.Stream(device=device)
        self.ev_dy, self.ev_dgu, self.ev_wgrad, self.ev_aux = (torch.cuda.Event() for _ in range(4))

    def __call__(self, d_out, x, gate_up, down, bufs, w_gate=None, logits=None, renorm=True, shared_gate_up=None,
                 shared_down=None, grads=None, stream=None):
        main = torch.cuda.current_stream() if stream is None else stream
        T, H = x.shape
        E = gate_up.shape[0] // H
        I = gate_up.shape[1] // 2
        k = bufs.topk_idx.shape[1]
        I_sh = 0 if shared_gate_up is None else shared_gate_up.shape[1] // 2
        if bufs.gu_saved is None:
            raise ValueError("OverlappedBackward: run the forward with save_for_backward=True")
        if grads is None:
            grads = LayerGrads(T, H, I, E, k, x.dtype, x.device, I_shared=I_sh, router=w_gate is not None)
        g = grads
        offs = bufs.plan.offsets
        # the side streams also wait for whatever the caller queued before (inputs, earlier users of grads)
        self.wgrad.wait_stream(main)
        self.aux.wait_stream(main)
        moe_unpermute_combine_bwd(d_out, bufs.y, bufs.plan.row_of_slot, bufs.topk_w, g.d_y, g.d_w, main)
        self.ev_dy.record(main)
        self.wgrad.wait_event(self.ev_dy)
        self.aux.wait_event(self.ev_dy)
        moe_grouped_gemm_wgrad(bufs.h, g.d_y, offs, g.d_down, self.wgrad_cus, self.wgrad)
        moe_grouped_gemm_down_bwd(g.d_y, down, bufs.gu_saved, offs, g.d_gu, main)
        self.ev_dgu.record(main)
        self.wgrad.wait_event(self.ev_dgu)
        moe_grouped_gemm_wgrad(bufs.x_perm, g.d_gu, offs, g.d_gate_up, self.wgrad_cus, self.wgrad)
        moe_grouped_gemm_gate_up_bwd(g.d_gu, gate_up, offs, g.d_x_perm, main)
        side = None
        if I_sh:
            sh = bufs.shared
            moe_grouped_swiglu_ffn_bwd(d_out, x, sh["gu_saved"], sh["h"], shared_gate_up, shared_down, sh["offsets"],
                                       g.d_x_side, g.d_shared_gate_up, g.d_shared_down, g.d_shared_gu, self.aux)
            side = g.d_x_side
        logits = bufs.logits if logits is None else logits
        moe_router_topk_bwd(logits, bufs.topk_idx, bufs.topk_w, g.d_w, renorm, g.d_logits, self.aux)
        if w_gate is not None:
            dst = g.d_x_side2 if side is not None else g.d_x_side
            moe_router_logits_bwd(x, w_gate, g.d_logits, g.d_w_gate, d_x_in=side, d_x=dst, stream=self.aux)
            side = dst
        self.ev_wgrad.record(self.wgrad)
        self.ev_aux.record(self.aux)
        main.wait_event(self.ev_wgrad)
        main.wait_event(self.ev_aux)
        moe_permute_bwd(g.d_x_perm, bufs.plan.row_of_slot, T, k, d_x_add=side, d_x=g.d_x, stream=main)
        return g


def moe_layer_backward(d_out, x, gate_up, down, bufs, w_gate=None, logits=None, renorm=True, shared_gate_up=None,
                       shared_down=None, grads=None, stream=None):
    """Backward of moe_layer_forward(..., save_for_backward=True) given d_out = dL/d(out):
    combine-bwd -> grouped FFN bwd (+ shared expert) -> top-k bwd -> router-logits bwd -> permute-bwd,
    which sums each token's k expert-row gradients with the shared-expert and router contributions."""
    T, H = x.shape
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    k = bufs.topk_idx.shape[1]
    I_sh = 0 if shared_gate_up is None else shared_gate_up.shape[1] // 2
    if bufs.gu_saved is None:
        raise ValueError("moe_layer_backward: run the forward with save_for_backward=True")
    if grads is None:
        grads = LayerGrads(T, H, I, E, k, x.dtype, x.device, I_shared=I_sh, router=w_gate is not None)
    g = grads
    moe_unpermute_combine_bwd(d_out, bufs.y, bufs.plan.row_of_slot, bufs.topk_w, g.d_y, g.d_w, stream)
    moe_grouped_swiglu_ffn_bwd(g.d_y, bufs.x_perm, bufs.gu_saved, bufs.h, gate_up, down, bufs.plan.offsets,
                               g.d_x_perm, g.d_gate_up, g.d_down, g.d_gu, stream)
    side = None   # dX contributions besides the expert rows
    if I_sh:
        sh = bufs.shared
        moe_grouped_swiglu_ffn_bwd(d_out, x, sh["gu_saved"], sh["h"], shared_gate_up, shared_down, sh["offsets"],
                                   g.d_x_side, g.d_shared_gate_up, g.d_shared_down, g.d_shared_gu, stream)
        side = g.d_x_side
    logits = bufs.logits if logits is None else logits
    moe_router_topk_bwd(logits, bufs.topk_idx, bufs.topk_w, g.d_w, renorm, g.d_logits, stream)
    if w_gate is not None:
        dst = g.d_x_side2 if side is not None else g.d_x_side
        moe_router_logits_bwd(x, w_gate, g.d_logits, g.d_w_gate, d_x_in=side, d_x=dst, stream=stream)
        side = dst
    moe_permute_bwd(g.d_x_perm, bufs.plan.row_of_slot, T, k, d_x_add=side, d_x=g.d_x, stream=stream)
    return g
