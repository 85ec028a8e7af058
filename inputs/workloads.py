"""The synthetic workloads of the MoE layer and their seeded inputs.

Shapes are written (T tokens, H hidden, I expert intermediate, E experts, k experts per token).
Weights use the fused layout of the MindSpeed-MM InternVL3.5 practice page (section 2, model
integration): gate_up [E*H, 2*I] and down [E*I, H], row-major. Distributions: activations
N(0, 1), every weight matrix N(0, 0.02^2), seeds built from 42 (the seed of that page's runs).

Workloads
---------
tiny_f32         T=64,    H=64,   I=32,   E=8,   k=2, fp32. Small enough for a pure-Python check.
qwen3_moe        T=4096,  H=2048, I=768,  E=128, k=8, bf16 (4 x 1024-token sequences).
ep_rank_zipf     one expert-parallel rank's local share after dispatch, bf16: 32 local experts,
                 H=2048, I=768, 8192 pre-dispatched rows (the 8 slots of 1024 source tokens).
                 Two experts are empty; the other 30 take Zipf(s=1.2) shares of the rows.
long_seq         T=16384, H=2048, I=768, E=128, k=8, bf16, router logits drawn directly from
                 N(0, 0.1^2) (near-uniform routing); forward only.
fine_grained     T=4096,  H=7168, I=2048, E=256, k=8, bf16, plus one always-active shared expert;
                 forward and backward with upstream gradient N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .generators import normal, permutation, uniform_open01, generator

SEED = 42

# tensor ids inside a workload's key space
X, W_GATE, GATE_UP, DOWN, LOGITS, SH_GATE_UP, SH_DOWN, D_OUT = range(8)
EP_EXPERT_ORDER, EP_COUNTS, EP_ROW_OF_SLOT, EP_GATE_W = 8, 9, 10, 11


@dataclass(frozen=True)
class Workload:
    name: str
    code: int
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: str
    logits_std: Optional[float] = None   # router logits drawn directly instead of x @ W_g
    shared: int = 0                      # always-active shared experts
    backward: bool = False
    ep_rows: int = 0                     # >0: pre-dispatched rows (one EP rank's share)
    description: str = ""

    @property
    def N(self) -> int:
        return self.ep_rows if self.ep_rows else self.T * self.k


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 64, 64, 32, 8, 2, "f32",
                         description="tiny MoE layer, fp32, T=64 H=64 I=32 E=8 k=2"),
    "qwen3_moe": Workload("qwen3_moe", 2, 4096, 2048, 768, 128, 8, "bf16",
                          description="Qwen3-MoE-shaped layer, bf16, T=4096 H=2048 I=768 E=128 k=8"),
    "ep_rank_zipf": Workload("ep_rank_zipf", 3, 1024, 2048, 768, 32, 8, "bf16", ep_rows=8192,
                             description="one EP rank's share: 32 experts, 8192 rows, Zipf(1.2) counts, 2 empty"),
    "long_seq": Workload("long_seq", 4, 16384, 2048, 768, 128, 8, "bf16", logits_std=0.1,
                         description="long-sequence micro-batch, bf16, T=16384, logits ~N(0,0.1^2), forward only"),
    "fine_grained": Workload("fine_grained", 5, 4096, 7168, 2048, 256, 8, "bf16", shared=1, backward=True,
                             description="fine-grained MoE, bf16, T=4096 H=7168 I=2048 E=256 k=8 + 1 shared, fwd+bwd"),
}


def make_layer_inputs(T: int, H: int, I: int, E: int, k: int, dtype: str, key: tuple,
                      x_std: float = 1.0, w_std: float = 0.02, wg_std: float = 0.02,
                      logits_std: Optional[float] = None, shared: int = 0,
                      backward: bool = False) -> dict:
    """Inputs of one MoE layer call. key = (SEED, workload code, ...) identifies the stream.

    Returns numpy arrays: x [T,H]; w_gate [H,E] (or logits [T,E] fp32 when logits_std is set);
    gate_up [E*H, 2I]; down [E*I, H]; shared_gate_up [H, 2I*shared] / shared_down [I*shared, H]
    when shared > 0; d_out [T,H] when backward. bf16 tensors are uint16 bit patterns."""
    key = tuple(key)
    out = {"x": normal((T, H), x_std, key + (X,), dtype)}
    if logits_std is None:
        out["w_gate"] = normal((H, E), wg_std, key + (W_GATE,), dtype)
    else:
        out["logits"] = normal((T, E), logits_std, key + (LOGITS,), "f32")
    out["gate_up"] = normal((E * H, 2 * I), w_std, key + (GATE_UP,), dtype)
    out["down"] = normal((E * I, H), w_std, key + (DOWN,), dtype)
    if shared:
        # a single shared expert with the routed experts' intermediate size; several shared
        # experts are the same thing with a wider intermediate dimension
        out["shared_gate_up"] = normal((H, 2 * I * shared), w_std, key + (SH_GATE_UP,), dtype)
        out["shared_down"] = normal((I * shared, H), w_std, key + (SH_DOWN,), dtype)
    if backward:
        out["d_out"] = normal((T, H), 1.0, key + (D_OUT,), dtype)
    return out


def workload_inputs(name: str) -> dict:
    wl = WORKLOADS[name]
    if wl.ep_rows:
        return make_ep_share_inputs(wl.E, wl.ep_rows, wl.H, wl.I, wl.k, (SEED, wl.code))
    return make_layer_inputs(wl.T, wl.H, wl.I, wl.E, wl.k, wl.dtype, (SEED, wl.code),
                             logits_std=wl.logits_std, shared=wl.shared, backward=wl.backward)


def zipf_counts(E: int, rows: int, n_empty: int, s: float, key: tuple) -> np.ndarray:
    """Per-expert row counts: n_empty experts (chosen by the seed) get none; the rest are ranked by
    a seeded permutation and take multinomial(rows, p_r ~ r^-s) rows, r = 1..E-n_empty."""
    key = tuple(key)
    order = permutation(E, key + (EP_EXPERT_ORDER,))
    ranked = order[n_empty:]
    r = np.arange(1, E - n_empty + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    counts = np.zeros(E, dtype=np.int32)
    counts[ranked] = generator(key + (EP_COUNTS,)).multinomial(rows, p).astype(np.int32)
    return counts


def make_ep_share_inputs(E: int, rows: int, H: int, I: int, k: int, key: tuple,
                         n_empty: int = 2, s: float = 1.2, dtype: str = "bf16") -> dict:
    """One EP rank's local share after dispatch (the buffer is already grouped by expert).

    Returns counts [E] int32 (rows per expert, expert-contiguous), x_perm [rows, H], gate_up,
    down, and for the return path: row_of_slot [rows] (slot t*k+j of source token t = rows//k
    tokens -> its row in the buffer, a seeded permutation) and topk_w [rows//k, k] float32 gate
    weights in (0, 1)."""
    key = tuple(key)
    assert rows % k == 0
    return {
        "counts": zipf_counts(E, rows, n_empty, s, key),
        "x_perm": normal((rows, H), 1.0, key + (X,), dtype),
        "gate_up": normal((E * H, 2 * I), 0.02, key + (GATE_UP,), dtype),
        "down": normal((E * I, H), 0.02, key + (DOWN,), dtype),
        "row_of_slot": permutation(rows, key + (EP_ROW_OF_SLOT,)),
        "topk_w": uniform_open01((rows // k, k), key + (EP_GATE_W,)),
    }
