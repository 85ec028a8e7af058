"""CPU oracle for the MoE expert layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct implementation (C, fp64, per-token loops; see moe_oracle.h)
used to check the GPU library. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it. It shares no code with the GPU path and never calls it.

Pins: tests/test_oracle_*.py check every function here against things other than itself
(brute force, closed forms, invariants, library routines, finite differences).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
# MOE_SANITIZE_ORACLE=1 loads the AddressSanitizer + UBSan build (tests/sanitizers.py preloads gcc's
# ASan runtime for it)
SANITIZE = os.environ.get("MOE_SANITIZE_ORACLE") == "1"
LIB = os.path.join(HERE, "liborc_moe_san.so" if SANITIZE else "liborc_moe.so")
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

F32, BF16 = 0, 1

_lib = None


def build(verbose: bool = False, sanitize: bool = None) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction, OpenMP over tokens); with
    sanitize, the AddressSanitizer + UBSan build liborc_moe_san.so."""
    san = SANITIZE if sanitize is None else sanitize
    out = os.path.join(HERE, "liborc_moe_san.so" if san else "liborc_moe.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *(SAN_FLAGS if san else []), "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 (uint16 bit patterns), got {a.dtype}")


def _same_dt(*arrays):
    if len({a.dtype for a in arrays}) != 1:
        raise TypeError("oracle: these operands must share one data type: "
                        + ", ".join(str(a.dtype) for a in arrays))


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _call(name, *args):
    f = getattr(_load(), name)
    f.restype = ctypes.c_int
    rc = f(*args)
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


I64 = ctypes.c_int64


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (independent tokens / rows)."""
    _load().orc_set_threads(ctypes.c_int(int(n)))


def max_threads() -> int:
    f = _load().orc_max_threads
    f.restype = ctypes.c_int
    return int(f())


def router_logit_block(H: int) -> int:
    """Hidden units per block of the router's four fp32 chains."""
    f = _load().orc_router_logit_block
    f.restype = ctypes.c_int
    return int(f(I64(H)))


def router_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    x, w_gate = _c(x), _c(w_gate)
    T, H = x.shape
    E = w_gate.shape[1]
    assert w_gate.shape[0] == H and x.dtype == w_gate.dtype
    out = np.empty((T, E), np.float32)
    _call("orc_router_logits", _p(x), _p(w_gate), _dt(x), I64(T), I64(H), I64(E), _p(out))
    return out


def router_topk(logits: np.ndarray, k: int, renorm: bool = True):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _call("orc_router_topk", _p(logits), I64(T), I64(E), I64(k), ctypes.c_int(int(renorm)), _p(idx), _p(w))
    return idx, w


def router_stats(logits: np.ndarray, topk_idx: np.ndarray, want_probs: bool = True):
    """(probs [T,E] or None, mean_prob [E], load [E]) in fp64 / int64: the full softmax per token,
    its mean over tokens, and how many (token, slot) pairs chose each expert."""
    logits = _c(logits, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    T, E = logits.shape
    k = topk_idx.shape[1]
    probs = np.empty((T, E), np.float64) if want_probs else None
    mean = np.empty(E, np.float64)
    load = np.empty(E, np.int64)
    _call("orc_router_stats", _p(logits), _p(topk_idx), I64(T), I64(E), I64(k), _p(probs), _p(mean), _p(load))
    return probs, mean, load


def permute_plan(topk_idx: np.ndarray, E: int):
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    N = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    ros = np.empty(N, np.int32)
    sor = np.empty(N, np.int32)
    _call("orc_permute_plan", _p(topk_idx), I64(T), I64(k), I64(E), _p(counts), _p(offsets), _p(ros), _p(sor))
    return counts, offsets, ros, sor


def permute_rows(x: np.ndarray, slot_of_row: np.ndarray, k: int) -> np.ndarray:
    x = _c(x)
    slot_of_row = _c(slot_of_row, np.int32)
    N = slot_of_row.shape[0]
    out = np.empty((N, x.shape[1]), x.dtype)
    _call("orc_permute_rows", _p(x), I64(x.itemsize), I64(x.shape[1]), _p(slot_of_row), I64(k), I64(N), _p(out))
    return out


def expert_rows(x_perm, offsets, gate_up, down, rows=None, want_act=False, want_gu=False):
    """FFN of each requested row of an expert-grouped buffer. Returns y (and a, gu if asked)."""
    x_perm, gate_up, down = _c(x_perm), _c(gate_up), _c(down)
    offsets = _c(offsets, np.int32)
    N, H = x_perm.shape
    E = offsets.shape[0] - 1
    I = gate_up.shape[1] // 2
    assert gate_up.shape == (E * H, 2 * I) and down.shape == (E * I, H)
    rows = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    n = rows.shape[0]
    y = np.empty((n, H), np.float64)
    a = np.empty((n, I), np.float64) if want_act else None
    gu = np.empty((n, 2 * I), np.float64) if want_gu else None
    _call("orc_expert_rows", _p(x_perm), _dt(x_perm), I64(H), I64(I), I64(E), _p(offsets), _p(gate_up), _p(down),
          _p(rows), I64(n), _p(y), _p(a), _p(gu))
    out = (y,)
    if want_act:
        out += (a,)
    if want_gu:
        out += (gu,)
    return out if len(out) > 1 else y


def combine(y, row_of_slot, topk_w, residual=None, tokens=None):
    y = _c(y)
    row_of_slot = _c(row_of_slot, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, k = topk_w.shape
    H = y.shape[1]
    if residual is not None:
        residual = _c(residual)
        assert residual.dtype == y.dtype
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((tokens.shape[0], H), np.float64)
    _call("orc_combine", _p(y), _dt(y), I64(H), I64(k), _p(row_of_slot), _p(topk_w), _p(residual), _p(tokens),
          I64(tokens.shape[0]), _p(out))
    return out


def moe_forward_tokens(x, topk_idx, topk_w, gate_up, down, shared_gate_up=None, shared_down=None,
                       tokens=None):
    x, gate_up, down = _c(x), _c(gate_up), _c(down)
    topk_idx = _c(topk_idx, np.int32)
    topk_w = _c(topk_w, np.float64)
    T, H = x.shape
    k = topk_idx.shape[1]
    I = gate_up.shape[1] // 2
    E = gate_up.shape[0] // H
    Is = 0
    if shared_gate_up is not None:
        shared_gate_up, shared_down = _c(shared_gate_up), _c(shared_down)
        Is = shared_gate_up.shape[1] // 2
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((tokens.shape[0], H), np.float64)
    _call("orc_moe_forward_tokens", _p(x), _dt(x), I64(H), I64(I), I64(E), I64(k), _p(topk_idx), _p(topk_w),
          _p(gate_up), _p(down), _p(shared_gate_up), _p(shared_down), I64(Is), _p(tokens),
          I64(tokens.shape[0]), _p(out))
    return out


def moe_forward(x, gate_up, down, k, w_gate=None, logits=None, renorm=True, shared_gate_up=None,
                shared_down=None, tokens=None):
    """Router (logits -> top-k -> weights) then the per-token layer. Returns (out, idx, w, logits)."""
    if logits is None:
        logits = router_logits(x, w_gate)
    idx, w = router_topk(logits, k, renorm)
    out = moe_forward_tokens(x, idx, w, gate_up, down, shared_gate_up, shared_down, tokens)
    return out, idx, w, logits


# ---- backward --------------------------------------------------------------------------------

def combine_bwd(d_out, y, row_of_slot, topk_w, tokens=None):
    d_out, y = _c(d_out), _c(y)
    row_of_slot = _c(row_of_slot, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, k = topk_w.shape
    H = y.shape[1]
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = tokens.shape[0]
    d_y = np.empty((n, k, H), np.float64)
    d_w = np.empty((n, k), np.float64)
    _call("orc_combine_bwd", _p(d_out), _dt(d_out), _p(y), _dt(y), I64(H), I64(k), _p(row_of_slot), _p(topk_w), _p(tokens),
          I64(n), _p(d_y), _p(d_w))
    return d_y, d_w


def expert_rows_bwd(x_perm, d_y, offsets, gate_up, down, rows=None, want_gu=False):
    x_perm, d_y, gate_up, down = _c(x_perm), _c(d_y), _c(gate_up), _c(down)
    offsets = _c(offsets, np.int32)
    N, H = x_perm.shape
    E = offsets.shape[0] - 1
    I = gate_up.shape[1] // 2
    rows = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    n = rows.shape[0]
    d_x = np.empty((n, H), np.float64)
    d_gu = np.empty((n, 2 * I), np.float64) if want_gu else None
    _same_dt(x_perm, gate_up, down)
    _call("orc_expert_rows_bwd", _p(x_perm), _p(d_y), _dt(x_perm), _dt(d_y), I64(H), I64(I), I64(E), _p(offsets),
          _p(gate_up), _p(down), _p(rows), I64(n), _p(d_x), _p(d_gu))
    return (d_x, d_gu) if want_gu else d_x


def expert_weight_grads(x_perm, d_y, offsets, gate_up, down, e):
    x_perm, d_y, gate_up, down = _c(x_perm), _c(d_y), _c(gate_up), _c(down)
    offsets = _c(offsets, np.int32)
    H = x_perm.shape[1]
    E = offsets.shape[0] - 1
    I = gate_up.shape[1] // 2
    dgu = np.empty((H, 2 * I), np.float64)
    ddn = np.empty((I, H), np.float64)
    _same_dt(x_perm, gate_up, down)
    _call("orc_expert_weight_grads", _p(x_perm), _p(d_y), _dt(x_perm), _dt(d_y), I64(H), I64(I), I64(E), _p(offsets),
          _p(gate_up), _p(down), I64(e), _p(dgu), _p(ddn))
    return dgu, ddn


def expert_weight_grads_units(x_perm, d_y, offsets, gate_up, down, e, units):
    """Entries of expert e's weight gradients for the intermediate units listed: returns
    (d_gate_up[:, units], d_gate_up[:, I + units], d_down[units, :]) as fp64 [H,n], [H,n], [n,H]."""
    x_perm, d_y, gate_up, down = _c(x_perm), _c(d_y), _c(gate_up), _c(down)
    offsets = _c(offsets, np.int32)
    units = _c(units, np.int64)
    H = x_perm.shape[1]
    E = offsets.shape[0] - 1
    I = gate_up.shape[1] // 2
    n = units.shape[0]
    cols = np.empty((n, 2, H), np.float64)
    rows = np.empty((n, H), np.float64)
    _same_dt(x_perm, gate_up, down)
    _call("orc_expert_weight_grads_units", _p(x_perm), _p(d_y), _dt(x_perm), _dt(d_y), I64(H), I64(I), I64(E), _p(offsets),
          _p(gate_up), _p(down), I64(e), _p(units), I64(n), _p(cols), _p(rows))
    return cols[:, 0].T.copy(), cols[:, 1].T.copy(), rows


def permute_bwd(d_x_perm, row_of_slot, k, d_x_add=None, tokens=None):
    d_x_perm = _c(d_x_perm)
    row_of_slot = _c(row_of_slot, np.int32)
    H = d_x_perm.shape[1]
    T = row_of_slot.shape[0] // k
    if d_x_add is not None:
        d_x_add = _c(d_x_add)
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((tokens.shape[0], H), np.float64)
    _call("orc_permute_bwd", _p(d_x_perm), _dt(d_x_perm), I64(H), I64(k), _p(row_of_slot), _p(d_x_add),
          _p(tokens), I64(tokens.shape[0]), _p(out))
    return out


def router_topk_bwd(logits, topk_idx, d_w, renorm=True):
    logits = _c(logits, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    d_w = _c(d_w, np.float64)
    T, E = logits.shape
    k = topk_idx.shape[1]
    out = np.empty((T, E), np.float64)
    _call("orc_router_topk_bwd", _p(logits), _p(topk_idx), _p(d_w), I64(T), I64(E), I64(k),
          ctypes.c_int(int(renorm)), _p(out))
    return out


def router_logits_bwd(x, w_gate, d_logits):
    x, w_gate = _c(x), _c(w_gate)
    d_logits = _c(d_logits, np.float64)
    T, H = x.shape
    E = w_gate.shape[1]
    dwg = np.empty((H, E), np.float64)
    dx = np.empty((T, H), np.float64)
    _call("orc_router_logits_bwd", _p(x), _p(w_gate), _dt(x), _p(d_logits), I64(T), I64(H), I64(E),
          _p(dwg), _p(dx))
    return dwg, dx


def moe_backward(x, gate_up, down, k, d_out, w_gate=None, logits=None, renorm=True, shared_gate_up=None,
                 shared_down=None, experts=None):
    """Gradients of <d_out, layer(x)> along the layer, composed from the per-step backward functions
    above in the order the forward ran them (the combine is the dispatch's backward and vice versa:
    "DeepSeek MoE: EP and FSDP" guide, Automodel/DeepEP section). The routing selection is fixed to
    the forward's. Returns a dict of fp64 arrays: d_x, d_logits, d_w_gate (None without w_gate),
    d_gate_up / d_down (only the experts listed in `experts`, default all, each [H, 2I] / [I, H]),
    d_shared_gate_up / d_shared_down, plus the intermediates d_w [T,k] and d_x_perm [N,H]."""
    x = _c(x)
    T, H = x.shape
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    if logits is None:
        logits = router_logits(x, w_gate)
    idx, w = router_topk(logits, k, renorm)
    _, offsets, ros, sor = permute_plan(idx, E)
    xp = permute_rows(x, sor, k)
    y = expert_rows(xp, offsets, gate_up, down)
    d_y_slots, d_w = combine_bwd(d_out, y.astype(np.float32), ros, w.astype(np.float32))
    d_y = np.empty((T * k, H), np.float64)
    d_y[ros] = d_y_slots.reshape(T * k, H)
    d_y32 = d_y.astype(np.float32)
    d_xp = expert_rows_bwd(xp, d_y32, offsets, gate_up, down)
    d_x = permute_bwd(d_xp.astype(np.float32), ros, k)
    res = {"d_w": d_w, "d_x_perm": d_xp, "d_w_gate": None, "d_shared_gate_up": None, "d_shared_down": None}
    if shared_gate_up is not None:
        # the shared expert is one segment holding every token, with weight 1
        sh_off = np.array([0, T], np.int32)
        d_x = d_x + expert_rows_bwd(x, d_out, sh_off, shared_gate_up, shared_down)
        res["d_shared_gate_up"], res["d_shared_down"] = expert_weight_grads(x, d_out, sh_off, shared_gate_up,
                                                                            shared_down, 0)
    d_l = router_topk_bwd(logits, idx, d_w, renorm)
    res["d_logits"] = d_l
    if w_gate is not None:
        res["d_w_gate"], d_x_router = router_logits_bwd(x, w_gate, d_l)
        d_x = d_x + d_x_router
    res["d_x"] = d_x
    experts = range(E) if experts is None else experts
    res["d_gate_up"], res["d_down"] = {}, {}
    for e in experts:
        res["d_gate_up"][e], res["d_down"][e] = expert_weight_grads(xp, d_y32, offsets, gate_up, down, e)
    return res


def moe_backward_tokens(x, gate_up, down, k, d_out, tokens, w_gate=None, logits=None, renorm=True,
                        shared_gate_up=None, shared_down=None):
    """moe_backward restricted to some tokens: the routing runs for every token (it is cheap), the
    expert rows only for the listed tokens' slots. Returns fp64 d_x [n,H], d_logits [n,E], d_w [n,k]
    for tokens in the order given; with the same inputs these equal moe_backward's rows."""
    x = _c(x)
    tokens = np.asarray(tokens, np.int64)
    T, H = x.shape
    E = gate_up.shape[0] // H
    if logits is None:
        logits = router_logits(x, w_gate)
    idx, w = router_topk(logits, k, renorm)
    _, offsets, ros, sor = permute_plan(idx, E)
    xp = permute_rows(x, sor, k)
    slots = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    R = ros[slots].astype(np.int64)                      # the grouped rows of these tokens' slots
    y_R = expert_rows(xp, offsets, gate_up, down, rows=R).astype(np.float32)
    ros_c = np.full(T * k, -1, np.int32)                 # row map into the compact buffers
    ros_c[slots] = np.arange(slots.shape[0], dtype=np.int32)
    d_y_slots, d_w = combine_bwd(d_out, y_R, ros_c, w.astype(np.float32), tokens=tokens)
    d_y = np.zeros((T * k, H), np.float32)
    d_y[R] = d_y_slots.reshape(-1, H)
    d_xp_R = expert_rows_bwd(xp, d_y, offsets, gate_up, down, rows=R).astype(np.float32)
    d_x = permute_bwd(d_xp_R, ros_c, k, tokens=tokens)
    if shared_gate_up is not None:
        d_x = d_x + expert_rows_bwd(x, d_out, np.array([0, T], np.int32), shared_gate_up, shared_down, rows=tokens)
    d_l = router_topk_bwd(logits[tokens], idx[tokens], d_w, renorm)
    if w_gate is not None:
        _, d_x_router = router_logits_bwd(x[tokens], w_gate, d_l)
        d_x = d_x + d_x_router
    return {"d_x": d_x, "d_logits": d_l, "d_w": d_w}


def moe_weight_grads_units(x, gate_up, down, topk_idx, topk_w, d_out, e, units):
    """Entries of the layer's d_gate_up / d_down for routed expert e and the listed intermediate
    units, given the routing (topk_idx, topk_w) of the forward. Returns the same triple as
    expert_weight_grads_units; equal to the matching entries of moe_backward's d_gate_up[e] /
    d_down[e]."""
    x = _c(x)
    T, H = x.shape
    k = topk_idx.shape[1]
    E = gate_up.shape[0] // H
    I = gate_up.shape[1] // 2
    _, offsets, _, sor = permute_plan(topk_idx, E)
    r0, r1 = int(offsets[e]), int(offsets[e + 1])
    slots = sor[r0:r1].astype(np.int64)
    xp_e = permute_rows(x, slots, k)                      # expert e's rows, in grouped order
    # a row's d_y is its slot weight times its token's d_out (the combine's backward); it does not
    # depend on y, so the combine backward runs with a placeholder y and its d_w is not used
    d_y_slots, _ = combine_bwd(d_out, np.zeros((1, H), np.float32), np.zeros(T * k, np.int32),
                               _c(topk_w, np.float32), tokens=slots // k)
    d_y_e = d_y_slots[np.arange(slots.shape[0]), slots % k].astype(np.float32)
    seg = np.array([0, r1 - r0], np.int32)
    return expert_weight_grads_units(xp_e, d_y_e, seg, gate_up[e * H:(e + 1) * H], down[e * I:(e + 1) * I], 0,
                                     units)
