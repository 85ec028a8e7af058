"""Pins for the oracle's permute plan, expert FFN, combine and whole-layer forward.

Independent checks: numpy's bincount / cumsum / lexsort for the plan, the hand example of
tests/golden/permute_page_order.json, numpy fp64 matmuls per expert segment, a brute-force dense
all-experts masked computation with its own selection, and special cases that reduce to a plain
dense FFN or a dense softmax mixture."""
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from inputs import bf16_bits_to_f32, make_layer_inputs, normal, randint

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def as64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def random_routing(T, E, k, key):
    """k distinct experts per token (order arbitrary), seeded."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))
    if T == 0:
        return np.zeros((0, k), np.int32)
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


# ---- permute plan --------------------------------------------------------------------------------
def test_permute_plan_golden_page_order():
    with open(os.path.join(GOLDEN, "permute_page_order.json")) as f:
        g = json.load(f)
    counts, offsets, ros, sor = oracle.permute_plan(np.array(g["topk_idx"], np.int32), g["E"])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert sor.tolist() == g["slot_of_row"]
    assert ros.tolist() == g["row_of_slot"]


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 4, 4), (64, 8, 2), (300, 128, 8), (257, 32, 3), (0, 5, 2)])
def test_permute_plan_against_library(T, E, k):
    idx = random_routing(T, E, k, (910, T, E, k))
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(counts))
    assert counts.sum() == T * k
    slots = np.arange(T * k)
    # stable order by (expert, slot); slot = t*k + j orders by token since experts are distinct per token
    assert np.array_equal(sor, np.lexsort((slots, flat)))
    assert np.array_equal(ros[sor], slots)              # inverse permutations
    assert np.array_equal(np.sort(ros), slots)


def plan_by_sorting(idx, E):
    """The plan written with library routines only: keep the slots whose index lies in [0, E),
    count them per expert, and order them by (expert, slot) with a stable sort."""
    flat = idx.ravel()
    slots = np.arange(flat.size)
    keep = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[keep], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = slots[keep][np.lexsort((slots[keep], flat[keep]))]
    ros = np.full(flat.size, -1, np.int32)
    ros[order] = np.arange(order.size)
    return counts, offsets, ros, order.astype(np.int32)


@pytest.mark.parametrize("T,E,k,kind", [(50, 6, 4, "repeat"), (300, 16, 8, "repeat"), (7, 1, 3, "repeat"),
                                        (200, 12, 5, "drop"), (64, 4, 2, "drop"), (129, 32, 32, "both")])
def test_permute_plan_repeats_and_drops(T, E, k, kind):
    """Reading r19: an index outside [0, E) is dropped (no row, not counted); a token that names one
    expert in several slots gets one row per slot, in slot order. Both against the sort above."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([912, T, E, k])))
    lo, hi = (0, E) if kind == "repeat" else (-1, E + 1)
    if kind == "drop":   # distinct valid experts per token, then a quarter of the slots knocked out
        idx = random_routing(T, E, min(k, E), (913, T, E, k))
        knock = g.random(idx.shape) < 0.25
        idx = np.where(knock, g.choice([-1, E, -7, 1 << 20], idx.shape), idx).astype(np.int32)
    else:
        idx = g.integers(lo, hi, (T, k)).astype(np.int32)
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    w_counts, w_offsets, w_ros, w_sor = plan_by_sorting(idx, E)
    n = int(offsets[E])
    assert np.array_equal(counts, w_counts) and np.array_equal(offsets, w_offsets)
    assert np.array_equal(ros, w_ros)
    assert np.array_equal(sor[:n], w_sor) and np.all(sor[n:] == -1)
    valid = (idx.ravel() >= 0) & (idx.ravel() < E)
    assert n == valid.sum() and np.all(ros[~valid] == -1)
    # a dropped slot behaves as if the slot were not there: the same rows as the routing with the
    # token's valid slots only, in the same order
    if kind == "drop":
        assert np.array_equal(idx.ravel()[sor[:n]], np.repeat(np.arange(E), counts))


def test_permute_rows_round_trip():
    T, H, E, k = 50, 24, 6, 3
    x = normal((T, H), 1.0, (911, 1), "bf16")
    idx = random_routing(T, E, k, (911, 2))
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    xp = oracle.permute_rows(x, sor, k)
    assert np.array_equal(xp, x[sor // k])
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xp[ros[t * k + j]], x[t])        # gathering back gives x bitwise
    # k = 1 with unit weights: unpermute(permute(x)) == x
    idx1 = random_routing(T, E, 1, (911, 3))
    _, _, ros1, sor1 = oracle.permute_plan(idx1, E)
    xp1 = oracle.permute_rows(x, sor1, 1)
    back = oracle.combine(xp1, ros1, np.ones((T, 1), np.float32))
    assert np.array_equal(back, as64(x))


# ---- expert FFN ------------------------------------------------------------------------------------
def dense_ffn(x64, gu64, dn64):
    I = dn64.shape[0]
    g = x64 @ gu64[:, :I]
    u = x64 @ gu64[:, I:]
    return (g * expit(g) * u) @ dn64


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_expert_rows_match_per_segment_matmul(dtype):
    H, I, E = 40, 24, 5
    counts = np.array([7, 0, 13, 1, 0], np.int32)        # includes empty experts
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    xp = normal((N, H), 1.0, (912, 1), dtype)
    gu = normal((E * H, 2 * I), 0.2, (912, 2), dtype)
    dn = normal((E * I, H), 0.2, (912, 3), dtype)
    y, a, guv = oracle.expert_rows(xp, offsets, gu, dn, want_act=True, want_gu=True)
    x64, gu64, dn64 = as64(xp), as64(gu), as64(dn)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        want = dense_ffn(x64[r0:r1], gu64[e * H:(e + 1) * H], dn64[e * I:(e + 1) * I])
        np.testing.assert_allclose(y[r0:r1], want, rtol=1e-12, atol=1e-14)
        g = x64[r0:r1] @ gu64[e * H:(e + 1) * H, :I]
        np.testing.assert_allclose(guv[r0:r1, :I], g, rtol=1e-12, atol=1e-14)
    # sampled rows give the same values as the full call
    rows = np.array([N - 1, 0, 9], np.int64)
    np.testing.assert_array_equal(oracle.expert_rows(xp, offsets, gu, dn, rows=rows), y[rows])
    with pytest.raises(ValueError):
        oracle.expert_rows(xp, offsets, gu, dn, rows=np.array([N], np.int64))


# ---- whole forward -----------------------------------------------------------------------------------
def brute_force_dense_masked(x64, logits, gu64, dn64, E, k, renorm=True):
    """sum_e 1[e in S_t] * w_te * FFN_e(x_t), every expert evaluated on every token; S_t chosen by
    counting how many experts beat e (larger logit, or equal and lower index)."""
    T, H = x64.shape
    I = dn64.shape[0] // E
    l = logits.astype(np.float64)
    beaten = ((l[:, None, :] > l[:, :, None]) |
              ((l[:, None, :] == l[:, :, None]) & (np.arange(E)[None, None, :] < np.arange(E)[None, :, None]))).sum(-1)
    mask = beaten < k                                   # [T, E]
    p = softmax(l, axis=1)
    w = p * mask
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    out = np.zeros((T, H))
    for e in range(E):
        out += w[:, e:e + 1] * dense_ffn(x64, gu64[e * H:(e + 1) * H], dn64[e * I:(e + 1) * I])
    return out


@pytest.mark.parametrize("T,H,I,E,k,dtype", [(64, 64, 32, 8, 2, "f32"), (33, 48, 16, 6, 3, "bf16"),
                                             (20, 16, 8, 4, 4, "f32"), (17, 24, 8, 9, 1, "bf16")])
@pytest.mark.parametrize("renorm", [True, False])
def test_forward_equals_dense_masked_brute_force(T, H, I, E, k, dtype, renorm):
    d = make_layer_inputs(T, H, I, E, k, dtype, (913, T, E), w_std=0.2, wg_std=0.3)
    out, idx, w, logits = oracle.moe_forward(d["x"], d["gate_up"], d["down"], k, w_gate=d["w_gate"],
                                             renorm=renorm)
    want = brute_force_dense_masked(as64(d["x"]), logits, as64(d["gate_up"]), as64(d["down"]), E, k, renorm)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-13 * np.abs(want).max())


def test_forward_identical_experts_is_one_dense_ffn():
    # all experts equal: the renormalised weights sum to one, so the layer is a plain FFN
    T, H, I, E, k = 40, 32, 16, 6, 3
    x = normal((T, H), 1.0, (914, 1), "f32")
    gu1 = normal((H, 2 * I), 0.2, (914, 2), "f32")
    dn1 = normal((I, H), 0.2, (914, 3), "f32")
    wg = normal((H, E), 0.5, (914, 4), "f32")
    out, *_ = oracle.moe_forward(x, np.tile(gu1, (E, 1)), np.tile(dn1, (E, 1)), k, w_gate=wg)
    np.testing.assert_allclose(out, dense_ffn(as64(x), as64(gu1), as64(dn1)), rtol=1e-12, atol=1e-15)


def test_forward_single_expert_is_plain_ffn_and_shared_adds():
    T, H, I = 12, 20, 12
    x = normal((T, H), 1.0, (915, 1), "bf16")
    gu = normal((H, 2 * I), 0.2, (915, 2), "bf16")
    dn = normal((I, H), 0.2, (915, 3), "bf16")
    wg = normal((H, 1), 0.2, (915, 4), "bf16")
    out, idx, w, _ = oracle.moe_forward(x, gu, dn, 1, w_gate=wg)
    assert np.all(idx == 0) and np.all(w == 1.0)
    ref = dense_ffn(as64(x), as64(gu), as64(dn))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)
    # a shared expert with weight 1 adds its own FFN
    sgu = normal((H, 2 * I), 0.2, (915, 5), "bf16")
    sdn = normal((I, H), 0.2, (915, 6), "bf16")
    out2, *_ = oracle.moe_forward(x, gu, dn, 1, w_gate=wg, shared_gate_up=sgu, shared_down=sdn)
    np.testing.assert_allclose(out2, ref + dense_ffn(as64(x), as64(sgu), as64(sdn)), rtol=1e-12, atol=1e-15)


def test_pipeline_equals_per_token_layer():
    # plan -> permute -> expert rows -> combine (the GPU's decomposition) equals the per-token loop
    T, H, I, E, k = 48, 32, 16, 8, 2
    d = make_layer_inputs(T, H, I, E, k, "f32", (916,))
    out, idx, w, _ = oracle.moe_forward(d["x"], d["gate_up"], d["down"], k, w_gate=d["w_gate"])
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    xp = oracle.permute_rows(d["x"], sor, k)
    y = oracle.expert_rows(xp, offsets, d["gate_up"], d["down"])
    got = (w[:, :, None] * y[ros.reshape(T, k)]).sum(axis=1)
    np.testing.assert_allclose(got, out, rtol=1e-12, atol=1e-15)
    # combine: gather + weighted sum by numpy fancy indexing
    yb = normal((T * k, H), 1.0, (916, 9), "bf16")
    wf = w.astype(np.float32)
    res = normal((T, H), 1.0, (916, 10), "bf16")
    want = (wf.astype(np.float64)[:, :, None] * as64(yb)[ros.reshape(T, k)]).sum(axis=1) + as64(res)
    np.testing.assert_allclose(oracle.combine(yb, ros, wf, residual=res), want, rtol=1e-13, atol=1e-13)
    tok = np.array([5, 0, 47])
    np.testing.assert_array_equal(oracle.combine(yb, ros, wf, residual=res, tokens=tok),
                                  oracle.combine(yb, ros, wf, residual=res)[tok])


def test_forward_k_equals_E_is_dense_softmax_mixture():
    T, H, I, E = 16, 16, 8, 4
    d = make_layer_inputs(T, H, I, E, E, "f32", (917,), w_std=0.3, wg_std=0.4)
    out, idx, w, logits = oracle.moe_forward(d["x"], d["gate_up"], d["down"], E, w_gate=d["w_gate"])
    p = softmax(logits.astype(np.float64), axis=1)
    x64, gu64, dn64 = as64(d["x"]), as64(d["gate_up"]), as64(d["down"])
    want = sum(p[:, e:e + 1] * dense_ffn(x64, gu64[e * H:(e + 1) * H], dn64[e * I:(e + 1) * I]) for e in range(E))
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-15)


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.router_topk(np.zeros((2, 3), np.float32), 4)       # k > E
    with pytest.raises(ValueError):
        oracle.permute_rows(np.zeros((2, 3), np.float32), np.array([0, -1], np.int32), 1)   # a row with no slot
    with pytest.raises(TypeError):
        oracle.router_logits(np.zeros((2, 2), np.float64), np.zeros((2, 2), np.float64))


def test_inputs_are_seeded_and_chunk_independent():
    a = normal((3, 5), 1.0, (1, 2, 3), "bf16")
    b = normal((3, 5), 1.0, (1, 2, 3), "bf16")
    c = normal((3, 5), 1.0, (1, 2, 4), "bf16")
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    r = randint((1000,), 0, 7, (5,))
    assert r.min() >= 0 and r.max() < 7
