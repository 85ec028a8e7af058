"""Pins for the oracle's router: logits, top-k selection, renormalised weights.

Each check compares the oracle with something other than itself: an exact rational replay of
the fp32 fused-multiply-add chain, a rank-counting brute force, numpy's stable argsort, scipy's
softmax, and closed forms (tests/golden/router_closed_forms.json)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from inputs import f32_to_bf16_bits, bf16_bits_to_f32, normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- exact fp32 rounding of a rational, for replaying fmaf step by step ----------------------
def round_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest float32 (ties to even), incl. subnormals."""
    if q == 0:
        return 0.0
    neg = q < 0
    q = -q if neg else q
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp_e = max(e - 23, -149)
    s = q / (Fraction(2) ** ulp_e)
    n = s.numerator // s.denominator
    rem = s - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(Fraction(n) * Fraction(2) ** ulp_e)
    assert abs(v) < 3.4028235e38
    return -v if neg else v


def exact_fma_chain(xrow, wcol):
    acc = 0.0
    for a, b in zip(xrow, wcol):
        acc = round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(acc))
    return acc


def exact_blocked_logit(xrow, wcol):
    """Four blocks of HB = 128 * ceil(H / 512) hidden units, each an exactly replayed fmaf chain
    from 0, then ((c0 + c1) + c2) + c3 with each addition rounded to fp32."""
    H = len(xrow)
    hb = 128 * ((H + 511) // 512)
    total = 0.0
    for b in range(4):
        c = exact_fma_chain(xrow[b * hb:(b + 1) * hb], wcol[b * hb:(b + 1) * hb])
        total = c if b == 0 else round_f32(Fraction(total) + Fraction(c))
    return total


def test_round_f32_helper_against_numpy():
    # the helper itself: rounding exact float64 values must agree with numpy's fp64->fp32 cast
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 30, 2000),
                           [1e-45, 1.5e-45, 3e-39, -2.5e-40]])
    for v in vals:
        assert round_f32(Fraction(float(v))) == float(np.float32(v)), v


@pytest.mark.parametrize("dtype,H", [("f32", 37), ("bf16", 37), ("f32", 300), ("bf16", 1100), ("bf16", 2048)])
def test_logits_are_the_blocked_fp32_fma_chains(dtype, H):
    T, E = 3 if H > 500 else 5, 6
    x = normal((T, H), 1.0, (901, 1, H), dtype)
    w = normal((H, E), 0.3, (901, 2, H), dtype)
    got = oracle.router_logits(x, w)
    xf = x if dtype == "f32" else bf16_bits_to_f32(x)
    wf = w if dtype == "f32" else bf16_bits_to_f32(w)
    want = np.array([[exact_blocked_logit(xf[t], wf[:, e]) for e in range(E)] for t in range(T)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert oracle.router_logit_block(H) == 128 * ((H + 511) // 512)
    if H > 128:   # the block split is not vacuous: one chain over all of h gives other bits somewhere
        one = np.array([[exact_fma_chain(xf[t], wf[:, e]) for e in range(E)] for t in range(T)], np.float32)
        assert not np.array_equal(one.view(np.uint32), want.view(np.uint32))
    # the pin is not vacuous: an unfused chain (round after multiply, then after add) differs
    if dtype == "f32":
        unfused = np.zeros((T, E), np.float32)
        for h in range(H):
            unfused = (unfused + (xf[:, h:h + 1] * wf[h:h + 1, :]).astype(np.float32)).astype(np.float32)
        assert not np.array_equal(unfused, got)
    # and it is within the textbook dot-product error bound of the fp64 value
    ref = xf.astype(np.float64) @ wf.astype(np.float64)
    bound = H * 2.0 ** -24 * (np.abs(xf).astype(np.float64) @ np.abs(wf).astype(np.float64)) * 1.01
    assert np.all(np.abs(got - ref) <= bound + 1e-45)


def rank_count_topk(l, k):
    """Brute force: e is selected iff fewer than k experts beat it (larger logit, or equal logit
    and lower index); its slot is that count."""
    E = l.shape[0]
    idx = np.full(k, -1, np.int64)
    for e in range(E):
        beaten_by = sum(1 for f in range(E) if l[f] > l[e] or (l[f] == l[e] and f < e))
        if beaten_by < k:
            idx[beaten_by] = e
    return idx


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (40, 16, 4), (20, 128, 8), (10, 5, 5), (7, 3, 1)])
def test_topk_selection_brute_force_and_argsort(T, E, k):
    rng = np.random.default_rng(T * 1000 + E * 10 + k)
    # quantised logits so that ties are frequent
    l = (np.round(rng.standard_normal((T, E)) * 2) / 4).astype(np.float32)
    idx, w = oracle.router_topk(l, k, renorm=True)
    for t in range(T):
        assert np.array_equal(idx[t], rank_count_topk(l[t], k))
        assert np.array_equal(idx[t], np.argsort(-l[t], kind="stable")[:k])


@pytest.mark.parametrize("renorm", [True, False])
def test_topk_weights_closed_form(renorm):
    T, E, k = 64, 32, 6
    l = normal((T, E), 1.7, (902, 1), "f32")
    idx, w = oracle.router_topk(l, k, renorm=renorm)
    l64 = l.astype(np.float64)
    p = softmax(l64, axis=1)
    for t in range(T):
        S = idx[t]
        if renorm:
            np.testing.assert_allclose(w[t], softmax(l64[t, S]), rtol=1e-14, atol=0)
            np.testing.assert_allclose(w[t], p[t, S] / p[t, S].sum(), rtol=1e-12, atol=0)
            assert abs(w[t].sum() - 1.0) <= 4 * k * 2.0 ** -53
        else:
            np.testing.assert_allclose(w[t], p[t, S], rtol=1e-13, atol=0)
        assert np.all(np.diff(w[t]) <= 0)


def test_topk_k_equals_E_is_dense_softmax():
    l = normal((16, 12), 1.0, (903, 1), "f32")
    idx, w = oracle.router_topk(l, 12, renorm=True)
    p = softmax(l.astype(np.float64), axis=1)
    for t in range(16):
        np.testing.assert_allclose(w[t], p[t, idx[t]], rtol=1e-14)
        assert sorted(idx[t].tolist()) == list(range(12))


def test_router_golden_closed_forms():
    with open(os.path.join(GOLDEN, "router_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        l = np.array([c["logits"]], np.float32)
        idx, w = oracle.router_topk(l, c["k"], renorm=True)
        assert idx[0].tolist() == c["idx"]
        if "w" in c:
            assert w[0].tolist() == c["w"]  # exact: exp(0) = 1 and the divisions are exact
        else:
            d = 2 + math.exp(-1)
            np.testing.assert_allclose(w[0], [1 / d, 1 / d, math.exp(-1) / d], rtol=1e-15)


def test_bf16_rounding_of_inputs_is_nearest_even():
    # the input generator's rounding (used by both sides) checked against hand cases
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -3.14159, 65504.0,
                     1.0078125 + 2 ** -8], np.float32)
    bits = f32_to_bf16_bits(vals)
    back = bf16_bits_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0            # exactly halfway between 1 and 1+2^-7: ties to even -> 1.0
    assert back[2] == 1.0078125      # 1 + 1.5*2^-8 rounds up
    assert back[3] == 1.0078125      # a quarter of the way to the next bf16: rounds down
    assert back[6] == 1.015625       # halfway between 0x3F81 (odd) and 0x3F82: ties to even -> up
    assert abs(back[4] + 3.140625) == 0.0
    for v, b in zip(vals, back):
        assert abs(float(v) - float(b)) <= abs(float(v)) * 2.0 ** -8


# ---- router statistics ------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (300, 128, 8), (17, 5, 5), (1, 1, 1)])
def test_router_stats_against_scipy_and_bincount(T, E, k):
    g = np.random.default_rng(1234 + T)
    logits = (g.standard_normal((T, E)) * 2).astype(np.float32)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    probs, mean, load = oracle.router_stats(logits, idx)
    ref = softmax(logits.astype(np.float64), axis=1)
    assert np.max(np.abs(probs - ref)) <= 1e-15
    assert np.max(np.abs(mean - ref.mean(axis=0))) <= 1e-15
    assert np.array_equal(load, np.bincount(idx.ravel(), minlength=E))
    assert load.sum() == T * k
    assert abs(mean.sum() - 1.0) <= 1e-12


def test_router_stats_closed_forms_and_dropped_slots():
    T, E, k = 10, 16, 4
    probs, mean, load = oracle.router_stats(np.zeros((T, E), np.float32), np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.all(probs == 1.0 / E) and np.all(mean == 1.0 / E)
    assert list(load) == [T] * k + [0] * (E - k)
    idx = np.array([[0, -1, E, 3]] * T, np.int32)           # out-of-range indices are not counted
    _, _, load = oracle.router_stats(np.zeros((T, E), np.float32), idx, want_probs=False)
    assert load[0] == T and load[3] == T and load.sum() == 2 * T


def test_router_stats_match_raw_softmax_weights():
    g = np.random.default_rng(99)
    logits = (g.standard_normal((50, 32)) * 3).astype(np.float32)
    idx, w = oracle.router_topk(logits, 6, renorm=False)
    probs, _, _ = oracle.router_stats(logits, idx)
    assert np.max(np.abs(np.take_along_axis(probs, idx.astype(np.int64), axis=1) - w)) <= 1e-15
