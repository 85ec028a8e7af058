"""GPU parity: every kernel of the layer, called through the C ABI, against the CPU oracle.

Integer results (indices, counts, offsets, row maps, permuted rows) must match bit for bit; the
router logits too (both sides run the same fp32 FMA chain). Floating-point outputs must satisfy
max|gpu - ref| / max|ref| <= 1e-2 in bf16 and <= 1e-5 in fp32. Inputs are seeded and synthetic."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
import oracle
from inputs import make_layer_inputs, normal
from inputs.generators import generator
from tests.gpu_util import TOL, as64, dev, host, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def routing(T, E, k, key, skew=None):
    """k distinct experts per token; skew='one' sends every token to expert 0 (plus k-1 others);
    skew='empty' never uses the last two experts."""
    g = generator(key)
    rows = []
    for _ in range(T):
        if skew == "empty":
            rows.append(g.permutation(E - 2)[:k])
        elif skew == "one":
            rows.append(np.concatenate([[0], 1 + g.permutation(E - 1)[:k - 1]]))
        else:
            rows.append(g.permutation(E)[:k])
    return np.array(rows, np.int32).reshape(T, k)


# ---- router -----------------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,E,dtype", [(64, 64, 8, "f32"), (300, 136, 72, "bf16"), (1, 8, 1, "bf16"),
                                         (513, 2048, 128, "bf16"), (37, 7168, 256, "bf16"), (70, 24, 130, "f32"),
                                         # matrix-core kernel: bf16, H % 32 == 0, E % 8 == 0; empty hidden
                                         # blocks (H < 384), a ragged expert tile, ragged token tiles
                                         (100, 96, 8, "bf16"), (257, 640, 40, "bf16"), (65, 1056, 200, "bf16"),
                                         (4096, 2048, 128, "bf16")])
def test_router_logits_bit_exact(T, H, E, dtype):
    x = normal((T, H), 1.0, (950, T, H), dtype)
    w = normal((H, E), 0.02, (951, H, E), dtype)
    got = host(moe.moe_router_logits(dev(x), dev(w)))
    want = oracle.router_logits(x, w)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("T,H,E,dtype", [(4096, 72, 256, "bf16"), (16384, 40, 64, "f32")])
def test_router_logits_eight_chains_per_lane(T, H, E, dtype):
    # shapes with at least 256 workgroups of 64 experts: the launch that gives each lane eight chains
    x = normal((T, H), 1.0, (953, T, H), dtype)
    w = normal((H, E), 0.02, (954, H, E), dtype)
    got = host(moe.moe_router_logits(dev(x), dev(w)))
    assert np.array_equal(got.view(np.uint32), oracle.router_logits(x, w).view(np.uint32))


def test_router_logits_subnormal_products():
    # |x w| ~ 1e-40: every product and most partial sums are subnormal, on both kinds of waves
    T, H, E = 130, 200, 40
    x = normal((T, H), 1e-20, (955, T, H), "f32")
    w = normal((H, E), 1e-20, (956, H, E), "f32")
    want = oracle.router_logits(x, w)
    assert np.count_nonzero((want != 0) & (np.abs(want) < np.finfo(np.float32).tiny)) > T * E // 2
    got = host(moe.moe_router_logits(dev(x), dev(w)))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_router_logits_subnormal_products_matrix_cores():
    # the same on the bf16 matrix-core kernel: subnormal products and partial sums are kept, not flushed
    T, H, E = 130, 256, 40
    x = normal((T, H), 1e-20, (957, T, H), "bf16")
    w = normal((H, E), 1e-20, (958, H, E), "bf16")
    want = oracle.router_logits(x, w)
    assert np.count_nonzero((want != 0) & (np.abs(want) < np.finfo(np.float32).tiny)) > T * E // 2
    got = host(moe.moe_router_logits(dev(x), dev(w)))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (1000, 128, 8), (77, 256, 8), (50, 1024, 32), (10, 5, 5),
                                   (33, 64, 1), (20, 3, 3), (129, 100, 7), (200, 16, 16), (70, 32, 32),
                                   (65, 250, 32), (4097, 128, 8), (100, 257, 9), (3, 200, 17)])
@pytest.mark.parametrize("renorm", [True, False])
def test_router_topk(T, E, k, renorm):
    g = generator((952, T, E, k))
    logits = (np.round(g.standard_normal((T, E)) * 4) / 4).astype(np.float32)   # frequent ties
    idx, w = moe.moe_router_topk(dev(logits), k, renorm)
    ridx, rw = oracle.router_topk(logits, k, renorm)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(w), rw) <= TOL["f32"]


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (1000, 128, 8), (77, 256, 8), (50, 1024, 32), (10, 5, 5),
                                   (4096, 128, 8), (300, 100, 7)])
def test_router_stats(T, E, k):
    g = generator((963, T, E, k))
    logits = (g.standard_normal((T, E)) * 2).astype(np.float32)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if T >= 10:
        idx[3, 0] = -1          # a dropped slot and an out-of-range index are not counted
        idx[5, k - 1] = E
    probs, mean, load = moe.moe_router_stats(dev(logits), dev(idx))
    rp, rm, rl = oracle.router_stats(logits, idx)
    assert rel_err(host(probs), rp) <= TOL["f32"]
    assert rel_err(host(mean), rm) <= TOL["f32"]
    assert np.array_equal(host(load), rl)
    _, mean2, _ = moe.moe_router_stats(dev(logits), dev(idx), want_probs=False)
    assert np.array_equal(host(mean).view(np.uint32), host(mean2).view(np.uint32))   # deterministic


def test_router_stats_no_tokens():
    _, mean, load = moe.moe_router_stats(torch.zeros((0, 16), device="cuda"),
                                         torch.zeros((0, 4), dtype=torch.int32, device="cuda"))
    assert torch.all(mean == 0) and torch.all(load == 0)


# ---- permute ----------------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,E,k,dtype,skew", [
    (64, 64, 8, 2, "f32", None), (1000, 136, 16, 4, "bf16", None), (257, 2048, 128, 8, "bf16", None),
    (1, 8, 1, 1, "bf16", None), (600, 40, 4, 4, "bf16", None), (700, 64, 32, 8, "bf16", "one"),
    (513, 24, 12, 3, "bf16", "empty"), (300, 30, 8, 2, "bf16", None), (2049, 16, 1024, 32, "f32", None)])
def test_permute_bit_exact(T, H, E, k, dtype, skew):
    x = normal((T, H), 1.0, (953, T, H), dtype)
    idx = routing(T, E, k, (954, T, E, k), skew)
    x_perm, plan = moe.moe_permute(dev(x), dev(idx), E)
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    assert np.array_equal(host(plan.counts), counts)
    assert np.array_equal(host(plan.offsets), offsets)
    assert np.array_equal(host(plan.row_of_slot), ros)
    assert np.array_equal(host(plan.slot_of_row), sor)
    want = oracle.permute_rows(x, sor, k)
    assert np.array_equal(host(x_perm), want)


def routing_repeats_drops(T, E, k, key, drop):
    """Caller-supplied routing that the router never produces: a token may name one expert in
    several slots, and with drop=True some indices lie outside [0, E) (-1, E, large)."""
    g = generator(key)
    idx = g.integers(0, E, (T, k)).astype(np.int32)
    if drop:
        knock = g.random((T, k)) < 0.2
        idx = np.where(knock, g.choice(np.array([-1, E, -5, 1 << 24]), (T, k)), idx).astype(np.int32)
        idx[0, 0] = -1
    return idx


@pytest.mark.parametrize("T,H,E,k,drop", [(300, 40, 8, 4, False), (257, 64, 16, 8, True), (64, 16, 3, 3, False),
                                          (1000, 24, 128, 8, True), (129, 8, 32, 32, True), (70, 48, 1024, 5, True),
                                          (2, 16, 3, 2, True), (50, 3, 40, 32, True)])
def test_permute_repeats_and_drops(T, H, E, k, drop):
    """Reading r19 through moe_permute: out-of-range indices get no row and are not counted; repeated
    experts get one row per slot in (expert, token, slot) order. Rows past offsets[E] are untouched."""
    x = normal((T, H), 1.0, (964, T, H), "bf16")
    idx = routing_repeats_drops(T, E, k, (965, T, E, k), drop)
    N = T * k
    x_perm = torch.full((N, H), 3.0, dtype=torch.bfloat16, device="cuda")
    plan = moe.Plan(torch.empty(E, dtype=torch.int32, device="cuda"),
                    torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                    torch.empty(N, dtype=torch.int32, device="cuda"),
                    torch.full((N,), -9, dtype=torch.int32, device="cuda"))
    x_perm, plan = moe.moe_permute(dev(x), dev(idx), E, x_perm=x_perm, plan=plan)
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    n = int(offsets[E])
    assert np.array_equal(host(plan.counts), counts)
    assert np.array_equal(host(plan.offsets), offsets)
    assert np.array_equal(host(plan.row_of_slot), ros)
    gs = host(plan.slot_of_row)
    assert np.array_equal(gs[:n], sor[:n]) and np.all(gs[n:] == -9)
    gx = host(x_perm)
    assert np.array_equal(gx[:n], oracle.permute_rows(x, sor[:n], k))
    assert np.all(as64(gx[n:]) == 3.0)
    if drop:
        assert n < N


@pytest.mark.parametrize("T,H,E,k,rows", [(1000, 64, 128, 8, True), (77, 40, 256, 8, True), (50, 24, 1024, 32, True),
                                          (64, 16, 8, 2, False), (130, 8, 200, 16, True), (4097, 16, 128, 8, False),
                                          (1, 8, 1, 1, True), (129, 32, 64, 32, True)])
@pytest.mark.parametrize("renorm", [True, False])
def test_router_topk_permute(T, H, E, k, rows, renorm):
    """The fused call: the same bits as moe_router_topk then moe_permute, and the oracle's plan."""
    g = generator((966, T, E, k))
    logits = (np.round(g.standard_normal((T, E)) * 4) / 4).astype(np.float32)   # frequent ties
    x = normal((T, H), 1.0, (967, T, H), "bf16")
    idx, w, xp, plan = moe.moe_router_topk_permute(dev(logits), k, dev(x), renorm=renorm, rows=rows)
    idx2, w2 = moe.moe_router_topk(dev(logits), k, renorm)
    xp2, plan2 = moe.moe_permute(dev(x), idx2, E, rows=rows)
    assert np.array_equal(host(idx), host(idx2))
    assert np.array_equal(host(w).view(np.uint32), host(w2).view(np.uint32))
    for a, b in [(plan.counts, plan2.counts), (plan.offsets, plan2.offsets), (plan.row_of_slot, plan2.row_of_slot),
                 (plan.slot_of_row, plan2.slot_of_row)]:
        assert np.array_equal(host(a), host(b))
    ridx, rw = oracle.router_topk(logits, k, renorm)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(w), rw) <= TOL["f32"]
    counts, offsets, ros, sor = oracle.permute_plan(ridx, E)
    assert np.array_equal(host(plan.counts), counts) and np.array_equal(host(plan.offsets), offsets)
    assert np.array_equal(host(plan.row_of_slot), ros) and np.array_equal(host(plan.slot_of_row), sor)
    if rows:
        assert np.array_equal(host(xp), oracle.permute_rows(x, sor, k))
    else:
        assert xp is None


# ---- grouped FFN ------------------------------------------------------------------------------
@pytest.mark.parametrize("counts,H,I,dtype", [
    ([0, 300, 1, 0, 257, 142], 136, 40, "bf16"),
    ([256, 256, 256, 256], 256, 192, "bf16"),
    ([1000], 64, 24, "bf16"),
    ([3, 0, 0, 517, 31, 64, 0, 1], 512, 128, "bf16"),
    ([16, 16, 16, 16, 16, 16, 16, 16], 64, 32, "f32"),
    ([0, 5, 0, 40], 48, 16, "f32"),
    ([288, 289, 270, 0, 256, 577], 136, 40, "bf16"),   # tiles with an extra band of one 32-row block
    ([260, 300], 256, 384, "bf16"),
    ([320, 321, 319, 0, 640, 641, 33, 290], 136, 40, "bf16"),   # two-block bands, 320-row tiles, splits
    ([300, 310, 256, 290, 333], 512, 256, "bf16"),
    # K just below, just above and three rows-of-64 past a multiple of the 64-deep row-operand stage
    ([290, 0, 300, 17, 320], 56, 72, "bf16"),
    ([301, 64, 0, 289], 120, 200, "bf16"),
    ([257, 33, 1], 200, 56, "bf16"),
    # bf16 widths that are not multiples of 8: the generic kernels
    ([0, 30, 1, 0, 25, 14], 36, 20, "bf16"),
    ([70, 3], 100, 13, "bf16"),
])
def test_grouped_swiglu_ffn(counts, H, I, dtype):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    pad = 5                                              # rows past offsets[E] must stay untouched
    xp = normal((N + pad, H), 1.0, (955, N, H), dtype)
    gu = normal((E * H, 2 * I), 0.02 * 4, (956, E, H, I), dtype)
    dn = normal((E * I, H), 0.02 * 4, (957, E, H, I), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.full((N + pad, H), 7.0, dtype=tdt, device="cuda")
    gu_saved = torch.zeros((N + pad, 2 * I), dtype=tdt, device="cuda")
    y, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets), y=y, gu_saved=gu_saved)
    ry, ra, rgu = oracle.expert_rows(xp[:N], offsets, gu, dn, want_act=True, want_gu=True)
    gy = host(y)
    assert rel_err(gy[:N], ry) <= TOL[dtype]
    assert rel_err(host(h)[:N], ra) <= TOL[dtype]
    assert rel_err(host(gu_saved)[:N], rgu) <= TOL[dtype]
    assert np.all(as64(gy[N:]) == 7.0)


# ---- combine ----------------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,k,dtype,res", [(64, 64, 2, "f32", False), (1000, 2048, 8, "bf16", True),
                                             (77, 136, 3, "bf16", False), (5, 40, 1, "bf16", True),
                                             (300, 7168, 8, "bf16", False), (31, 20, 4, "f32", True),
                                             (200, 2048, 9, "bf16", True), (65, 136, 16, "bf16", False),
                                             (33, 256, 32, "bf16", True), (17, 40, 32, "f32", False),
                                             (19, 20, 32, "f32", True), (23, 12, 16, "bf16", False)])
def test_unpermute_combine(T, H, k, dtype, res):
    N = T * k
    g = generator((958, T, H, k))
    ros = g.permutation(N).astype(np.int32)
    if k > 8:
        ros[::11] = -1                             # dropped slots, also in the second batch of loads
    y = normal((N, H), 1.0, (959, N, H), dtype)
    w = g.random((T, k), dtype=np.float32)
    r = normal((T, H), 1.0, (960, T, H), dtype) if res else None
    out = moe.moe_unpermute_combine(dev(y), dev(ros), dev(w), residual=dev(r) if res else None)
    assert rel_err(host(out), oracle.combine(y, ros, w, residual=r)) <= TOL[dtype]


# ---- whole layer, small shapes -------------------------------------------------------------------
@pytest.mark.parametrize("T,H,I,E,k,dtype", [(64, 64, 32, 8, 2, "f32"), (300, 136, 40, 16, 4, "bf16"),
                                             (1, 64, 32, 8, 8, "bf16"), (257, 256, 64, 64, 8, "bf16"),
                                             (100, 48, 16, 1, 1, "bf16"), (50, 32, 16, 4, 4, "f32"),
                                             (130, 64, 32, 32, 16, "bf16"), (70, 40, 24, 64, 32, "bf16"),
                                             (90, 32, 16, 300, 9, "f32")])
@pytest.mark.parametrize("renorm", [True, False])
def test_layer_small(T, H, I, E, k, dtype, renorm):
    d = make_layer_inputs(T, H, I, E, k, dtype, (961, T, E), w_std=0.08, wg_std=0.3)
    out, bufs = moe.moe_layer_forward(dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), k, w_gate=dev(d["w_gate"]),
                                      renorm=renorm)
    ref, ridx, rw, rlog = oracle.moe_forward(d["x"], d["gate_up"], d["down"], k, w_gate=d["w_gate"], renorm=renorm)
    assert np.array_equal(host(bufs.logits).view(np.uint32), rlog.view(np.uint32))
    assert np.array_equal(host(bufs.topk_idx), ridx)
    assert rel_err(host(out), ref) <= TOL[dtype]


def test_layer_determinism():
    d = make_layer_inputs(512, 256, 128, 32, 4, "bf16", (962,), w_std=0.08)
    args = (dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), 4)
    o1, b1 = moe.moe_layer_forward(*args, w_gate=dev(d["w_gate"]))
    o1 = host(o1).copy()
    p1 = host(b1.plan.row_of_slot).copy()
    o2, b2 = moe.moe_layer_forward(*args, w_gate=dev(d["w_gate"]))
    assert np.array_equal(o1, host(o2)) and np.array_equal(p1, host(b2.plan.row_of_slot))
