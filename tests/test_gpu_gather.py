"""GPU parity of the gathering grouped FFN (the permute folded into the first grouped matmul): its
h, g|u and y must equal, bit for bit, those of the same FFN run on the materialised x_perm, and
match the oracle within the float tolerance. The plan-only permute must produce the same plan as
the full one. Inputs are seeded and synthetic."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
import oracle
from inputs import make_layer_inputs, normal
from inputs.generators import generator
from tests.gpu_util import TOL, dev, host, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def routing(T, E, k, key, weights=None):
    """k distinct experts per token, drawn with optional per-expert weights (skew, empty experts)."""
    g = generator(key)
    p = None if weights is None else np.asarray(weights, np.float64) / np.sum(weights)
    return np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


CASES = [
    # T, H, I, E, k, dtype, expert weights (None = uniform; zeros make empty experts)
    (64, 64, 32, 8, 2, "f32", None),
    (300, 136, 40, 16, 4, "bf16", [0, 1, 1, 0, 4, 1, 1, 1, 0.2, 1, 1, 1, 1, 1, 3, 1]),
    (600, 136, 40, 4, 2, "bf16", None),          # ~300 rows per expert: tiles with the extra band
    (1100, 256, 64, 4, 1, "bf16", [1, 1, 0.1, 0]),  # > 288 rows: two row tiles per expert
    (513, 2048, 768, 128, 8, "bf16", None),
    (77, 48, 16, 5, 3, "f32", [1, 0, 1, 1, 1]),
    (600, 120, 72, 4, 2, "bf16", None),          # K = 120 / 72: ragged 64-deep row-operand stages, band tiles
    (700, 200, 56, 4, 2, "bf16", [1, 1, 1, 0.2]),
]


@pytest.mark.parametrize("T,H,I,E,k,dtype,wts", CASES)
def test_gather_ffn_equals_permuted(T, H, I, E, k, dtype, wts):
    x = normal((T, H), 1.0, (970, T, H), dtype)
    gu = normal((E * H, 2 * I), 0.08, (971, E, H, I), dtype)
    dn = normal((E * I, H), 0.08, (972, E, H, I), dtype)
    idx = routing(T, E, k, (973, T, E, k), wts)
    xd, gud, dnd = dev(x), dev(gu), dev(dn)
    x_perm, plan = moe.moe_permute(xd, dev(idx), E)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    N = T * k
    g1 = torch.zeros((N, 2 * I), dtype=tdt, device="cuda")
    y1, h1 = moe.moe_grouped_swiglu_ffn(x_perm, gud, dnd, plan.offsets, gu_saved=g1)
    # gathering run, into buffers pre-filled with a marker: every row below offsets[E] gets written
    g2 = torch.full((N, 2 * I), 3.0, dtype=tdt, device="cuda")
    y2 = torch.full((N, H), 3.0, dtype=tdt, device="cuda")
    h2 = torch.full((N, I), 3.0, dtype=tdt, device="cuda")
    y2, h2 = moe.moe_grouped_swiglu_ffn_gather(xd, plan.slot_of_row, k, gud, dnd, plan.offsets, h=h2, y=y2,
                                                gu_saved=g2)
    n = int(host(plan.offsets)[-1])
    for a, b in ((h1, h2), (g1, g2), (y1, y2)):
        assert torch.equal(a[:n].view(torch.int16 if dtype == "bf16" else torch.int32),
                           b[:n].view(torch.int16 if dtype == "bf16" else torch.int32))
    # and against the oracle on the oracle's own permutation
    _, offsets, _, sor = oracle.permute_plan(idx, E)
    ry, ra, _ = oracle.expert_rows(oracle.permute_rows(x, sor, k), offsets, gu, dn, want_act=True, want_gu=True)
    assert rel_err(host(y2)[:n], ry) <= TOL[dtype]
    assert rel_err(host(h2)[:n], ra) <= TOL[dtype]


def test_gather_first_matmul_alone():
    T, H, I, E, k = 200, 136, 40, 6, 3
    x = normal((T, H), 1.0, (974,), "bf16")
    gu = normal((E * H, 2 * I), 0.08, (975,), "bf16")
    idx = routing(T, E, k, (976,))
    xd, gud = dev(x), dev(gu)
    x_perm, plan = moe.moe_permute(xd, dev(idx), E)
    h1 = moe.moe_grouped_gemm_swiglu(x_perm, gud, plan.offsets)
    h2 = moe.moe_grouped_gemm_swiglu_gather(xd, plan.slot_of_row, k, gud, plan.offsets)
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))


@pytest.mark.parametrize("T,E,k", [(1000, 16, 4), (257, 128, 8), (5, 3, 3)])
def test_permute_plan_only(T, E, k):
    x = normal((T, 64), 1.0, (977, T), "bf16")
    idx = routing(T, E, k, (978, T, E, k))
    _, p1 = moe.moe_permute(dev(x), dev(idx), E)
    none, p2 = moe.moe_permute(dev(x), dev(idx), E, rows=False)
    assert none is None
    for name in ("counts", "offsets", "row_of_slot", "slot_of_row"):
        assert torch.equal(getattr(p1, name), getattr(p2, name))


@pytest.mark.parametrize("T,H,I,E,k,dtype", [(256, 128, 64, 16, 4, "bf16"), (64, 64, 32, 8, 2, "f32")])
def test_layer_gather_equals_permuted(T, H, I, E, k, dtype):
    d = make_layer_inputs(T, H, I, E, k, dtype, (979, T, E), w_std=0.08, wg_std=0.3)
    args = (dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), k)
    o1, _ = moe.moe_layer_forward(*args, w_gate=dev(d["w_gate"]))
    o1 = o1.clone()
    o2, b2 = moe.moe_layer_forward(*args, w_gate=dev(d["w_gate"]), gather=True)
    assert b2.x_perm is None
    assert torch.equal(o1, o2)
    ref, _, _, _ = oracle.moe_forward(d["x"], d["gate_up"], d["down"], k, w_gate=d["w_gate"])
    assert rel_err(host(o2), ref) <= TOL[dtype]


def test_gather_rejects_bad_arguments():
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    gu = torch.zeros((2 * 16, 16), dtype=torch.bfloat16, device="cuda")
    sor = torch.zeros(8, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, 4, 8], dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm_swiglu_gather(x, sor, 2, gu, offs, N=9)      # N > T*k
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm_swiglu_gather(x, sor, 0, gu, offs, N=0)      # k < 1
