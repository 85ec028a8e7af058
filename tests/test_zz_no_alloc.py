"""The allocation-free permute (moe_permute_noalloc) against moe_permute with a workspace: bit-identical
plan and permuted rows on two calls in a row, the second with a smaller input (the fixed scratch keeps
the first call's contents), and the size limit of the fixed scratch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
from inputs import normal
from inputs.generators import generator
from tests.gpu_util import dev, host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _routing(T, E, k, key, repeats):
    g = generator(key)
    if repeats:
        idx = g.integers(0, E, (T, k))
        idx[g.random((T, k)) < 0.1] = -1
        return idx.astype(np.int32)
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _buffers(T, H, E, k):
    N = T * k
    plan = moe.Plan(torch.full((E,), -3, dtype=torch.int32, device="cuda"),
                    torch.full((E + 1,), -3, dtype=torch.int32, device="cuda"),
                    torch.full((N,), -3, dtype=torch.int32, device="cuda"),
                    torch.full((N,), -3, dtype=torch.int32, device="cuda"))
    return torch.zeros((N, H), dtype=torch.bfloat16, device="cuda"), plan


def _same(a, b):
    return np.array_equal(host(a), host(b))


@pytest.mark.parametrize("first,second", [((4096, 256, 128, 8, False), (1000, 64, 16, 4, False)),
                                          ((2049, 72, 1024, 32, True), (300, 40, 64, 8, True)),
                                          ((513, 2048, 128, 8, False), (1, 8, 1, 1, False))])
def test_noalloc_matches_workspace_permute(first, second):
    for n, (T, H, E, k, repeats) in enumerate([first, second]):
        x = dev(normal((T, H), 1.0, (1200, n, T, H), "bf16"))
        idx = dev(_routing(T, E, k, (1201, n, T, E, k), repeats))
        xp_ref, plan_ref = moe.moe_permute(x, idx, E)
        xp, plan = _buffers(T, H, E, k)
        moe.moe_permute_noalloc(x, idx, E, xp, plan)
        torch.cuda.synchronize()
        assert _same(plan.counts, plan_ref.counts) and _same(plan.offsets, plan_ref.offsets)
        assert _same(plan.row_of_slot, plan_ref.row_of_slot)
        nrows = int(host(plan_ref.offsets)[E])
        assert _same(plan.slot_of_row[:nrows], plan_ref.slot_of_row[:nrows])
        assert _same(xp[:nrows], xp_ref[:nrows])


def test_noalloc_plan_only_and_size_limit():
    T, H, E, k = 700, 32, 32, 4
    x = dev(normal((T, H), 1.0, (1202,), "bf16"))
    idx = dev(_routing(T, E, k, (1203,), False))
    _, plan_ref = moe.moe_permute(x, idx, E, rows=False)
    _, plan = _buffers(T, H, E, k)
    moe.moe_permute_noalloc(x, idx, E, None, plan, rows=False)
    torch.cuda.synchronize()
    assert _same(plan.row_of_slot, plan_ref.row_of_slot) and _same(plan.slot_of_row, plan_ref.slot_of_row)
    # ceil(T/16) * E above 2^20 chunk counts: refused before anything is launched
    Tb, Eb = 16 * 1025, 1024
    xb = torch.zeros((Tb, 8), dtype=torch.bfloat16, device="cuda")
    ib = torch.zeros((Tb, 1), dtype=torch.int32, device="cuda")
    xpb, planb = _buffers(Tb, 8, Eb, 1)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_permute_noalloc(xb, ib, Eb, xpb, planb)
    assert err.value.status == moe.MOE_ERR_WORKSPACE
