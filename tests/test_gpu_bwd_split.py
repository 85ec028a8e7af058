"""GPU parity of the FFN backward's products called one at a time (down backward, gate_up backward,
grouped weight gradient with and without a workgroup cap) against the CPU oracle, and of the
three-stream backward schedule against the one-stream layer backward (bit-identical: the same kernels
on the same inputs). Tolerance as elsewhere: max|gpu - ref| / max|ref| <= 1e-2 in bf16."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
import oracle
from inputs import make_layer_inputs, normal
from tests.gpu_util import TOL, as64, dev, host, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


@pytest.mark.parametrize("counts,H,I", [([3, 0, 300, 17, 256], 136, 40), ([0, 0, 1], 64, 32),
                                        ([129, 160, 161, 0, 40], 256, 96), ([512], 2048, 768)])
@pytest.mark.parametrize("cap", [0, 8, 24])
def test_split_products(counts, H, I, cap):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    xp = normal((N, H), 1.0, (991, N, H), "bf16")
    gu = normal((E * H, 2 * I), 0.08, (992, E, H, I), "bf16")
    dn = normal((E * I, H), 0.08, (993, E, H, I), "bf16")
    d_y = normal((N, H), 1.0, (994, N, H), "bf16")
    offs = dev(offsets)
    gu_saved = torch.empty((N, 2 * I), dtype=torch.bfloat16, device="cuda")
    _, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), offs, gu_saved=gu_saved)
    d_gu = moe.moe_grouped_gemm_down_bwd(dev(d_y), dev(dn), gu_saved, offs)
    d_xp = moe.moe_grouped_gemm_gate_up_bwd(d_gu, dev(gu), offs)
    d_down = torch.full((E * I, H), 7.0, dtype=torch.bfloat16, device="cuda")
    d_gate_up = torch.full((E * H, 2 * I), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm_wgrad(h, dev(d_y), offs, d_down, max_workgroups=cap)
    moe.moe_grouped_gemm_wgrad(dev(xp), d_gu, offs, d_gate_up, max_workgroups=cap)
    # the fused call runs the same kernels: bit-identical
    f_dxp, f_dgu_w, f_ddn, f_dgu = moe.moe_grouped_swiglu_ffn_bwd(dev(d_y), dev(xp), gu_saved, h, dev(gu), dev(dn), offs)
    assert torch.equal(d_gu, f_dgu) and torch.equal(d_xp, f_dxp)
    assert torch.equal(d_down, f_ddn) and torch.equal(d_gate_up, f_dgu_w)
    ref_dx, ref_dgu = oracle.expert_rows_bwd(xp, d_y, offsets, gu, dn, want_gu=True)
    assert rel_err(host(d_gu), ref_dgu) <= TOL["bf16"]
    assert rel_err(host(d_xp), ref_dx) <= TOL["bf16"]
    g_dgu, g_ddn = as64(host(d_gate_up)), as64(host(d_down))
    for e in range(E):
        blk_gu, blk_dn = g_dgu[e * H:(e + 1) * H], g_ddn[e * I:(e + 1) * I]
        if counts[e] == 0:
            assert np.all(blk_gu == 0.0) and np.all(blk_dn == 0.0), f"expert {e} without rows"
            continue
        r_gu, r_dn = oracle.expert_weight_grads(xp, d_y, offsets, gu, dn, e)
        assert rel_err(blk_gu, r_gu) <= TOL["bf16"], f"d_gate_up of expert {e}"
        assert rel_err(blk_dn, r_dn) <= TOL["bf16"], f"d_down of expert {e}"


@pytest.mark.parametrize("dtype,M,Nq", [("bf16", 64, 36), ("bf16", 20, 48), ("f32", 64, 64), ("f32", 24, 12)])
def test_wgrad_generic_shapes(dtype, M, Nq):
    # widths that are not multiples of 8 in bf16, and fp32: the generic kernels, against P_e^T Q_e in
    # fp64 (bf16 inputs are exact in fp64); experts without rows get zeros
    counts = [16, 0, 9, 1]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N, E = int(offs[-1]), len(counts)
    P = normal((N, M), 1.0, (1301, N, M), dtype)
    Q = normal((N, Nq), 1.0, (1302, N, Nq), dtype)
    d_w = host(moe.moe_grouped_gemm_wgrad(dev(P), dev(Q), dev(offs)))
    p64, q64 = as64(P), as64(Q)
    for e in range(E):
        blk = as64(d_w[e * M:(e + 1) * M])
        if counts[e] == 0:
            assert np.all(blk == 0.0)
            continue
        ref = p64[offs[e]:offs[e + 1]].T @ q64[offs[e]:offs[e + 1]]
        assert rel_err(blk, ref) <= TOL[dtype], f"expert {e}"


def test_wgrad_argument_errors():
    P = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    Q = torch.zeros((16, 36), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError):            # E = 0: no expert
        moe.moe_grouped_gemm_wgrad(P, Q, torch.tensor([0], dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("T,H,I,E,k,shared,renorm,cus", [(300, 136, 40, 16, 4, 1, True, 16),
                                                         (257, 256, 64, 64, 8, 0, False, 64),
                                                         (64, 64, 32, 8, 2, 1, False, 8),
                                                         (1024, 512, 128, 32, 8, 1, True, 128)])
def test_overlapped_backward(T, H, I, E, k, shared, renorm, cus):
    d = make_layer_inputs(T, H, I, E, k, "bf16", (995, T, E), w_std=0.08, wg_std=0.3, shared=shared, backward=True)
    sgu = dev(d["shared_gate_up"]) if shared else None
    sdn = dev(d["shared_down"]) if shared else None
    x, gu, dn, wg, d_out = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"]), dev(d["d_out"])
    _, bufs = moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, renorm=renorm, shared_gate_up=sgu, shared_down=sdn,
                                    save_for_backward=True)
    ref = moe.moe_layer_backward(d_out, x, gu, dn, bufs, w_gate=wg, renorm=renorm, shared_gate_up=sgu,
                                 shared_down=sdn)
    ob = moe.OverlappedBackward(device=x.device, wgrad_cus=cus)
    for _ in range(2):                             # the schedule's streams and events are reused
        got = moe.LayerGrads(T, H, I, E, k, x.dtype, x.device, I_shared=I if shared else 0, router=True)
        ob(d_out, x, gu, dn, bufs, w_gate=wg, renorm=renorm, shared_gate_up=sgu, shared_down=sdn, grads=got)
        torch.cuda.synchronize()
        for name in ("d_x", "d_gate_up", "d_down", "d_w_gate", "d_y", "d_w", "d_logits", "d_shared_gate_up",
                     "d_shared_down"):
            a, b = getattr(got, name), getattr(ref, name)
            if b is None:
                continue
            assert torch.equal(a, b), name
    # and against the oracle's layer backward, on the token gradient
    ref64 = oracle.moe_backward(d["x"], d["gate_up"], d["down"], k, d["d_out"], w_gate=d["w_gate"], renorm=renorm,
                                shared_gate_up=d.get("shared_gate_up"), shared_down=d.get("shared_down"), experts=[])
    assert rel_err(host(got.d_x), ref64["d_x"]) <= TOL["bf16"]


@pytest.mark.parametrize("counts,H,I", [([0, 300, 1, 0, 257, 142, 640, 33], 200, 64), ([290, 0, 17, 700], 520, 128),
                                        ([256] * 12 + [0, 321], 264, 192)])
def test_gate_up_bwd_row_tile_weights(counts, H, I):
    """dX = dGU gate_up_e^T with 2I a multiple of 128 runs on the persistent kernel with the weights
    staged as row tiles: empty experts, 1-row, band (257-320-row) and multi-row-tile experts, and an
    H that is not a multiple of the 256-column tile. Against the oracle's input gradient."""
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    xp = normal((N, H), 1.0, (1311, N, H), "bf16")
    gu = normal((E * H, 2 * I), 0.08, (1312, E, H, I), "bf16")
    dn = normal((E * I, H), 0.08, (1313, E, H, I), "bf16")
    d_y = normal((N, H), 1.0, (1314, N, H), "bf16")
    offs = dev(offsets)
    gu_saved = torch.empty((N, 2 * I), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), offs, gu_saved=gu_saved)
    d_gu = moe.moe_grouped_gemm_down_bwd(dev(d_y), dev(dn), gu_saved, offs)
    d_xp = torch.full((N + 3, H), 5.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm_gate_up_bwd(d_gu, dev(gu), offs, d_x_perm=d_xp[:N])
    ref_dx, _ = oracle.expert_rows_bwd(xp, d_y, offsets, gu, dn, want_gu=True)
    assert rel_err(host(d_xp[:N]), ref_dx) <= TOL["bf16"]
    assert np.all(as64(host(d_xp[N:])) == 5.0)
