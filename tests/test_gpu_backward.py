"""GPU parity of the backward pass: every backward call through the C ABI against the CPU oracle,
then the whole layer (routed experts + shared expert + router) against the oracle's composition.
Tolerance as for the forward: max|gpu - ref| / max|ref| <= 1e-2 in bf16, <= 1e-5 in fp32 (fp32
outputs of fp32-accumulated reductions, e.g. d_w and d_logits, use the fp32 bound)."""
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


@pytest.mark.parametrize("T,H,k,dtype", [(64, 64, 2, "f32"), (500, 2048, 8, "bf16"), (77, 136, 3, "bf16"),
                                         (5, 40, 1, "bf16"), (33, 7168, 8, "bf16"), (31, 20, 4, "f32"),
                                         (100, 2048, 9, "bf16"), (40, 136, 16, "bf16"), (21, 256, 32, "bf16"),
                                         (9, 24, 32, "f32"), (13, 12, 32, "bf16"), (7, 5, 20, "f32")])
def test_combine_bwd(T, H, k, dtype):
    N = T * k + 3                                  # three rows no slot points at: left untouched
    g = generator((970, T, H, k))
    ros = g.permutation(N)[:T * k].astype(np.int32)
    if k > 8:
        ros[5::13] = -1                            # dropped slots: zero d_w, no row written
    y = normal((N, H), 1.0, (971, N, H), dtype)
    w = g.random((T, k), dtype=np.float32)
    d_out = normal((T, H), 1.0, (972, T, H), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d_y = torch.full((N, H), 7.0, dtype=tdt, device="cuda")
    d_y, d_w = moe.moe_unpermute_combine_bwd(dev(d_out), dev(y), dev(ros), dev(w), d_y=d_y)
    ref_dy, ref_dw = oracle.combine_bwd(d_out, y, ros, w)
    gy = host(d_y)
    valid = (ros >= 0).reshape(T, k)
    got_dy = gy[np.where(ros >= 0, ros, 0)].reshape(T, k, H)
    assert rel_err(got_dy[valid], ref_dy[valid]) <= TOL[dtype]
    assert rel_err(host(d_w), ref_dw) <= TOL["f32"]
    assert np.all(host(d_w)[~valid] == 0.0)
    untouched = np.setdiff1d(np.arange(N), ros[ros >= 0])
    assert np.all(as64(gy[untouched]) == 7.0)


@pytest.mark.parametrize("T,H,k,dtype,add", [(64, 64, 2, "f32", False), (500, 2048, 8, "bf16", True),
                                             (77, 136, 3, "bf16", False), (5, 40, 1, "bf16", True),
                                             (33, 7168, 8, "bf16", True), (31, 20, 4, "f32", True),
                                             (100, 2048, 9, "bf16", True), (40, 136, 16, "bf16", False),
                                             (21, 256, 32, "bf16", True), (9, 24, 32, "f32", False),
                                             (13, 12, 32, "bf16", True), (7, 5, 20, "f32", True)])
def test_permute_bwd(T, H, k, dtype, add):
    N = T * k
    g = generator((973, T, H, k))
    ros = g.permutation(N).astype(np.int32)
    ros[::7] = -1                                  # dropped slots contribute nothing
    dxp = normal((N, H), 1.0, (974, N, H), dtype)
    dxa = normal((T, H), 1.0, (975, T, H), dtype) if add else None
    got = moe.moe_permute_bwd(dev(dxp), dev(ros), T, k, d_x_add=dev(dxa) if add else None)
    assert rel_err(host(got), oracle.permute_bwd(dxp, ros, k, d_x_add=dxa)) <= TOL[dtype]


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (1000, 128, 8), (77, 256, 8), (50, 1024, 32), (10, 5, 5),
                                   (33, 64, 1), (129, 100, 7)])
@pytest.mark.parametrize("renorm", [True, False])
def test_router_topk_bwd(T, E, k, renorm):
    g = generator((976, T, E, k))
    logits = g.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.router_topk(logits, k, renorm)
    d_w = g.standard_normal((T, k)).astype(np.float32)
    got = moe.moe_router_topk_bwd(dev(logits), dev(idx), dev(w.astype(np.float32)), dev(d_w), renorm)
    ref = oracle.router_topk_bwd(logits, idx, d_w, renorm)
    assert rel_err(host(got), ref) <= TOL["f32"]
    if renorm:                                     # exact zeros off the selected set
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert np.all(host(got)[mask] == 0.0)


@pytest.mark.parametrize("T,H,E,dtype", [(64, 64, 8, "f32"), (300, 136, 72, "bf16"), (1, 8, 1, "bf16"),
                                         (513, 2048, 128, "bf16"), (37, 7168, 256, "bf16"), (70, 24, 130, "f32")])
@pytest.mark.parametrize("add", [False, True])
def test_router_logits_bwd(T, H, E, dtype, add):
    x = normal((T, H), 1.0, (977, T, H), dtype)
    wg = normal((H, E), 0.02, (978, H, E), dtype)
    dl = generator((979, T, E)).standard_normal((T, E)).astype(np.float32)
    dxa = normal((T, H), 0.01, (980, T, H), dtype) if add else None
    dwg, dx = moe.moe_router_logits_bwd(dev(x), dev(wg), dev(dl), d_x_in=dev(dxa) if add else None)
    ref_dwg, ref_dx = oracle.router_logits_bwd(x, wg, dl)
    if add:
        ref_dx = ref_dx + as64(dxa)
    assert rel_err(host(dwg), ref_dwg) <= TOL["f32"]
    assert rel_err(host(dx), ref_dx) <= TOL[dtype]


def test_router_logits_bwd_no_tokens():
    """T = 0: d_w_gate = x^T dl over no tokens is zero; nothing else is written."""
    H, E = 64, 16
    dwg = torch.full((H, E), 5.0, device="cuda")
    x = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
    dwg, dx = moe.moe_router_logits_bwd(x, torch.zeros((H, E), dtype=torch.bfloat16, device="cuda"),
                                        torch.zeros((0, E), device="cuda"), d_w_gate=dwg)
    torch.cuda.synchronize()
    assert torch.all(dwg == 0) and dx.shape == (0, H)


@pytest.mark.parametrize("counts,H,I,dtype", [
    ([0, 300, 1, 0, 257, 142], 136, 40, "bf16"),
    ([256, 256, 256, 256], 256, 192, "bf16"),
    ([1000], 64, 24, "bf16"),
    ([3, 0, 0, 517, 31, 64, 0, 1], 512, 128, "bf16"),
    ([0, 0, 0], 64, 32, "bf16"),
    ([600, 5], 7168, 256, "bf16"),
    ([288, 289, 270, 0, 257], 136, 40, "bf16"),        # tiles with an extra band of one or two blocks
    ([320, 321, 300, 0, 641], 136, 40, "bf16"),        # two-block bands and 320-row tiles
    # the generic kernels: fp32, and bf16 widths that are not multiples of 8
    ([17, 0, 40], 64, 32, "f32"),
    ([5, 9, 0, 2], 24, 12, "f32"),
    ([0, 30, 1, 0, 25, 14], 36, 20, "bf16"),
])
def test_grouped_swiglu_ffn_bwd(counts, H, I, dtype):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xp = normal((N, H), 1.0, (981, N, H), dtype)
    gu = normal((E * H, 2 * I), 0.08, (982, E, H, I), dtype)
    dn = normal((E * I, H), 0.08, (983, E, H, I), dtype)
    d_y = normal((N, H), 1.0, (984, N, H), dtype)
    gu_saved = torch.empty((N, 2 * I), dtype=tdt, device="cuda")
    _, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets), gu_saved=gu_saved)
    d_gate_up = torch.full((E * H, 2 * I), 7.0, dtype=tdt, device="cuda")
    d_down = torch.full((E * I, H), 7.0, dtype=tdt, device="cuda")
    d_xp, d_gate_up, d_down, d_gu = moe.moe_grouped_swiglu_ffn_bwd(dev(d_y), dev(xp), gu_saved, h, dev(gu), dev(dn),
                                                                   dev(offsets), d_gate_up=d_gate_up, d_down=d_down)
    g_dgu, g_ddn = as64(host(d_gate_up)), as64(host(d_down))
    if N:
        ref_dx, ref_dgu = oracle.expert_rows_bwd(xp, d_y, offsets, gu, dn, want_gu=True)
        assert rel_err(host(d_gu), ref_dgu) <= TOL[dtype]
        assert rel_err(host(d_xp), ref_dx) <= TOL[dtype]
    for e in range(E):
        blk_gu, blk_dn = g_dgu[e * H:(e + 1) * H], g_ddn[e * I:(e + 1) * I]
        if counts[e] == 0:                         # experts without rows: exact zeros
            assert np.all(blk_gu == 0.0) and np.all(blk_dn == 0.0)
            continue
        r_gu, r_dn = oracle.expert_weight_grads(xp, d_y, offsets, gu, dn, e)
        assert rel_err(blk_gu, r_gu) <= TOL[dtype], f"d_gate_up of expert {e}"
        assert rel_err(blk_dn, r_dn) <= TOL[dtype], f"d_down of expert {e}"


@pytest.mark.parametrize("T,H,I,E,k,shared,dtype", [(300, 136, 40, 16, 4, 1, "bf16"), (257, 256, 64, 64, 8, 0, "bf16"),
                                                    (64, 64, 32, 8, 2, 1, "bf16"), (1, 64, 32, 8, 8, 1, "bf16"),
                                                    (96, 48, 24, 8, 2, 1, "f32"), (40, 36, 20, 4, 2, 0, "bf16")])
@pytest.mark.parametrize("renorm", [True, False])
def test_layer_backward(T, H, I, E, k, shared, dtype, renorm):
    d = make_layer_inputs(T, H, I, E, k, dtype, (985, T, E), w_std=0.08, wg_std=0.3, shared=shared,
                          backward=True)
    sgu = dev(d["shared_gate_up"]) if shared else None
    sdn = dev(d["shared_down"]) if shared else None
    x, gu, dn, wg, d_out = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"]), dev(d["d_out"])
    out, bufs = moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, renorm=renorm, shared_gate_up=sgu, shared_down=sdn,
                                      save_for_backward=True)
    g = moe.moe_layer_backward(d_out, x, gu, dn, bufs, w_gate=wg, renorm=renorm, shared_gate_up=sgu,
                               shared_down=sdn)
    ref_out, ridx, _, _ = oracle.moe_forward(d["x"], d["gate_up"], d["down"], k, w_gate=d["w_gate"], renorm=renorm,
                                             shared_gate_up=d.get("shared_gate_up"), shared_down=d.get("shared_down"))
    assert np.array_equal(host(bufs.topk_idx), ridx)
    assert rel_err(host(out), ref_out) <= TOL[dtype]
    r = oracle.moe_backward(d["x"], d["gate_up"], d["down"], k, d["d_out"], w_gate=d["w_gate"], renorm=renorm,
                            shared_gate_up=d.get("shared_gate_up"), shared_down=d.get("shared_down"))
    assert rel_err(host(g.d_w), r["d_w"]) <= TOL[dtype]
    assert rel_err(host(g.d_logits), r["d_logits"]) <= TOL[dtype]
    assert rel_err(host(g.d_w_gate), r["d_w_gate"]) <= TOL[dtype]
    assert rel_err(host(g.d_x), r["d_x"]) <= TOL[dtype]
    assert rel_err(host(g.d_gate_up), np.concatenate([r["d_gate_up"][e] for e in range(E)])) <= TOL[dtype]
    assert rel_err(host(g.d_down), np.concatenate([r["d_down"][e] for e in range(E)])) <= TOL[dtype]
    if shared:
        assert rel_err(host(g.d_shared_gate_up), r["d_shared_gate_up"]) <= TOL[dtype]
        assert rel_err(host(g.d_shared_down), r["d_shared_down"]) <= TOL[dtype]
