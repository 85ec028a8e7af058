"""The layer's library calls captured in a HIP graph (torch.cuda.graph on the calls' stream): every
replay, with eager work and synchronisations between the replays, gives the eager result bit for
bit. Covers the forward step the benchmark times (rows gathered from x, and from x_perm) and a
training step (forward with saved activations, shared expert, then the whole backward)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
from inputs import make_layer_inputs
from tests.gpu_util import dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _capture(fn):
    side = torch.cuda.Stream()                 # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("T,H,I,E,k,gather", [(4096, 2048, 768, 128, 8, True), (300, 136, 40, 16, 4, True),
                                              (1000, 256, 96, 32, 8, False)])
def test_forward_graph_replays(T, H, I, E, k, gather):
    d = make_layer_inputs(T, H, I, E, k, "bf16", (1101, T, E), w_std=0.02, wg_std=0.3)
    x, gu, dn, wg = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"])
    bufs = moe.LayerBuffers(T, H, I, E, k, x.dtype, x.device, x_perm=not gather)
    run = lambda: moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, bufs=bufs, gather=gather)
    out_ref, _ = run()
    ref = out_ref.clone()
    g = _capture(run)
    for i in range(4):
        bufs.out.fill_(-1.0)                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.out, ref), f"replay {i}"
        # an eager call between replays must not disturb the next replay
        out_e, _ = run()
        assert torch.equal(out_e, ref)


def test_training_step_graph_replays():
    T, H, I, E, k = 257, 256, 64, 16, 4
    d = make_layer_inputs(T, H, I, E, k, "bf16", (1102, T, E), w_std=0.08, wg_std=0.3, shared=1, backward=True)
    x, gu, dn, wg, d_out = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"]), dev(d["d_out"])
    sgu, sdn = dev(d["shared_gate_up"]), dev(d["shared_down"])
    bufs = moe.LayerBuffers(T, H, I, E, k, x.dtype, x.device, gu_saved=True, I_shared=I)
    grads = moe.LayerGrads(T, H, I, E, k, x.dtype, x.device, I_shared=I, router=True)

    def run():
        moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, bufs=bufs, shared_gate_up=sgu, shared_down=sdn,
                              save_for_backward=True)
        moe.moe_layer_backward(d_out, x, gu, dn, bufs, w_gate=wg, shared_gate_up=sgu, shared_down=sdn, grads=grads)

    run()
    names = ("d_x", "d_gate_up", "d_down", "d_w_gate", "d_shared_gate_up", "d_shared_down")
    ref = {n: getattr(grads, n).clone() for n in names}
    out_ref = bufs.out.clone()
    g = _capture(run)
    for i in range(3):
        for n in names:
            getattr(grads, n).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.out, out_ref), f"replay {i}: out"
        for n in names:
            assert torch.equal(getattr(grads, n), ref[n]), f"replay {i}: {n}"
