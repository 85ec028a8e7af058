"""GPU parity of the multi-stream schedules. The Domino-style chunked forward routes chunk c+1 on a
side stream while chunk c's grouped FFN runs on the main stream; the expert-group FFN runs groups of
experts on their own streams. Per token the output must equal, bit for bit, the one-shot layer
forward (and hence the oracle within tolerance), on every call of a reused schedule. Inputs are
seeded and synthetic."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
import oracle
from inputs import make_layer_inputs
from tests.gpu_util import TOL, dev, host, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


@pytest.mark.parametrize("T,H,I,E,k,dtype,chunks,gather", [
    (1000, 256, 128, 16, 4, "bf16", 2, True),
    (1000, 256, 128, 16, 4, "bf16", 2, False),
    (777, 136, 40, 8, 2, "bf16", 3, True),
    (64, 64, 32, 8, 2, "f32", 2, True),
])
def test_chunked_forward_equals_one_shot(T, H, I, E, k, dtype, chunks, gather):
    d = make_layer_inputs(T, H, I, E, k, dtype, (980, T, E), w_std=0.08, wg_std=0.3)
    x, gu, dn, wg = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"])
    ref, _ = moe.moe_layer_forward(x, gu, dn, k, w_gate=wg)
    ref = ref.clone()
    cf = moe.ChunkedForward(T, H, I, E, k, x.dtype, x.device, chunks=chunks, gather=gather)
    for overlap in (True, False, True):
        for _ in range(3):                      # reused buffers, calls queued back to back
            out = cf(x, gu, dn, w_gate=wg, overlap=overlap)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    want, _, _, _ = oracle.moe_forward(d["x"], d["gate_up"], d["down"], k, w_gate=d["w_gate"])
    assert rel_err(host(out), want) <= TOL[dtype]


def test_chunked_forward_given_logits():
    T, H, I, E, k = 512, 128, 64, 32, 4
    d = make_layer_inputs(T, H, I, E, k, "bf16", (981,), w_std=0.08, logits_std=0.1)
    x, gu, dn, lg = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["logits"])
    ref, _ = moe.moe_layer_forward(x, gu, dn, k, logits=lg)
    ref = ref.clone()
    cf = moe.ChunkedForward(T, H, I, E, k, x.dtype, x.device, chunks=2, logits=False)
    out = cf(x, gu, dn, logits=lg)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("T,H,I,E,k,groups,gather", [
    (1000, 256, 128, 16, 4, 2, True), (1000, 256, 128, 16, 4, 3, False), (300, 136, 40, 5, 2, 5, True),
    (513, 2048, 768, 128, 8, 2, True)])
def test_expert_groups_ffn_equals_one_stream(T, H, I, E, k, groups, gather):
    d = make_layer_inputs(T, H, I, E, k, "bf16", (982, T, E), w_std=0.08, wg_std=0.3)
    x, gu, dn, wg = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"])
    ref, _ = moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, gather=gather)
    ref = ref.clone()
    fg = moe.ExpertGroupsFfn(groups, device=x.device)
    bufs = None
    for _ in range(3):
        out, bufs = moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, gather=gather, ffn_groups=fg, bufs=bufs)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
