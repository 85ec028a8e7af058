"""GPU parity at the workloads' full sizes, through the same calls and launch configuration that the
benchmark times. Integer results (logits bits, expert indices, the permute plan, permuted rows)
are compared in full; floating-point outputs on seeded samples of tokens, grouped rows and
weight-gradient units, each of which the oracle computes on its own. Tolerances as everywhere:
max|gpu - ref| / max|ref| <= 1e-2 (bf16), <= 1e-5 (fp32)."""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
import oracle
from inputs import WORKLOADS, workload_inputs
from inputs.generators import generator
from tests.gpu_util import TOL, as64, dev, host, rel_err

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def sample(n, count, key):
    """Sorted distinct indices in [0, n): the first, the last and count-2 seeded others."""
    pick = generator(key).choice(n, size=min(n, count), replace=False)
    return np.unique(np.concatenate([[0, n - 1], pick])).astype(np.int64)


def slots_rows(ros, tokens, k):
    return ros[(tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)].astype(np.int64)


def check_routing_and_plan(bufs, x, k, E, w_gate=None, logits=None):
    """Full bit-exact check of logits (when computed), indices, plan and permuted rows; returns the
    oracle's routing and plan for the sampled float checks."""
    if logits is None:
        logits = oracle.router_logits(x, w_gate)
        assert np.array_equal(host(bufs.logits).view(np.uint32), logits.view(np.uint32)), "router logits"
    idx, w = oracle.router_topk(logits, k)
    assert np.array_equal(host(bufs.topk_idx), idx), "top-k indices"
    assert rel_err(host(bufs.topk_w), w) <= TOL["f32"], "top-k weights"
    counts, offsets, ros, sor = oracle.permute_plan(idx, E)
    assert np.array_equal(host(bufs.plan.counts), counts)
    assert np.array_equal(host(bufs.plan.offsets), offsets)
    assert np.array_equal(host(bufs.plan.row_of_slot), ros)
    assert np.array_equal(host(bufs.plan.slot_of_row), sor)
    xp = oracle.permute_rows(x, sor, k)
    if bufs.x_perm is not None:
        assert np.array_equal(host(bufs.x_perm), xp), "permuted rows"
    return logits, idx, w, offsets, ros, xp


def release():
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,gather", [("qwen3_moe", False), ("qwen3_moe", True), ("long_seq", False),
                                         ("long_seq", True)])
def test_layer_forward_full(name, gather):
    """gather=True is the benchmark's step: plan-only permute, the gate_up GEMM gathering its rows
    from x through slot_of_row (x_perm is never written)."""
    wl = WORKLOADS[name]
    d = workload_inputs(name)
    x, gu, dn = dev(d["x"]), dev(d["gate_up"]), dev(d["down"])
    if wl.logits_std is None:
        out, bufs = moe.moe_layer_forward(x, gu, dn, wl.k, w_gate=dev(d["w_gate"]), gather=gather)
    else:
        out, bufs = moe.moe_layer_forward(x, gu, dn, wl.k, logits=dev(d["logits"]), gather=gather)
    torch.cuda.synchronize()
    _, idx, w, offsets, ros, xp = check_routing_and_plan(bufs, d["x"], wl.k, wl.E, d.get("w_gate"), d.get("logits"))
    toks = sample(wl.T, 48, (990, wl.code))
    ref = oracle.moe_forward_tokens(d["x"], idx, w, d["gate_up"], d["down"], tokens=toks)
    assert rel_err(host(out)[toks], ref) <= TOL["bf16"], "layer output"
    rows = slots_rows(ros, toks, wl.k)
    ry, ra = oracle.expert_rows(xp, offsets, d["gate_up"], d["down"], rows=rows, want_act=True)
    assert rel_err(host(bufs.h)[rows], ra) <= TOL["bf16"], "SwiGLU activations"
    assert rel_err(host(bufs.y)[rows], ry) <= TOL["bf16"], "expert outputs"
    del out, bufs, x, gu, dn
    release()


def test_ep_rank_share_full():
    wl = WORKLOADS["ep_rank_zipf"]
    d = workload_inputs("ep_rank_zipf")
    counts = d["counts"]
    assert (counts == 0).sum() >= 2 and counts.sum() == wl.ep_rows
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xp = d["x_perm"]
    y, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(d["gate_up"]), dev(d["down"]), dev(offsets))
    out = moe.moe_unpermute_combine(y, dev(d["row_of_slot"]), dev(d["topk_w"]))
    torch.cuda.synchronize()
    # grouped rows: a seeded sample plus the first and last row of every non-empty expert
    edges = np.concatenate([offsets[:-1][counts > 0], offsets[1:][counts > 0] - 1])
    rows = np.unique(np.concatenate([sample(wl.ep_rows, 64, (991,)), edges])).astype(np.int64)
    ry, ra = oracle.expert_rows(xp, offsets, d["gate_up"], d["down"], rows=rows, want_act=True)
    assert rel_err(host(h)[rows], ra) <= TOL["bf16"]
    assert rel_err(host(y)[rows], ry) <= TOL["bf16"]
    # combine of sampled source tokens, from the oracle's own expert rows
    ntok = wl.ep_rows // wl.k
    toks = sample(ntok, 32, (992,))
    R = slots_rows(d["row_of_slot"], toks, wl.k)
    y_R = oracle.expert_rows(xp, offsets, d["gate_up"], d["down"], rows=R).astype(np.float32)
    ros_c = np.zeros(ntok * wl.k, np.int32)
    ros_c[(toks[:, None] * wl.k + np.arange(wl.k)[None, :]).reshape(-1)] = np.arange(R.shape[0], dtype=np.int32)
    ref = oracle.combine(y_R, ros_c, d["topk_w"], tokens=toks)
    assert rel_err(host(out)[toks], ref) <= TOL["bf16"]
    del y, h, out
    release()


def test_tiny_f32_full():
    wl = WORKLOADS["tiny_f32"]
    d = workload_inputs("tiny_f32")
    out, bufs = moe.moe_layer_forward(dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), wl.k, w_gate=dev(d["w_gate"]))
    ref, ridx, _, rlog = oracle.moe_forward(d["x"], d["gate_up"], d["down"], wl.k, w_gate=d["w_gate"])
    assert np.array_equal(host(bufs.logits).view(np.uint32), rlog.view(np.uint32))
    assert np.array_equal(host(bufs.topk_idx), ridx)
    assert rel_err(host(out), ref) <= TOL["f32"]


def test_fine_grained_forward_backward_full():
    wl = WORKLOADS["fine_grained"]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    d = workload_inputs("fine_grained")
    x, gu, dn, wg = dev(d["x"]), dev(d["gate_up"]), dev(d["down"]), dev(d["w_gate"])
    sgu, sdn, d_out = dev(d["shared_gate_up"]), dev(d["shared_down"]), dev(d["d_out"])
    out, bufs = moe.moe_layer_forward(x, gu, dn, k, w_gate=wg, shared_gate_up=sgu, shared_down=sdn,
                                      save_for_backward=True)
    g = moe.moe_layer_backward(d_out, x, gu, dn, bufs, w_gate=wg, shared_gate_up=sgu, shared_down=sdn)
    torch.cuda.synchronize()
    _, idx, w, offsets, ros, xp = check_routing_and_plan(bufs, d["x"], k, E, d["w_gate"])
    # forward, sampled tokens (routed experts + shared expert)
    toks = sample(T, 12, (993,))
    ref = oracle.moe_forward_tokens(d["x"], idx, w, d["gate_up"], d["down"], d["shared_gate_up"],
                                    d["shared_down"], tokens=toks)
    assert rel_err(host(out)[toks], ref) <= TOL["bf16"], "layer output"
    # backward, sampled tokens: d_x (routed + shared + router), d_logits, d_w
    rb = oracle.moe_backward_tokens(d["x"], d["gate_up"], d["down"], k, d["d_out"], toks, w_gate=d["w_gate"],
                                    shared_gate_up=d["shared_gate_up"], shared_down=d["shared_down"])
    assert rel_err(host(g.d_w)[toks], rb["d_w"]) <= TOL["bf16"], "d_w"
    assert rel_err(host(g.d_logits)[toks], rb["d_logits"]) <= TOL["bf16"], "d_logits"
    assert rel_err(host(g.d_x)[toks], rb["d_x"]) <= TOL["bf16"], "d_x"
    # weight gradients: sampled intermediate units of the busiest, the least busy and a seeded expert
    counts = np.diff(offsets)
    busy = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, counts.max() + 1))),
            int(generator((994,)).integers(E))]
    units = sample(I, 8, (995,))
    dgu, ddn = g.d_gate_up, g.d_down
    for e in busy:
        rg, ru, rd = oracle.moe_weight_grads_units(d["x"], d["gate_up"], d["down"], idx, w, d["d_out"], e, units)
        blk = host(dgu[e * H:(e + 1) * H])
        assert rel_err(blk[:, units], rg) <= TOL["bf16"], f"d_gate_up gate columns, expert {e}"
        assert rel_err(blk[:, I + units], ru) <= TOL["bf16"], f"d_gate_up up columns, expert {e}"
        assert rel_err(host(ddn[e * I:(e + 1) * I])[units], rd) <= TOL["bf16"], f"d_down rows, expert {e}"
    # shared expert: one segment of all T tokens with weight 1, so its d_y is d_out itself
    rg, ru, rd = oracle.expert_weight_grads_units(d["x"], d["d_out"], np.array([0, T], np.int32),
                                                  d["shared_gate_up"], d["shared_down"], 0, units)
    sblk = host(g.d_shared_gate_up)
    assert rel_err(sblk[:, units], rg) <= TOL["bf16"]
    assert rel_err(sblk[:, I + units], ru) <= TOL["bf16"]
    assert rel_err(host(g.d_shared_down)[units], rd) <= TOL["bf16"]
    # router weight gradient: column of the least busy expert (only its tokens contribute)
    e = busy[1]
    toks_e = np.nonzero((idx == e).any(axis=1))[0]
    rb_e = oracle.moe_backward_tokens(d["x"], d["gate_up"], d["down"], k, d["d_out"], toks_e, w_gate=d["w_gate"])
    dwg_ref, _ = oracle.router_logits_bwd(d["x"][toks_e], d["w_gate"], rb_e["d_logits"])
    assert rel_err(host(g.d_w_gate)[:, e], dwg_ref[:, e]) <= TOL["bf16"], "d_w_gate column"
    del out, bufs, g, x, gu, dn, wg, sgu, sdn, d_out, dgu, ddn
    release()
