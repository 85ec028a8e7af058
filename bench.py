#!/usr/bin/env python3
"""Benchmark of the MoE expert layer on one MI355X.

One step = one pass of the whole layer over one batch of synthetic tokens already resident in HBM,
each stage a call into libmoe_rocm.so on the current stream:
  forward:  router logits -> top-k/renormalise -> permute -> grouped GEMM + SwiGLU -> grouped GEMM
            -> unpermute/combine (+ the shared expert, run as a one-segment grouped FFN, when the
            workload has one);
  backward (workloads with a backward pass): combine-bwd -> grouped FFN bwd (+ shared expert) ->
            top-k bwd -> router-logits bwd -> permute-bwd.

Prints ONE JSON line. `value` is tokens/s of the layer. The timed region is bracketed by
torch.cuda.synchronize(). An eager pass with HIP events recorded on the launch stream between the
calls gives each stage's duration, from which the roofline of the dominant kernel (the gate_up
grouped GEMM) is computed; the timed step is then the same one-stream sequence captured once in a
HIP graph and replayed (--no-graph: the eager pass is the timed step). Every timed region follows
its own untimed warm-up (by default about one second of steps: from idle, the clocks take that long
to settle at the board's power limit). The CPU baseline is the oracle (C, fp64, OpenMP) timed on a
bounded sample of the same tokens. --copy-calibration runs one 512 MiB device-to-device copy first,
the known-size kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters into HBM bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
WARMUP_SECONDS = 1.0         # default warm-up length (see --warmup)
METRIC = "MoE layer tokens/s at 1 GPU; grouped-GEMM MFMA util %; permute/combine HBM GB/s"
KERNEL_SOURCES = ["mixture_experts_layer_renorm_amd/csrc/grouped_gemm.hip",
                  "mixture_experts_layer_renorm_amd/csrc/common.hpp"]   # the dominant kernel's sources


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, rows: str):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter runs, if they
    were taken on the current kernel source with the same source of its rows; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_gemm_gate_up_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or d.get("gemm1_rows", "x_perm") != rows:
        return None
    return d.get("hbm_bytes_per_launch")


def dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(wl, d, budget_s: float):
    """Tokens/s of the oracle over the first tokens of the workload, in chunks of 32 tokens, until
    the budget is used: router logits, top-k, then the per-token layer."""
    import oracle
    chunk = 32
    done = 0
    t0 = time.perf_counter()
    while done < wl.T and time.perf_counter() - t0 < budget_s:
        sel = np.arange(done, min(wl.T, done + chunk))
        xs = d["x"][sel]
        logits = d["logits"][sel] if "logits" in d else oracle.router_logits(xs, d["w_gate"])
        idx, w = oracle.router_topk(logits, wl.k, True)
        oracle.moe_forward_tokens(xs, idx, w, d["gate_up"], d["down"], d.get("shared_gate_up"),
                                  d.get("shared_down"))
        done += len(sel)
    el = time.perf_counter() - t0
    return done, el


def _oracle_rate_ep(wl, d, budget_s: float):
    """Tokens/s of the oracle on one expert-parallel rank's share: each source token's k rows through
    their experts' FFN, then the weighted combine, 32 source tokens at a time."""
    import oracle
    counts = d["counts"]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ntok = wl.ep_rows // wl.k
    done = 0
    t0 = time.perf_counter()
    while done < ntok and time.perf_counter() - t0 < budget_s:
        toks = np.arange(done, min(ntok, done + 32))
        rows = d["row_of_slot"][(toks[:, None] * wl.k + np.arange(wl.k)[None, :]).reshape(-1)].astype(np.int64)
        y = oracle.expert_rows(d["x_perm"], offsets, d["gate_up"], d["down"], rows=rows).astype(np.float32)
        ros = np.arange(rows.shape[0], dtype=np.int32)
        oracle.combine(y, ros, d["topk_w"][toks])
        done += len(toks)
    return done, time.perf_counter() - t0


def cpu_baseline(wl, d, budget_s: float):
    """The oracle as it stands, on a bounded sample of the workload: half the budget on all host
    threads, half on one thread."""
    import oracle
    rate = _oracle_rate_ep if wl.ep_rows else _oracle_rate
    unit_tokens = wl.ep_rows // wl.k if wl.ep_rows else wl.T
    cores = oracle.max_threads()
    done, el = rate(wl, d, budget_s / 2)
    oracle.set_threads(1)
    try:
        done1, el1 = rate(wl, d, budget_s / 2)
    finally:
        oracle.set_threads(cores)
    what = ("k expert rows per source token through their SwiGLU experts + combine, fp64" if wl.ep_rows else
            "router logits + top-k + per-token SwiGLU experts + combine, fp64"
            f"{', forward only' if wl.backward else ''}")
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {done} of {unit_tokens} tokens of {wl.name} ({what}), {el:.1f} s on {cores} threads",
            "one_core": {"value": round(done1 / el1, 2), "unit": "tokens/s", "cores": 1,
                         "sample": f"first {done1} tokens, {el1:.1f} s on 1 thread"},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def tile_schedule(counts, N_cols, bm=320, bm_min=256, bn=256, xcds=8, cus=256, sort_max_e=256):
    """The persistent forward GEMMs' tile list and walk as the kernel derives them on the device: an
    expert with c rows gets n = ceil(c / hm) row tiles of near-equal height (none when c = 0), each
    with ceil(N_cols / bn) column tiles; hm = bm, or (one expert) bm_min when that list differs, takes
    as many rounds, and either only it splits into whole rounds on every XCD or there are two or more.
    With whole rounds on every XCD (or more
    than four rounds on average) XCD x takes the contiguous eighth of the list in expert order;
    otherwise ("balance") the experts are listed tallest first (ties by index, up to sort_max_e
    experts) and row tile R goes to XCD R mod 8. Each XCD deals its tiles to its cus / 8 workgroups
    in rounds, back and forth. Returns per-expert tile counts, per-XCD tile counts and row-tile work
    (rows x columns), the most tiles any workgroup runs, and whether the walk balanced."""
    ntn = (N_cols + bn - 1) // bn
    G = max(8, cus // 8 * 8)
    nbx = G // xcds

    def row_tiles_at(h):
        return [(c + h - 1) // h if c > 0 else 0 for c in counts]

    def whole_rounds(RT):
        return RT % xcds == 0 and (RT // xcds * ntn) % nbx == 0

    def rounds(RT):
        return (RT * ntn + G - 1) // G

    rx, rb = sum(row_tiles_at(bm)), sum(row_tiles_at(bm_min))
    hm = bm_min if (len(counts) == 1 and rb != rx and rounds(rb) == rounds(rx) and
                    ((whole_rounds(rb) and not whole_rounds(rx)) or rounds(rx) >= 2)) else bm
    rt = row_tiles_at(hm)
    height = [(c + r - 1) // r if r > 0 else 0 for c, r in zip(counts, rt)]
    RT = sum(rt)
    total = RT * ntn
    whole = whole_rounds(RT)
    balance = not whole and total <= 4 * G
    order = (sorted(range(len(counts)), key=lambda e: (-height[e], e))
             if balance and len(counts) <= sort_max_e else list(range(len(counts))))
    row_tiles = []
    for e in order:
        c = counts[e]
        for j in range(rt[e]):
            row_tiles.append((j + 1) * c // rt[e] - j * c // rt[e])
    tiles = [rows for rows in row_tiles for _ in range(ntn)]
    per_xcd = [0] * xcds
    work = [0] * xcds
    Q = (total + xcds - 1) // xcds
    for L, rows in enumerate(tiles):
        x = (L // ntn) % xcds if balance else L // Q
        per_xcd[x] += 1
        work[x] += rows * N_cols
    mean_w = sum(work) / xcds if xcds else 0
    return {"tiles": total, "tiles_per_expert": [int(r * ntn) for r in rt],
            "empty_experts": int(sum(1 for c in counts if c == 0)),
            "tiles_of_empty_experts": int(sum(r * ntn for r, c in zip(rt, counts) if c == 0)),
            "tiles_per_xcd": per_xcd, "xcd_work_max_over_mean": round(max(work) / mean_w, 4) if mean_w else None,
            "workgroup_tiles_max": max((n + nbx - 1) // nbx for n in per_xcd), "balanced_walk": balance,
            "tile_rows_max": hm}


def pct(a, q):
    return round(float(np.percentile(np.asarray(a), q)), 4)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before each timed region (default: as many as fill about "
                         f"{WARMUP_SECONDS:g} s; from idle the clocks take that long to settle at the board's power "
                         "limit, and a shorter warm-up times the ramp rather than the layer)")
    ap.add_argument("--workload", default="qwen3_moe",
                    choices=["qwen3_moe", "long_seq", "tiny_f32", "fine_grained", "ep_rank_zipf"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline budget (0 = skip)")
    ap.add_argument("--ffn-groups", type=int, default=1,
                    help="forward only: the routed FFN as this many expert groups on their own streams in the timed "
                         "step (1 = one stream); per-kernel figures come from a one-stream pass")
    ap.add_argument("--chunks", type=int, default=1,
                    help="forward only: split the tokens in N chunks and route chunk c+1 on a side stream while "
                         "chunk c's experts run (Domino-style overlap); the step time is the chunked one")
    ap.add_argument("--bwd-wgrad-cus", type=int, default=0,
                    help="backward workloads: time the step with the backward on three streams and the weight "
                         "gradients capped to this many CUs (0 = one stream); per-kernel figures come from a "
                         "one-stream pass")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time the step as eager launches; by default the one-stream step is captured once in a HIP "
                         "graph and the timed steps are its replays (the same kernels on the same buffers, without "
                         "per-launch host overhead); the per-kernel figures always come from the eager pass")
    ap.add_argument("--no-gather", action="store_true",
                    help="forward: copy the rows to x_perm in the permute instead of gathering them in GEMM-1")
    ap.add_argument("--separate-routing", action="store_true",
                    help="forward: moe_router_topk then moe_permute as two calls instead of moe_router_topk_permute")
    ap.add_argument("--no-mall-cold", dest="mall_cold", action="store_false",
                    help="skip the per-kernel pass with a 512 MiB read before every call (last-level cache cold)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 512 MiB device copy before the warm-up (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              "(the layer's multi-GPU sharding is a design note, not code)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_renorm_amd as moe
    from inputs.workloads import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moe.load_library()
    wl = WORKLOADS[args.workload]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    N = wl.N
    t_gen = time.perf_counter()
    d = workload_inputs(wl.name)
    print(f"[bench] {wl.name}: inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    ep = wl.ep_rows > 0
    if ep:   # one expert-parallel rank's share: the rows arrive grouped; T = source tokens
        T = wl.ep_rows // k
        x = dev(d["x_perm"], torch)
    else:
        x = dev(d["x"], torch)
    gate_up = dev(d["gate_up"], torch)
    down = dev(d["down"], torch)
    w_gate = dev(d["w_gate"], torch) if "w_gate" in d else None
    given_logits = dev(d["logits"], torch) if "logits" in d else None
    sh_gu = dev(d["shared_gate_up"], torch) if "shared_gate_up" in d else None
    sh_dn = dev(d["shared_down"], torch) if "shared_down" in d else None
    d_out = dev(d["d_out"], torch) if "d_out" in d else None
    tdt = x.dtype
    I_sh = 0 if sh_gu is None else sh_gu.shape[1] // 2
    # forward-only workloads fold the row copy of the permute into the first grouped matmul (it
    # gathers its rows from x); a training step keeps x_perm, which the weight gradients read
    gather = not wl.backward and not args.no_gather and not ep
    fused_routing = not args.separate_routing
    bufs = moe.LayerBuffers(T, H, I, E, k, tdt, x.device, logits=given_logits is None and w_gate is not None,
                            gu_saved=wl.backward, I_shared=I_sh, x_perm=not gather and not ep)
    if ep:   # the exchange's layout handle, handed straight to the FFN and the combine
        counts_np = d["counts"].astype(np.int32)
        bufs.x_perm = x
        bufs.plan.counts.copy_(torch.from_numpy(counts_np))
        bufs.plan.offsets.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(counts_np)]).astype(np.int32)))
        bufs.plan.row_of_slot.copy_(torch.from_numpy(d["row_of_slot"].astype(np.int32)))
        bufs.topk_w.copy_(torch.from_numpy(d["topk_w"].astype(np.float32)))
    grads = moe.LayerGrads(T, H, I, E, k, tdt, x.device, I_shared=I_sh, router=w_gate is not None) if wl.backward else None
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=x.device).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the stages of one step, in order; HIP events go between them
    sh = bufs.shared
    stages = []
    if given_logits is None and w_gate is not None:
        stages.append(("router_logits", lambda: moe.moe_router_logits(x, w_gate, bufs.logits)))
    logits = bufs.logits if given_logits is None else given_logits
    if ep:
        pass
    elif fused_routing:
        stages.append(("router_topk_permute", lambda: moe.moe_router_topk_permute(
            logits, k, x, E, True, bufs.topk_idx, bufs.topk_w, bufs.x_perm, bufs.plan, bufs.workspace,
            rows=not gather)))
    else:
        stages.append(("router_topk", lambda: moe.moe_router_topk(logits, k, True, bufs.topk_idx, bufs.topk_w)))
        stages.append(("permute", lambda: moe.moe_permute(x, bufs.topk_idx, E, bufs.x_perm, bufs.plan,
                                                          bufs.workspace, rows=not gather)))
    if gather:
        stages.append(("gemm_gate_up", lambda: moe.moe_grouped_gemm_swiglu_gather(
            x, bufs.plan.slot_of_row, k, gate_up, bufs.plan.offsets, None, bufs.h, bufs.gu_saved)))
    else:
        stages.append(("gemm_gate_up", lambda: moe.moe_grouped_gemm_swiglu(bufs.x_perm, gate_up, bufs.plan.offsets,
                                                                           bufs.h, bufs.gu_saved)))
    stages.append(("gemm_down", lambda: moe.moe_grouped_gemm_down(bufs.h, down, bufs.plan.offsets, bufs.y)))
    if sh is not None:
        stages.append(("shared_ffn", lambda: moe.moe_grouped_swiglu_ffn(x, sh_gu, sh_dn, sh["offsets"], sh["h"], sh["y"],
                                                                         sh["gu_saved"])))
    stages.append(("combine", lambda: moe.moe_unpermute_combine(bufs.y, bufs.plan.row_of_slot, bufs.topk_w,
                                                                None if sh is None else sh["y"], bufs.out)))
    if grads is not None:
        g = grads
        stages += [
            ("combine_bwd", lambda: moe.moe_unpermute_combine_bwd(d_out, bufs.y, bufs.plan.row_of_slot, bufs.topk_w,
                                                                  g.d_y, g.d_w)),
            ("ffn_bwd", lambda: moe.moe_grouped_swiglu_ffn_bwd(g.d_y, bufs.x_perm, bufs.gu_saved, bufs.h, gate_up, down,
                                                               bufs.plan.offsets, g.d_x_perm, g.d_gate_up, g.d_down,
                                                               g.d_gu)),
        ]
        if sh is not None:
            stages.append(("shared_ffn_bwd", lambda: moe.moe_grouped_swiglu_ffn_bwd(
                d_out, x, sh["gu_saved"], sh["h"], sh_gu, sh_dn, sh["offsets"], g.d_x_side, g.d_shared_gate_up,
                g.d_shared_down, g.d_shared_gu)))
        stages.append(("router_topk_bwd", lambda: moe.moe_router_topk_bwd(logits, bufs.topk_idx, bufs.topk_w, g.d_w, True,
                                                                          g.d_logits)))
        # (the buffers are bound when each stage is defined: `side` changes below)
        side = g.d_x_side if sh is not None else None
        if w_gate is not None:
            dst = g.d_x_side2 if sh is not None else g.d_x_side
            stages.append(("router_logits_bwd", lambda d_in=side, d_out_=dst: moe.moe_router_logits_bwd(
                x, w_gate, g.d_logits, g.d_w_gate, d_x_in=d_in, d_x=d_out_)))
            side = dst
        stages.append(("permute_bwd", lambda d_add=side: moe.moe_permute_bwd(g.d_x_perm, bufs.plan.row_of_slot, T, k,
                                                                             d_x_add=d_add, d_x=g.d_x)))
    names = [n for n, _ in stages]
    ns = len(stages)

    def step(evs=None):
        for i, (_, fn) in enumerate(stages):
            if evs is not None:
                evs[i].record(stream)
            fn()
        if evs is not None:
            evs[ns].record(stream)

    done = 0
    if args.warmup is None:
        # after a first step (module loading, first-touch), three steps give the step time from which
        # the default warm-up length follows; all four are part of the warm-up
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        per_step = (time.perf_counter() - t0) / 3
        args.warmup = max(5, int(np.ceil(WARMUP_SECONDS / per_step)))
        done = 4
    for _ in range(args.warmup - done):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.zeros(ns)
    total_ev = 0.0
    for evs in events:
        for i in range(ns):
            seg[i] += evs[i].elapsed_time(evs[i + 1])
        total_ev += evs[0].elapsed_time(evs[ns])
    seg /= args.steps
    ms_per_step = max(wall * 1e3 / args.steps, total_ev / args.steps)
    step_ms = [evs[0].elapsed_time(evs[ns]) for evs in events]
    seg_med = [float(np.median([evs[i].elapsed_time(evs[i + 1]) for evs in events])) for i in range(ns)]
    cold_us = None
    if args.mall_cold:
        # every call after a read of 512 MiB (twice the last-level cache), so that its inputs come
        # from HBM; a read leaves no dirty lines whose write-back would be charged to the call. The
        # same stages in the same order, timed one by one.
        flush = torch.ones(128 << 20, dtype=torch.float32, device=x.device)
        flush_sum = torch.empty((), dtype=torch.float32, device=x.device)
        cold = np.zeros(ns)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * ns)] for _ in range(args.steps)]
        for s_ in range(args.steps):
            for i, (_, fn) in enumerate(stages):
                torch.sum(flush, dim=0, out=flush_sum)
                cev[s_][2 * i].record(stream)
                fn()
                cev[s_][2 * i + 1].record(stream)
        torch.cuda.synchronize()
        for evs in cev:
            for i in range(ns):
                cold[i] += evs[2 * i].elapsed_time(evs[2 * i + 1])
        cold_us = {n: round(cold[i] / args.steps * 1e3, 2) for i, (n, _) in enumerate(stages)}
        del flush, flush_sum
    one_stream_ms = ms_per_step
    step_us = None
    ffn_groups = max(1, args.ffn_groups)
    if wl.backward or sh is not None:
        ffn_groups = 1
    st2 = None
    if ffn_groups > 1 and args.chunks == 1:
        # the timed step: the same stages, with the routed FFN as expert groups on their own streams
        fgs = moe.ExpertGroupsFfn(ffn_groups, device=x.device)
        ffn = lambda: fgs(gate_up, down, bufs.plan.offsets, bufs.h, bufs.y, x_perm=bufs.x_perm,
                          x=x if gather else None, slot_of_row=bufs.plan.slot_of_row, k=k)
        st2 = [(n, f) for n, f in stages if n not in ("gemm_gate_up", "gemm_down")]
        pos = [n for n, _ in stages].index("gemm_gate_up")
        st2.insert(pos, ("ffn_expert_groups", ffn))
    if wl.backward and args.bwd_wgrad_cus > 0:
        # the timed step: the same forward, then the backward with its independent products on three
        # streams (weight gradients capped to --bwd-wgrad-cus CUs)
        ob = moe.OverlappedBackward(device=x.device, wgrad_cus=args.bwd_wgrad_cus)
        bwd = lambda: ob(d_out, x, gate_up, down, bufs, w_gate=w_gate, logits=given_logits, renorm=True,
                         shared_gate_up=sh_gu, shared_down=sh_dn, grads=grads)
        bwd_names = ("combine_bwd", "ffn_bwd", "shared_ffn_bwd", "router_topk_bwd", "router_logits_bwd", "permute_bwd")
        st2 = [(n, f) for n, f in stages if n not in bwd_names] + [("backward_overlapped", bwd)]
    if st2 is not None:
        n2 = len(st2)

        def step2(evs=None):
            for i, (_, fn) in enumerate(st2):
                if evs is not None:
                    evs[i].record(stream)
                fn()
            if evs is not None:
                evs[n2].record(stream)

        for _ in range(args.warmup):
            step2()
        torch.cuda.synchronize()
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(n2 + 1)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            step2(ev2[s_])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        seg2 = np.zeros(n2)
        tot2 = 0.0
        for evs in ev2:
            for i in range(n2):
                seg2[i] += evs[i].elapsed_time(evs[i + 1])
            tot2 += evs[0].elapsed_time(evs[n2])
        seg2 /= args.steps
        ms_per_step = max(wall * 1e3 / args.steps, tot2 / args.steps)
        step_us = {n: round(seg2[i] * 1e3, 2) for i, (n, _) in enumerate(st2)}
    graph_ms = None
    use_graph = args.graph and st2 is None and args.chunks == 1   # multi-stream schedules run eagerly
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        cap_side = torch.cuda.Stream()      # default priority
        cap_side.wait_stream(stream)
        with torch.cuda.stream(cap_side):
            step()
        stream.wait_stream(cap_side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        # the timed region: K replays back to back, nothing else on the stream
        t0 = time.perf_counter()
        for i in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        # then K more with an event before every replay and after the last: the per-step
        # distribution (each event is a small command of its own between two replays)
        rev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        for i in range(args.steps):
            rev[i].record(stream)
            graph.replay()
        rev[args.steps].record(stream)
        torch.cuda.synchronize()
        step_ms = [rev[i].elapsed_time(rev[i + 1]) for i in range(args.steps)]
        ms_per_step = graph_ms
    unchunked_ms = ms_per_step
    if args.chunks > 1:
        # the timed step is the chunked, two-stream forward; the per-kernel figures above (and the
        # roofline of the dominant kernel) come from the one-shot stages
        if wl.backward or sh is not None:
            print("bench.py: --chunks applies to forward-only workloads without a shared expert", file=sys.stderr)
            sys.exit(2)
        cf = moe.ChunkedForward(T, H, I, E, k, tdt, x.device, chunks=args.chunks, logits=given_logits is None,
                                gather=gather)
        run = lambda: cf(x, gate_up, down, w_gate=w_gate, logits=given_logits)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            run()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = max(wall * 1e3 / args.steps, ev0.elapsed_time(ev1) / args.steps)
    tokens_per_s = T / (ms_per_step / 1e3)
    t_of = {n: seg[i] * 1e-3 for i, n in enumerate(names)}

    counts = bufs.plan.counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    route_name = "router_topk_permute" if "router_topk_permute" in t_of else ("permute" if "permute" in t_of else None)
    b = 2 if tdt == torch.bfloat16 else 4
    # algorithmic work of each call (what the method must read, write and compute)
    gu_flops = 2.0 * N * H * 2 * I
    # the gathering GEMM reads each token's row of x (once, algorithmically) instead of x_perm
    gu_bytes = n_active * H * 2 * I * b + (T if gather else N) * H * b + N * I * b
    dn_flops = 2.0 * N * I * H
    dn_bytes = n_active * I * H * b + N * I * b + N * H * b
    perm_bytes = (0 if gather else T * H * b + N * H * b) + T * k * 4 * 3 + E * 4 * 2
    if route_name == "router_topk_permute":
        perm_bytes += T * E * 4 + T * k * 8          # the top-k reads the logits, writes indices and weights
    comb_bytes = N * H * b + T * H * b + T * k * 8
    t_gu, t_dn = t_of["gemm_gate_up"], t_of["gemm_down"]
    peak_tf = PEAK_BF16_TFLOPS if tdt == torch.bfloat16 else PEAK_F32_TFLOPS
    ridge = peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    if gu_flops / gu_bytes < ridge:
        roof = {"bound": "hbm", "achieved": round(gu_bytes / t_gu / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(gu_flops / t_gu / 1e12, 1), "peak": peak_tf, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = load_traffic(wl.name, "gathered" if gather else "x_perm")
    if tdt == torch.bfloat16 and H % 8 == 0 and I % 8 == 0:
        kf = "true" if H % 128 == 0 else "false"   # K = H a multiple of four K steps
        roof["kernel"] = f"grouped_gemm_fwd_kernel<0, {'true' if gather else 'false'}, {kf}, false> (gate_up + SwiGLU)"
    else:
        roof["kernel"] = "gen_ffn1_kernel (gate_up + SwiGLU, generic path)"
    roof["algorithmic_bytes"] = gu_bytes
    roof["algorithmic_flops"] = gu_flops
    roof["avg_launch_us"] = round(t_gu * 1e6, 2)

    breakdown = {n: round(seg[i] * 1e3, 2) for i, n in enumerate(names)}
    perf = {
        "kernel_us": breakdown,
        "grouped_gemm_mfma_util_pct": round(100 * (gu_flops + dn_flops) / (t_gu + t_dn) / (peak_tf * 1e12), 2),
        "gemm_gate_up_tflops": round(gu_flops / t_gu / 1e12, 1),
        "gemm_down_tflops": round(dn_flops / t_dn / 1e12, 1),
        "gemm_gate_up_hbm_gbs": round(gu_bytes / t_gu / 1e9, 1),
        "gemm_down_hbm_gbs": round(dn_bytes / t_dn / 1e9, 1),
        "combine_hbm_gbs": round(comb_bytes / t_of["combine"] / 1e9, 1),
        "active_experts": n_active,
        "step_ms_median": pct(step_ms, 50), "step_ms_p10": pct(step_ms, 10), "step_ms_p90": pct(step_ms, 90),
        "kernel_us_median": {n: round(seg_med[i] * 1e3, 2) for i, n in enumerate(names)},
        "tile_schedule_gate_up": tile_schedule([int(c) for c in counts], 2 * I),
        "tile_schedule_down": tile_schedule([int(c) for c in counts], H),
    }
    if route_name is not None:
        perf[f"{route_name}_hbm_gbs"] = round(perm_bytes / t_of[route_name] / 1e9, 1)
    if cold_us is not None:
        perf["kernel_us_mall_cold"] = cold_us
        perf["combine_hbm_gbs_mall_cold"] = round(comb_bytes / (cold_us["combine"] * 1e-6) / 1e9, 1)
        perf["gemm_gate_up_hbm_gbs_mall_cold"] = round(gu_bytes / (cold_us["gemm_gate_up"] * 1e-6) / 1e9, 1)
        perf["gemm_down_hbm_gbs_mall_cold"] = round(dn_bytes / (cold_us["gemm_down"] * 1e-6) / 1e9, 1)
        if route_name is not None:
            perf[f"{route_name}_hbm_gbs_mall_cold"] = round(perm_bytes / (cold_us[route_name] * 1e-6) / 1e9, 1)
    if args.chunks > 1:
        perf["one_shot_ms_per_step"] = round(unchunked_ms, 4)
    if step_us is not None:
        perf["timed_step_us"] = step_us
        perf["one_stream_ms_per_step"] = round(one_stream_ms, 4)
    if graph_ms is not None:
        perf["eager_ms_per_step"] = round(one_stream_ms, 4)
    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if tdt == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": H, "I": I, "E": E, "k": k, "renorm": True,
                   "router": ("none: rows arrive grouped by expert" if ep else
                              "logits given" if given_logits is not None else "x @ W_g"),
                   "routing_call": (None if ep else "moe_router_topk_permute" if fused_routing else
                                    "moe_router_topk + moe_permute"),
                   "shared_experts": wl.shared, "pass": "forward+backward" if wl.backward else "forward",
                   "gemm1_rows": "gathered from x" if gather else "x_perm", "chunks": args.chunks,
                   "rows": N,
                   "ffn_expert_groups": ffn_groups if args.chunks == 1 else 1,
                   "backward_wgrad_cus": args.bwd_wgrad_cus if wl.backward else None,
                   "hip_graph": use_graph},
        "roofline": roof, "perf": perf,
    }
    if args.cpu_seconds > 0:
        print(f"[bench] timing the oracle on the CPU for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, d, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
