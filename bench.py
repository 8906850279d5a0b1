"""Benchmark: one routed block-sparse attention layer per step on one MI355X.

A step is the whole hot path on one layer's Q/K/V already resident in HBM:
fva_route (block-mean pooling, pooled scores, softmax, sort, cumulative Top-p
count, Top-k floor, mask) followed by fva_sparse_attn (work costs, LPT order,
persistent block-sparse flash attention).  Prints one JSON line.

Inputs are seeded synthetic Q/K/V shaped like a Wan2.2 14B-like attention
layer (27280 = 31x22x40 tokens, 40 heads, head_dim 128, (4,8,8) blocks); no
model weights or real activations are used.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan14b")
    ap.add_argument("--sched", default="lpt", choices=["lpt", "naive", "xcd"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-items", type=int, default=160, help="work items in the CPU oracle sample")
    ap.add_argument("--no-dense", action="store_true", help="skip timing the dense reference")
    ap.add_argument("--overlap", type=int, default=0, metavar="G",
                    help="also measure the whole-layer call (fva_routed_attn) with groups = 1 and pipelined over "
                         "G head groups, on one stream and alternating between two streams")
    ap.add_argument("--sasa", type=int, default=0, metavar="R",
                    help="also measure slack-aware augmentation with R rounds on the per-XCD schedule, with its "
                         "error against the dense oracle on sampled items")
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer captured once in a HIP graph and replayed (outputs checked bitwise "
                         "against the eager loop)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 2 GiB device-to-device three times (reference for rocprofv3 FETCH/WRITE_SIZE)")
    ap.add_argument("--calibrate-gemm", action="store_true",
                    help="only time torch's bf16 GEMM (n = 8192 and 16384), a reference for what the bf16 MFMA "
                         "peak yields to a library kernel on this part")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (across GPUs it would shard the "
              "heads). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = 2 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_per_launch": n}))
        return
    if args.calibrate_gemm:
        for n, reps in ((8192, 20), (16384, 5)):
            a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
            b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
            for _ in range(3):
                c = a @ b
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            print(json.dumps({"calibrate_gemm_n": n, "dtype": "bf16", "ms": round(ms, 3), "tflops": round(tf, 1),
                              "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 3)}), flush=True)
            del a, b, c
        return

    import adaptive_block_sparse_tile_amd as fva
    import fvgen

    wl = fvgen.WORKLOADS[args.workload]
    t0 = time.time()
    host = fvgen.generate_qkv(wl, seed=args.seed)
    gen_s = time.time() - t0
    dev = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in host]
    q, k, v = dev
    shape = tuple(q.shape)
    B, L, heads, D = shape
    N = fva.num_blocks(wl.grid, wl.block)
    words = (N + 31) // 32
    mask = torch.empty((B, heads, N, words), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, heads, N), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    ws_r = fva.workspace(fva.route_workspace_bytes(shape, wl.grid, wl.block), q.device)
    ws_a = fva.workspace(fva.attn_workspace_bytes(shape, wl.grid, wl.block), q.device)
    stream = torch.cuda.current_stream()

    def make_mask():
        # the router, or for a static-mask workload the local + anchor block mask
        if wl.static:
            fva.static_mask(shape, wl.grid, wl.block, local=wl.static[0], anchor_t=wl.static[1], out=(mask, cnt),
                            stream=stream)
        else:
            fva.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r, out=(mask, cnt, status), stream=stream)

    def step():
        # one layer: the mask, then the sparse attention call (plan + attention kernel)
        make_mask()
        fva.attn_plan(k, v, wl.grid, wl.block, mask, sched=args.sched, ws=ws_a, stream=stream)
        fva.attn_exec(q, wl.grid, wl.block, mask, ws_a, sched=args.sched, out=o, stream=stream)

    print("[bench] workload %s: generated inputs in %.1fs; warmup %d" % (wl.name, gen_s, args.warmup),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, plus per-stage events on the launching stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        ev[s][0].record(stream)
        make_mask()
        ev[s][1].record(stream)
        fva.attn_plan(k, v, wl.grid, wl.block, mask, sched=args.sched, ws=ws_a, stream=stream)
        ev[s][2].record(stream)
        fva.attn_exec(q, wl.grid, wl.block, mask, ws_a, sched=args.sched, out=o, stream=stream)
        ev[s][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    per_stage = {"mask" if wl.static else "route": [e[0].elapsed_time(e[1]) for e in ev],
                 "plan": [e[1].elapsed_time(e[2]) for e in ev],
                 "kernel": [e[2].elapsed_time(e[3]) for e in ev],
                 "layer": [e[0].elapsed_time(e[3]) for e in ev]}
    stages = {name: {"mean": round(float(np.mean(x)), 4), "median": round(float(np.median(x)), 4),
                     "min": round(float(np.min(x)), 4)} for name, x in per_stage.items()}
    route_ms = float(np.median(per_stage["mask" if wl.static else "route"]))
    plan_ms = float(np.mean(per_stage["plan"]))
    kern_ms = float(np.mean(per_stage["kernel"]))   # the roofline uses the mean launch duration
    attn_ms = plan_ms + kern_ms
    print("[bench] timed %d steps: %.3f ms/step (route %.3f ms, attention plan %.3f ms, attention kernel %.3f ms)"
          % (args.steps, ms_step, route_ms, plan_ms, kern_ms), file=sys.stderr, flush=True)

    # algorithmic work of the routed mask (real token pairs)
    mask_h = mask.cpu().numpy().view(np.uint32)
    cnt_h = cnt.cpu().numpy()
    counts = _block_counts(wl)
    kept = ((mask_h[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(B, heads, N, -1)[..., :N]
    kv_tok = (kept * counts[None, None, None, :]).sum(-1)
    pairs = int((kv_tok * counts[None, None, :]).sum())
    eff_flop = 4.0 * D * pairs
    dense_flop = 4.0 * D * float(L) * L * heads * B
    eff_tflops = eff_flop / (ms_step * 1e-3) / 1e12
    kern_tflops = eff_flop / (kern_ms * 1e-3) / 1e12
    frac_per_head = cnt_h.mean(axis=(0, 2)) / N

    # route stage bytes: Q and K read once by the pooling kernel
    route_bytes = 2.0 * B * L * heads * D * 2

    # dense reference (same MFMA core over all tokens), for the speedup
    dense_ms = None
    if not args.no_dense:
        od = torch.empty_like(q)
        ws_d = fva.workspace(fva.dense_workspace_bytes(shape), q.device)
        for _ in range(2):
            fva.dense_attn_ref(q, k, v, out=od, ws=ws_d, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nd = max(3, args.steps // 4)
        e0.record(stream)
        for _ in range(nd):
            fva.dense_attn_ref(q, k, v, out=od, ws=ws_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / nd
        del ws_d

    # CU imbalance of the persistent kernel (separate, untimed run with a trace)
    nwg = fva.attn_workgroups(shape, wl.grid, wl.block)
    imb = {}
    for sched in ("lpt", "naive"):
        tr = torch.zeros(nwg * 4, dtype=torch.int64, device="cuda")
        fva.sparse_attn(q, k, v, wl.grid, wl.block, mask, sched=sched, trace=tr, ws=ws_a, out=o, stream=stream)
        torch.cuda.synchronize()
        busy, finish, ncu = fva.trace_imbalance(tr.cpu().numpy())
        imb[sched] = {"busy_max_over_mean": round(busy, 4), "finish_max_over_mean": round(finish, 4), "cus": ncu}

    traffic = _profiled_traffic(wl.name)

    overlap = None
    if args.overlap > 0 and not wl.static:
        overlap = _overlap_leg(fva, wl, q, k, v, o, mask, args)

    graph = None
    if args.graph:
        graph = _graph_leg(fva, wl, q, k, v, shape, ws_r, ws_a, o, mask, args)

    sasa = None
    if args.sasa > 0 and not wl.static:
        sasa = _sasa_leg(fva, wl, q, k, v, host, shape, ws_r, ws_a, stream, args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(wl, host, mask_h, counts, args.oracle_items)

    res = {
        "metric": ("effective TFLOP/s of block-sparse attention per layer under a static local + anchor block mask"
                   if wl.static else
                   "effective TFLOP/s of routed sparse attention per layer (Wan 27280-token, 40-head layer)"),
        "value": round(eff_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth-field + noise Q/K/V; no model weights)",
        "config": {
            "workload": "%s: B=%d, heads=%d, head_dim=%d, grid=%s=%d tokens, block=%s -> %d blocks, %s, sched=%s"
                        % (wl.name, B, heads, D, list(wl.grid), L, list(wl.block), N,
                           ("static mask: local boxes %s blocks, anchor slabs every %d temporal blocks"
                            % (list(wl.static[0]), wl.static[1])) if wl.static else
                           "top_p=%g, k_floor=%d" % (wl.top_p, wl.k_floor), args.sched),
        },
        "ms_per_layer": round(ms_step, 4),
        "route_ms": round(route_ms, 4),
        "route_gbs": round(route_bytes / (route_ms * 1e-3) / 1e9, 1),
        "attn_call_ms": round(attn_ms, 4),
        "attn_plan_ms": round(plan_ms, 4),
        "attn_kernel_ms": round(kern_ms, 4),
        "stage_ms": stages,
        "effective_flop": eff_flop,
        "dense_equiv_tflops": round(dense_flop / (ms_step * 1e-3) / 1e12, 2),
        "kept_fraction_per_head": {"min": round(float(frac_per_head.min()), 4),
                                   "mean": round(float(frac_per_head.mean()), 4),
                                   "max": round(float(frac_per_head.max()), 4)},
        "dense_ref_ms": None if dense_ms is None else round(dense_ms, 4),
        "dense_ref_tflops": None if dense_ms is None else round(dense_flop / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense_ref": None if dense_ms is None else round(dense_ms / ms_step, 3),
        "cu_imbalance": imb,
        "roofline": {
            "bound": "mfma",
            "achieved": round(kern_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "sasa": sasa,
        "overlap": overlap,
        "graph": graph,
    }
    print(json.dumps(res), flush=True)


def _profiled_traffic(workload: str):
    """HBM bytes per launch of the sparse attention kernel from the committed
    rocprofv3 summary, or None if it was taken on another version of the
    kernel source (or another workload)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "attn_%s_traffic.md" % workload)
    src = os.path.join(ROOT, "adaptive_block_sparse_tile_amd", "csrc", "fva_attn.hip")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes:
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_hash.group(1):
        return None
    return float(m_bytes.group(1))


def _block_counts(wl):
    """Real tokens per block (harness arithmetic on the grid, for FLOP counting)."""
    T, H, W = wl.grid
    bt, bh, bw = wl.block
    et = [min(bt, T - i * bt) for i in range(-(-T // bt))]
    eh = [min(bh, H - i * bh) for i in range(-(-H // bh))]
    ew = [min(bw, W - i * bw) for i in range(-(-W // bw))]
    return np.array([a * b * c for a in et for b in eh for c in ew], dtype=np.int64)


def _graph_leg(fva, wl, q, k, v, shape, ws_r, ws_a, o_ref, mask_ref, args):
    """The same layer (mask, plan, attention kernel) captured once into a HIP
    graph on a side stream and replayed: no host work between the kernels.
    Same timing protocol as the main loop; each timed run's output checked
    bitwise against the main loop's, with eager work between replays."""
    import torch
    B, L, heads, D = shape
    N = fva.num_blocks(wl.grid, wl.block)
    o = torch.empty_like(q)
    mask = torch.empty((B, heads, N, (N + 31) // 32), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, heads, N), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()

    def layer(s):
        if wl.static:
            fva.static_mask(shape, wl.grid, wl.block, local=wl.static[0], anchor_t=wl.static[1], out=(mask, cnt),
                            stream=s)
        else:
            fva.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r, out=(mask, cnt, status), stream=s)
        fva.attn_plan(k, v, wl.grid, wl.block, mask, sched=args.sched, ws=ws_a, stream=s)
        fva.attn_exec(q, wl.grid, wl.block, mask, ws_a, sched=args.sched, out=o, stream=s)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(side)            # warm the side stream before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layer(side)
    torch.cuda.synchronize()
    equal = True
    main = torch.cuda.current_stream()
    for _ in range(args.warmup):
        o.zero_()
        mask.zero_()
        g.replay()
    torch.cuda.synchronize()
    equal &= bool(torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(mask, mask_ref))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for _ in range(args.steps):
        g.replay()
    e1.record(main)
    torch.cuda.synchronize()
    equal &= bool(torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(mask, mask_ref))
    res = {"ms_per_layer_graph": round(e0.elapsed_time(e1) / args.steps, 4), "bitwise_equal": equal}
    del g
    return res


def _overlap_leg(fva, wl, q, k, v, o_ref, mask_ref, args):
    """Overlap/Opt. through the library (fva_routed_attn): the whole layer as
    one call with groups = 1, and pipelined over G head groups on one stream
    and alternating between two streams (default priority).  Same timing
    protocol as the main loop; outputs checked bitwise against it."""
    import torch
    G = args.overlap
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    res = {"groups": G}
    variants = (("ms_per_layer_groups_1", 1, None), ("ms_per_layer_groups_G_one_stream", G, None),
                ("ms_per_layer_groups_G_two_streams", G, side))
    for name, groups, s in variants:
        ws = fva.workspace(fva.routed_attn_workspace_bytes(tuple(q.shape), wl.grid, wl.block, groups), q.device)
        out = fva.routed_attn(q, k, v, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups, side_stream=s, ws=ws)
        for _ in range(args.warmup):
            fva.routed_attn(q, k, v, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups, side_stream=s, ws=ws,
                            out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for _ in range(args.steps):
            fva.routed_attn(q, k, v, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups, side_stream=s, ws=ws,
                            out=out)
        e1.record(main)
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / args.steps, 4)
        res[name.replace("ms_per_layer", "bitwise_equal")] = bool(
            torch.equal(out[0].view(torch.int16), o_ref.view(torch.int16)) and torch.equal(out[1], mask_ref))
        del ws
    return res


def _sasa_leg(fva, wl, q, k, v, host, shape, ws_r, ws_a, stream, args):
    """Slack-aware augmentation on the per-XCD schedule: ms/layer without it
    (the plan's own LPT placement), with it on equal XCDs, and with it on
    measured XCD speeds (a traced per-XCD run under SASA's placement gives each
    XCD's time per unit of cost; fva_trace_xcd_speed turns that into weights).
    Same timing protocol as the main loop.  Also the mean absolute error of O
    against dense attention (fp64 oracle) on sampled query blocks, most of them
    blocks that received extra key blocks."""
    import torch
    import oracle
    B, L, heads, D = shape
    N = fva.num_blocks(wl.grid, wl.block)
    o = torch.empty_like(q)
    mask = torch.empty((B, heads, N, (N + 31) // 32), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, heads, N), dtype=torch.int32, device="cuda")
    mask_s, cnt_s = torch.empty_like(mask), torch.empty_like(cnt)
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    sws = fva.workspace(fva.sasa_workspace_bytes(shape, wl.grid, wl.block, args.sasa), q.device)

    def layer(rounds, weight):
        fva.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r, out=(mask, cnt, status), stream=stream)
        m, hx = mask, None
        if rounds is not None:
            m, _, hx, _ = fva.sasa(shape, wl.grid, wl.block, mask, ws_r, rounds=rounds, xcd_weight=weight,
                                   out=(mask_s, cnt_s), ws=sws, stream=stream)
        fva.attn_plan(k, v, wl.grid, wl.block, m, sched="xcd", head_xcd=hx, ws=ws_a, stream=stream)
        fva.attn_exec(q, wl.grid, wl.block, m, ws_a, sched="xcd", out=o, stream=stream)
        return m

    def timed(rounds, weight):
        for _ in range(args.warmup):
            layer(rounds, weight)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            m = layer(rounds, weight)
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / args.steps, 4), o.clone(), m.clone()

    # XCD speeds: a traced per-XCD run under SASA's placement (no augmentation)
    layer(0, None)
    _, _, hx0, load0 = fva.sasa(shape, wl.grid, wl.block, mask, ws_r, rounds=0, out=(mask_s, cnt_s), ws=sws)
    ws_t = fva.attn_plan(k, v, wl.grid, wl.block, mask, sched="xcd", head_xcd=hx0)
    nwg = fva.attn_workgroups(shape, wl.grid, wl.block)
    # eight launches after a warm-up one, their traces pooled: one launch's
    # per-XCD speeds vary by 0.5-0.8% (one sigma) on the 7 ms layer, about
    # the size of the slack SASA fills there
    tr = torch.zeros((9, nwg * 4), dtype=torch.int64, device="cuda")
    for i in range(9):
        fva.attn_exec(q, wl.grid, wl.block, mask, ws_t, sched="xcd", trace=tr[i])
    torch.cuda.synchronize()
    weight = fva.xcd_speed(tr[1:].cpu().numpy(), load0.cpu().numpy())
    del ws_t

    res = {"rounds": args.sasa, "xcd_weight": weight.tolist()}
    ms_xcd, o_xcd, m_xcd = timed(None, None)
    ms_sasa, o_sasa, m_sasa = timed(args.sasa, None)
    ms_place, _, _ = timed(0, weight)
    ms_wsasa, o_wsasa, m_wsasa = timed(args.sasa, weight)
    res.update({"ms_per_layer_xcd": ms_xcd, "ms_per_layer_sasa": ms_sasa,
                "ms_per_layer_xcd_weighted_placement": ms_place, "ms_per_layer_sasa_weighted": ms_wsasa})
    _, _, _, load = fva.sasa(shape, wl.grid, wl.block, mask, ws_r, rounds=args.sasa, xcd_weight=weight,
                             out=(mask_s, cnt_s), ws=sws)
    torch.cuda.synchronize()
    ld = load.cpu().numpy()
    kept0 = m_xcd.cpu().numpy().view(np.uint32)
    kept1 = m_wsasa.cpu().numpy().view(np.uint32)
    bits = lambda m: int(np.unpackbits(m.view(np.uint8)).sum())
    grown = np.nonzero((kept1 != kept0).any(-1).reshape(-1))[0]
    rng = np.random.default_rng(2)
    pick = set(rng.choice(grown, size=min(24, grown.size), replace=False).tolist()) if grown.size else set()
    while len(pick) < min(32, B * heads * N):
        pick.add(int(rng.integers(B * heads * N)))
    items = np.array(sorted(pick))
    print("[bench] sasa: dense oracle on %d sampled items" % len(items), file=sys.stderr, flush=True)
    qh, kh, vh = host
    dense = oracle.attn(qh, kh, vh, wl.grid, wl.block, oracle.dense_mask(B, heads, N), 1.0 / math.sqrt(D),
                        items=items, nthreads=oracle.host_threads())
    tb = oracle.token_block(wl.grid, wl.block)
    import fvgen
    err = {}
    grown_set = set(grown.tolist())
    for name, out in (("xcd", o_xcd), ("xcd_sasa_weighted", o_wsasa)):
        out = fvgen.bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
        e_all, e_grown = [], []
        for it in items:
            i, h, b = it % N, (it // N) % heads, it // (N * heads)
            d = np.abs(out[b, tb == i, h] - dense[b, tb == i, h]).mean()
            e_all.append(d)
            if it in grown_set:
                e_grown.append(d)
        err[name] = (float(np.mean(e_all)), float(np.mean(e_grown)) if e_grown else None)
    res.update({
        "xcd_load_before": [int(x) for x in ld[:8]],
        "xcd_added": [int(x) for x in ld[8:]],
        "kept_blocks_before": bits(kept0),
        "kept_blocks_after": bits(kept1),
        "rows_augmented": int(grown.size),
        "sampled_items": int(items.size),
        "mean_abs_err_vs_dense": {k2: round(v2[0], 6) for k2, v2 in err.items()},
        "mean_abs_err_vs_dense_on_augmented_rows": {k2: None if v2[1] is None else round(v2[1], 6)
                                                    for k2, v2 in err.items()},
    })
    return res


def _cpu_baseline(wl, host, mask_h, counts, n_items):
    """The fp64 oracle, as it stands, on the host cores this process may use
    (its CPU affinity, capped by OMP_NUM_THREADS when set: the host's share
    for one GPU): the full router, plus attention on a seeded sample of work
    items (including the heaviest and the lightest).  Reported as effective
    TFLOP/s on that sample, with the thread count, the host's hardware
    threads and the CPU model."""
    import oracle
    q, k, v = host
    N = len(counts)
    B, heads = mask_h.shape[0], mask_h.shape[1]
    threads = oracle.host_threads()
    print("[bench] cpu baseline: oracle router + %d attention items on %d threads (%s, %d hardware threads)"
          % (n_items, threads, oracle.cpu_model(), oracle.hardware_threads()), file=sys.stderr, flush=True)
    t0 = time.time()
    if wl.static:
        oracle.static_mask(wl.grid, wl.block, wl.static[0], wl.static[1], B=B, heads=heads)
    else:
        oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, nthreads=threads)
    route_s = time.time() - t0
    kept = ((mask_h[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(B * heads * N, -1)[:, :N]
    cost = counts[np.arange(B * heads * N) % N] * (kept * counts[None, :]).sum(1)
    rng = np.random.default_rng(1)
    pick = {int(np.argmax(cost)), int(np.argmin(cost))}
    while len(pick) < min(n_items, cost.size):
        pick.add(int(rng.integers(cost.size)))
    items = np.array(sorted(pick))
    t0 = time.time()
    oracle.attn(q, k, v, wl.grid, wl.block, mask_h, 1.0 / math.sqrt(wl.head_dim), items=items, nthreads=threads)
    attn_s = time.time() - t0
    flop = 4.0 * wl.head_dim * float(cost[items].sum())
    total_flop = 4.0 * wl.head_dim * float(cost.sum())
    return {
        "value": round(flop / attn_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_hardware_threads": oracle.hardware_threads(),
        "cpu_model": oracle.cpu_model(),
        "kind": "oracle",
        "sample": "%d of %d work items (heaviest, lightest, seeded random), %.2f%% of the layer's effective FLOPs; "
                  "attention %.1fs, full %s %.2fs; whole layer extrapolated %.0fs"
                  % (len(items), cost.size, 100 * flop / total_flop, attn_s,
                     "static mask" if wl.static else "router", route_s,
                     route_s + attn_s * total_flop / flop),
    }


if __name__ == "__main__":
    main()
