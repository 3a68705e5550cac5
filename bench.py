#!/usr/bin/env python
"""Throughput of the DFlash 2 drafter's forward pass on one MI355X.

Workloads (synthetic, seeded; random-init sidecars of the stated shapes,
int4 q/k/v/o/gate/up/down, f16 fc, kernel projections, head, selector):

  27b stream (the headline `value`)  the 27B-target-shaped sidecar (hidden
          5120, intermediate 17408, 5 layers, 32/8 heads, head_dim 128, vocab
          248320, block 16, 5 taps = tap width 25600, windows [2048 x4, 0],
          layer 4 without rotary): 32768 context positions settled first
          (untimed); then each step settles the next 8 tap rows and runs one
          block at the next anchor (k = 15 draft rows, head width = the
          vocabulary, a uniform anchor token). `value` = steps per second =
          draft blocks per second, the 8-row settle included.
  27b settle  the same sidecar: 16384 tap rows (N(0,1), 1 % of the channels
          x20) settled in 64 calls of 256 rows: settle rows per second.
  4b      the Qwen3-4B-shaped sidecar (hidden 2560, intermediate 9728, vocab
          151936): 4096 rows settled in 16 calls of 256 (timed: rows/s), then
          200 blocks at a = 4096 (timed: blocks/s).
  27b long  the 27B sidecar with every window 0, vocab 262144, top 32, rank
          128: 131071 positions settled (untimed), then 200 steps of one new
          row settled and one block at a = 131072 + i.

One JSON line on stdout; progress on stderr. Inputs are resident in device
memory before any timed region. The per-kernel rooflines come from the
library's stage timers (hipEvents on its stream) in a separate timed pass.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
F16_MFMA_PEAK_TFS = 2500.0   # MI355X dense f16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-calls", type=int, default=64)
    ap.add_argument("--timing-steps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (x*1 into another buffer), the "
                         "reference kernel for scaling the HBM byte counters")
    ap.add_argument("--cpu-steps", type=int, default=4,
                    help="stream steps the CPU oracle baseline runs")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 4B and long-context legs")
    ap.add_argument("--no-batch", action="store_true", help="skip the batched-blocks leg")
    ap.add_argument("--blocks-4b", type=int, default=200)
    ap.add_argument("--steps-long", type=int, default=200)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the drafter's path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_drafter_settle_amd as pkg
    from block_drafter_settle_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # one side stream for everything (torch's work and events included): a
    # block can then also be captured into a graph on it
    side = torch.cuda.Stream(dev)
    torch.cuda.set_stream(side)
    stream = side.cuda_stream
    g = synth.geometry("t27b")
    hs, V, tw, L = g["hidden"], g["vocab"], synth.tap_width(g), g["layers"]
    kd = g["kv_heads"] * g["head_dim"]
    k, width, per_step = g["block"] - 1, g["vocab"], 8
    ctx0 = 32768
    steps, warm = args.steps, args.warmup
    cap = max(ctx0 + per_step * (warm + steps + 2 * args.timing_steps) + 16, 16384 + 256)

    t0 = time.time()
    w = synth.make_weights(g, seed=0, device=dev)
    log(f"weights generated in {time.time() - t0:.1f}s")
    t0 = time.time()
    d = pkg.Drafter(g, w, max_context=cap, stream=stream)
    d.reserve(cap)  # the full layer's store at its final size: no store moves later
    log(f"drafter created in {time.time() - t0:.1f}s (store capacity {cap} rows)")

    if args.calibrate_copy:
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: {src.numel() * 4} bytes read, {dst.numel() * 4} bytes written")
        del src, dst

    # ------------------------------------------------ settle-bound workload
    n_set = 256 * args.settle_calls
    taps4 = synth.make_taps(g, n_set, seed=0, name="settle_taps", outliers=True, device=dev)
    calls = args.settle_calls
    for i in range(4):
        d.settle(0, 256, taps4[256 * (i % calls):].data_ptr())
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.settle_calls):
        d.settle(256 * i, 256, taps4[256 * i:].data_ptr())
    ev1.record()
    torch.cuda.synchronize()
    settle_s = ev0.elapsed_time(ev1) / 1e3
    # per-call times (an events pair around each call), for the median
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.settle_calls)]
    for i, (a0, a1) in enumerate(cev):
        a0.record()
        d.settle(256 * i, 256, taps4[256 * i:].data_ptr())
        a1.record()
    torch.cuda.synchronize()
    settle_call_med_us = float(np.median([a0.elapsed_time(a1) * 1e3 for a0, a1 in cev]))
    settle_rows_s = n_set / settle_s
    log(f"settle: {n_set} rows in {settle_s * 1e3:.2f} ms -> {settle_rows_s / 1e6:.3f} M rows/s")
    d.set_timing(True)
    for i in range(8):
        d.settle(256 * i, 256, taps4[256 * (i % calls):].data_ptr())
    st_settle, _, n_settles = d.stage_times()
    d.set_timing(False)
    del taps4

    # ------------------------------------------------------ stream workload
    t0 = time.time()
    for c in range(ctx0 // 256):
        tp = synth.make_taps(g, 256, seed=0, name=f"context.{c}", device=dev)
        d.settle(256 * c, 256, tp.data_ptr())
    torch.cuda.synchronize()
    log(f"context of {ctx0} positions settled in {time.time() - t0:.1f}s")
    total = warm + steps + 2 * args.timing_steps
    stream_taps = synth.make_taps(g, per_step * total, seed=0, name="stream", device=dev)
    anchors = synth.uniform_tokens(g, total, seed=0)
    top = g["selector_top"]
    out = dict(logits=torch.empty(k, width, device=dev),
               cand=torch.empty(k, top, dtype=torch.int32, device=dev),
               unary=torch.empty(k, top, device=dev), score=torch.empty(k, top, device=dev),
               chosen=torch.empty(k, dtype=torch.int32, device=dev))
    ptrs = [out[n].data_ptr() for n in ("logits", "cand", "unary", "score", "chosen")]
    pos = ctx0

    def step(i):
        nonlocal pos
        d.settle(pos, per_step, stream_taps[per_step * i:].data_ptr())
        pos += per_step
        d.block(anchors[i], pos, k, width, *ptrs)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warm, warm + steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    value = steps / dt
    log(f"stream: {steps} steps in {dt * 1e3:.1f} ms -> {value:.1f} blocks/s")

    # per-step times over a further stretch (events around each step)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.timing_steps)]
    for j, (a0, a1) in enumerate(sev):
        a0.record()
        step(warm + steps + j)
        a1.record()
    torch.cuda.synchronize()
    step_med_us = float(np.median([a0.elapsed_time(a1) * 1e3 for a0, a1 in sev]))

    # the head at the pages' CUDA default width (65536 columns) over a short
    # stretch: the same blocks, fewer head bytes; re-anchored at the same
    # positions (the store already holds them)
    w2 = 65536
    out2 = torch.empty(k, w2, device=dev)
    p2 = [out2.data_ptr()] + ptrs[1:]
    n2 = args.timing_steps
    for i in range(5):
        d.block(anchors[i], pos, k, w2, *p2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n2):
        d.block(anchors[i], pos, k, w2, *p2)
    torch.cuda.synchronize()
    w2_us = (time.perf_counter() - t0) / n2 * 1e6
    del out2
    # blocks alone at the full width over the same stretch: the block pass's
    # own throughput, with no settle between blocks and no stage timers
    for i in range(5):
        d.block(anchors[i], pos, k, width, *ptrs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n2):
        d.block(anchors[i], pos, k, width, *ptrs)
    torch.cuda.synchronize()
    bo_us = (time.perf_counter() - t0) / n2 * 1e6
    pos_bo = pos
    # the same block as one submission: captured into a graph once, replayed
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=side, capture_error_mode="thread_local"):
        d.block(anchors[0], pos, k, width, *ptrs)
    for i in range(5):
        gr.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n2):
        gr.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) / n2 * 1e6
    del gr

    # batched blocks: B handles sharing the weights, each over its own
    # 32768-position context (the lead is this stream's handle)
    batched = {} if args.no_batch else leg_batch(pkg, synth, dev, stream, d, g, ctx0, pos, k,
                                                 width, anchors, n2)

    # stage timers over a further stretch of the stream
    d.set_timing(True)
    for i in range(warm + steps + args.timing_steps, total):
        step(i)
    st_stream, n_blocks, n_str_settles = d.stage_times()
    d.set_timing(False)
    block_stages = ("kproj", "conv_norm", "qkv", "qk_post", "attention", "o", "gate_up", "down",
                    "head", "select")
    block_us = sum(st_stream[s][0] for s in block_stages) / n_blocks
    head_us = st_stream["head"][0] / st_stream["head"][1]
    # algorithmic bytes of one head launch: head rows and selector rows (f16)
    # read once, the logits written once
    head_bytes = width * hs * 2 + g["selector_rank"] * hs * 2 + k * width * 4
    head_gbs = head_bytes / (head_us * 1e-6) / 1e9
    bo_bytes = block_bytes(g, 0, pos_bo, width, k)
    # the same blocks with the head over the first 65536 columns
    w2_bytes = bo_bytes - head_bytes + (w2 * hs * 2 + g["selector_rank"] * hs * 2 + k * w2 * 4)
    # settle: the fc GEMM's flops per 256-row launch
    fc_us = st_settle["settle_fc"][0] / st_settle["settle_fc"][1]
    fc_flops = 2.0 * 256 * tw * hs
    # bytes the fc must move at least: its weight once, the 256 f16 tap rows,
    # the 256 f32 output rows. At 256 rows the weight stream (hbm) takes longer
    # at peak than the products (mfma): 244 flop/B is under the chip's
    # 2.5 PFLOP/s ÷ 8 TB/s = 312 flop/B.
    fc_bytes = tw * hs * 2 + 256 * tw * 2 + 256 * hs * 4
    fc_bound = "hbm" if fc_bytes / (HBM_PEAK_GBS * 1e9) >= fc_flops / (F16_MFMA_PEAK_TFS * 1e12) \
        else "mfma"
    call_flops = settle_flops(g, 256)
    settle_call_us = sum(v[0] for n, v in st_settle.items() if n.startswith("settle")) / n_settles

    stages = {n: round(st_stream[n][0] / n_blocks, 2) for n in block_stages}
    # the stream's own 8-row settles, per call
    stages["stream_settle"] = round(sum(v[0] for n, v in st_stream.items() if n.startswith("settle"))
                                    / max(n_str_settles, 1), 2)
    stages.update({n: round(st_settle[n][0] / n_settles, 2) for n in st_settle
                   if n.startswith("settle")})
    res = {
        "metric": "draft blocks/s + settle rows/s (27B-shaped sidecar), % of HBM/MFMA roofline",
        "value": round(value, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(dt * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "27b_stream: 27B-target-shaped drafter (hidden 5120, ffn 17408, 5 layers, "
                        "32/8 heads, hd 128, vocab 248320, block 16, tap width 25600, windows "
                        "[2048x4,0], layer 4 no_rope), 32768 settled positions, each step settles "
                        "8 new tap rows then drafts one block (k=15, width=vocab) at the next anchor",
            "weights": "int4 g32 f16-scale q/k/v/o/gate/up/down; f16 fc/kproj/head/selector; "
                       "f32 context K/V held as f16 hi/lo pairs; f16 MFMA operands, f32 accumulate",
            "block_rows": g["block"], "k": k, "width": width, "context": ctx0,
            "settle_rows_per_step": per_step,
        },
        "block_only": {
            "blocks_per_s": round(1e6 / bo_us, 1),
            "us_per_block": round(bo_us, 1),
            "algorithmic_bytes": int(bo_bytes),
            "hbm_frac": round(bo_bytes / (bo_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "blocks alone at the full width, back to back (no settle between, no "
                    "stage timers); stage_timer_us is the same pass under per-kernel events",
            "stage_timer_us": round(block_us, 1),
            "graph_replay_us": round(graph_us, 1),
            "graph_note": "the same block captured once into a HIP graph and replayed "
                          "(one submission a block)",
        },
        "batched": batched,
        "roofline": {
            "kernel": "k_head (head logits over the vocabulary + selector projection)",
            "bound": "hbm",
            "achieved": round(head_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head_gbs / HBM_PEAK_GBS, 4),
            "traffic": head_traffic(),
            "us_per_launch": round(head_us, 2),
            "bytes_per_launch": int(head_bytes),
        },
        "settle": {
            "workload": "27b_settle: 16384 tap rows (1% channels x20) in 64 calls of 256 rows",
            "rows_per_s": round(settle_rows_s, 1),
            "us_per_call": round(settle_call_us, 2),
            "mfma_frac_call": round(call_flops / (settle_call_us * 1e-6) / 1e12 /
                                    F16_MFMA_PEAK_TFS, 4),
            "roofline": {
                "kernel": "k_gemm_big_f16 (fc, 256 rows)",
                "bound": fc_bound,
                "achieved": round(fc_bytes / (fc_us * 1e-6) / 1e9, 1) if fc_bound == "hbm"
                else round(fc_flops / (fc_us * 1e-6) / 1e12, 2),
                "peak": HBM_PEAK_GBS if fc_bound == "hbm" else F16_MFMA_PEAK_TFS,
                "unit": "GB/s" if fc_bound == "hbm" else "TFLOP/s",
                "frac": round((fc_bytes / (fc_us * 1e-6) / 1e9 / HBM_PEAK_GBS) if fc_bound == "hbm"
                              else (fc_flops / (fc_us * 1e-6) / 1e12 / F16_MFMA_PEAK_TFS), 4),
                "traffic": fc_traffic(),
                "us_per_launch": round(fc_us, 2),
                "bytes_per_launch": int(fc_bytes),
                "flops_per_launch": fc_flops,
                "tflops": round(fc_flops / (fc_us * 1e-6) / 1e12, 2),
            },
        },
        "stages_us": stages,
        "block_width_65536": {
            "blocks_per_s": round(1e6 / w2_us, 1), "us_per_block": round(w2_us, 1),
            "algorithmic_bytes": int(w2_bytes),
            "hbm_frac": round(w2_bytes / (w2_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "blocks alone (no settle), head and selection over the first 65536 columns"},
        "median_us": {"stream_step": round(step_med_us, 2),
                      "settle_call": round(settle_call_med_us, 2)},
    }
    # the same rates against what this GPU sustains, measured by two probes
    # (a streaming read of the head weights; back-to-back f16 MFMAs)
    read_gbs, mfma_tfs = d.probe_peaks(3)
    log(f"measured peaks: streaming read {read_gbs:.0f} GB/s, f16 MFMA {mfma_tfs:.0f} TFLOP/s")
    res["measured_peaks"] = {"hbm_read_gbs": round(read_gbs, 1), "mfma_f16_tfs": round(mfma_tfs, 1)}
    res["roofline"]["frac_measured"] = round(head_gbs / read_gbs, 4)
    sr = res["settle"]["roofline"]
    sr["frac_measured"] = round((sr["achieved"] / read_gbs) if sr["bound"] == "hbm"
                                else (sr["achieved"] / mfma_tfs), 4)
    sr["mfma_frac"] = round(sr["tflops"] / F16_MFMA_PEAK_TFS, 4)
    sr["mfma_frac_measured"] = round(sr["tflops"] / mfma_tfs, 4)
    res["router"] = leg_route(synth, dev, d, hs)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(g, w, synth, args.cpu_steps)
        cpu["tiny"] = cpu_tiny(synth)
    d.close()
    del w, d
    torch.cuda.empty_cache()
    if not args.no_extra:
        res["qwen3_4b"], w4 = leg_4b(pkg, synth, dev, stream, args.blocks_4b)
        torch.cuda.empty_cache()
        if cpu is not None:
            cpu["qwen3_4b"] = cpu_4b(synth, w4)
        del w4
        res["t27b_long"], long_w = leg_long(pkg, synth, dev, stream, args.steps_long)
        torch.cuda.empty_cache()
        if cpu is not None:
            cpu["t27b_long_block"] = cpu_long_block(synth, long_w)
        del long_w
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def block_bytes(g, first, a, width, k):
    """Algorithmic bytes of one block at anchor position a over a context
    starting at `first` (settled through a): int4 weights with their scales,
    f16 kernel projections, the head rows read and the logits written, the
    selector projection, the visible K/V rows of every layer, the gathered
    codebook rows and the two embedding rows."""
    hs, L = g["hidden"], g["layers"]
    kd = g["kv_heads"] * g["head_dim"]
    qd = g["heads"] * g["head_dim"]
    ffn = g["intermediate"]
    rank, top = g["selector_rank"], g["selector_top"]
    i4 = L * (qd * hs + 2 * kd * hs + hs * qd + 3 * ffn * hs) * (0.5 + 2 / 32)
    kproj = L * 2 * (2 * g["conv_kernel"] * hs // g["conv_group"]) * hs * 2
    head = width * hs * 2 + rank * hs * 2 + k * width * 4
    kv_rows = 0
    for l in range(L):
        wdw = g["windows"][l]
        lo = max(first, a + 1 - wdw) if wdw > 0 else first
        kv_rows += max(0, a - lo)
    return i4 + kproj + head + kv_rows * kd * 4 * 2 + k * (1 + top) * rank * 2 + 2 * hs * 2


def batch_bytes(g, seqs, width, k):
    """Algorithmic bytes of one batched pass: the weights once, and each
    sequence's own K/V rows, logits, codebook and embedding rows. seqs:
    (first, a) per sequence."""
    one = [block_bytes(g, f, a, width, k) for f, a in seqs]
    hs, rank, top = g["hidden"], g["selector_rank"], g["selector_top"]
    own = [block_bytes(g, f, a, width, k) - block_bytes(g, 0, 0, width, k) +
           k * width * 4 + k * (1 + top) * rank * 2 + 2 * hs * 2 for f, a in seqs]
    return one[0] - own[0] + sum(own)


def block_flops(g, width, k, nseq):
    """Products of nseq blocks: every layer's projections on the block's 16
    rows, the head on rows 1..k and the selector projection on all 16."""
    hs, L = g["hidden"], g["layers"]
    kd, qd = g["kv_heads"] * g["head_dim"], g["heads"] * g["head_dim"]
    ffn, rows = g["intermediate"], g["block"]
    kp = 2 * (2 * g["conv_kernel"] * hs // g["conv_group"]) * hs
    per_layer = qd * hs + 2 * kd * hs + hs * qd + 3 * ffn * hs + kp
    return nseq * 2.0 * (rows * L * per_layer + k * width * hs + rows * g["selector_rank"] * hs)


def leg_route(synth, dev, d, hs, rank=64, calls=500):
    """The router margin (dflash_route_margin) of m = 1 and 8 target rows
    against two synthetic rank-64 subspaces, back to back on the handle's
    stream."""
    import torch

    blk_h = synth.make_subspace(hs, rank, seed=9)
    blk = [blk_h[0].to(dev), blk_h[1].to(dev)]
    chn = [t.to(dev) for t in synth.make_subspace(hs, rank, seed=9, name="route.chain")[:2]]
    bp = (blk[0].data_ptr(), blk[1].data_ptr(), rank)
    cp = (chn[0].data_ptr(), chn[1].data_ptr(), rank)
    out = {"workload": f"router: Route::margin of m target rows (hidden {hs}) against two "
                       f"synthetic rank-{rank} subspaces (f16 mean and basis)"}
    for m in (1, 8):
        rows = synth.make_route_rows(hs, m, seed=10, near=blk_h, share=0.5).to(dev)
        mg = torch.empty(m, device=dev)
        for _ in range(20):
            d.route_margin(rows.data_ptr(), m, bp, cp, mg.data_ptr())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(calls):
            d.route_margin(rows.data_ptr(), m, bp, cp, mg.data_ptr())
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        nbytes = m * hs * 4 + 2 * (hs + rank * hs) * 2 + m * 4
        out[f"m{m}"] = {"us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                        "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5)}
        log(f"router: m={m}: {us:.2f} us a call")
    return out


def leg_batch(pkg, synth, dev, stream, lead, g, ctx0, lead_pos, k, width, anchors, nb):
    """Batched blocks at B = 2, 4, 8: the lead plus B−1 context handles on the
    same weights, each holding a synthetic 32768-position store; nb passes
    each, timed back to back."""
    import torch

    store = synth.make_store(g, ctx0, seed=7, device=dev)
    others = []
    for i in range(7):
        o = pkg.Drafter.context_of(lead, ctx0 + 64, stream)
        o.debug_load_store(0, ctx0, [x[0].data_ptr() for x in store],
                           [x[1].data_ptr() for x in store])
        others.append(o)
    del store
    top = g["selector_top"]
    res = {}
    for nseq in (2, 4, 8):
        ds = [lead] + others[:nseq - 1]
        out = [torch.empty(nseq, k, width, device=dev),
               torch.empty(nseq, k, top, dtype=torch.int32, device=dev),
               torch.empty(nseq, k, top, device=dev), torch.empty(nseq, k, top, device=dev),
               torch.empty(nseq, k, dtype=torch.int32, device=dev)]
        ptrs = [t.data_ptr() for t in out]
        pos = [lead_pos] + [ctx0] * (nseq - 1)
        firsts = [0] * nseq
        for i in range(3):
            pkg.block_batch(ds, anchors[i:i + nseq], pos, k, width, *ptrs)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nb):
            pkg.block_batch(ds, anchors[i:i + nseq], pos, k, width, *ptrs)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / nb * 1e6
        by = batch_bytes(g, list(zip(firsts, pos)), width, k)
        fl = block_flops(g, width, k, nseq)
        res[f"B{nseq}"] = {
            "blocks_per_s": round(nseq * 1e6 / us, 1), "us_per_batch": round(us, 1),
            "algorithmic_bytes": int(by), "hbm_frac": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_flops": fl,
            "mfma_frac": round(fl / (us * 1e-6) / 1e12 / F16_MFMA_PEAK_TFS, 4),
        }
        log(f"batch of {nseq}: {us:.1f} us a pass -> {nseq * 1e6 / us:.1f} blocks/s")
        del out
    for o in others:
        o.close()
    res["workload"] = ("27b_batch: B sequences on the 27B-shaped sidecar's shared weights, each "
                       "over its own 32768-position context (the stream's, then synthetic "
                       "stores), one dflash_block_batch pass drafting all B blocks (k=15, "
                       "width=vocab); the weights are read once a pass")
    return res


def settle_flops(g, rows):
    """The settle's products: fc (tap width x hidden) and every layer's K and
    V (2 x kv_heads*head_dim x hidden), a multiply-add each, per row."""
    hs, tw = g["hidden"], g["n_taps"] * g["hidden"]
    kd = g["kv_heads"] * g["head_dim"]
    return 2.0 * rows * (tw * hs + g["layers"] * 2 * kd * hs)


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def leg_4b(pkg, synth, dev, stream, nblocks):
    """The 4B-shaped sidecar: 4096 rows settled in 16 calls of 256, then
    nblocks blocks at a = 4096 (width = vocab, k = 15)."""
    import numpy as np
    import torch

    g = synth.geometry("qwen3_4b")
    t0 = time.time()
    w = synth.make_weights(g, seed=0, device=dev)
    d = pkg.Drafter(g, w, max_context=4096 + 256, stream=stream)
    d.reserve(4096 + 256)
    log(f"4b: sidecar ready in {time.time() - t0:.1f}s")
    calls, n = 16, 4096
    taps = synth.make_taps(g, n, seed=0, name="settle_taps", outliers=True, device=dev)
    for i in range(4):  # warm
        d.settle(0, 256, taps[256 * i:].data_ptr())
    torch.cuda.synchronize()
    e0, e1 = _events(1)[0]
    e0.record()
    for i in range(calls):
        d.settle(256 * i, 256, taps[256 * i:].data_ptr())
    e1.record()
    torch.cuda.synchronize()
    settle_s = e0.elapsed_time(e1) / 1e3
    k, width, top = g["block"] - 1, g["vocab"], g["selector_top"]
    out = [torch.empty(k, width, device=dev), torch.empty(k, top, dtype=torch.int32, device=dev),
           torch.empty(k, top, device=dev), torch.empty(k, top, device=dev),
           torch.empty(k, dtype=torch.int32, device=dev)]
    ptrs = [t.data_ptr() for t in out]
    anchors = synth.uniform_tokens(g, max(nblocks, 10) + 10, seed=0)  # 10 warm, 20 timed stages
    for i in range(10):
        d.block(anchors[i], n, k, width, *ptrs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(nblocks):
        d.block(anchors[10 + i], n, k, width, *ptrs)
    torch.cuda.synchronize()
    blk_s = time.perf_counter() - t0
    d.set_timing(True)
    for i in range(20):
        d.block(anchors[i], n, k, width, *ptrs)
    st, nb, _ = d.stage_times()
    d.set_timing(False)
    d.close()
    bb = block_bytes(g, 0, n, width, k)
    us = blk_s / nblocks * 1e6
    sfl = settle_flops(g, n)
    log(f"4b: settle {n / settle_s / 1e6:.3f} M rows/s; blocks {nblocks / blk_s:.1f}/s")
    res = {
        "workload": "4b: Qwen3-4B-shaped sidecar (hidden 2560, ffn 9728, 5 layers, 32/8 heads, "
                    "hd 128, vocab 151936, block 16, tap width 12800, windows 0); 4096 rows "
                    "settled in 16 calls of 256, then blocks at a=4096 (k=15, width=vocab)",
        "blocks_per_s": round(nblocks / blk_s, 1), "us_per_block": round(us, 1),
        "blocks": nblocks, "algorithmic_bytes": int(bb),
        "hbm_frac": round(bb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "settle_rows_per_s": round(n / settle_s, 1),
        "settle_us_per_call": round(settle_s / calls * 1e6, 2),
        "settle_mfma_frac": round(sfl / settle_s / 1e12 / F16_MFMA_PEAK_TFS, 4),
        "stages_us": {s_: round(v[0] / nb, 2) for s_, v in st.items()
                      if not s_.startswith("settle") and v[1]},
    }
    return res, (g, w)


def leg_long(pkg, synth, dev, stream, steps):
    """The long-context sidecar: 131071 positions settled (untimed), then
    `steps` steps of one row settled + one block at a = 131072 + i."""
    import torch

    g = synth.geometry("t27b_long")
    t0 = time.time()
    w = synth.make_weights(g, seed=0, device=dev)
    ctx0 = 131071
    d = pkg.Drafter(g, w, max_context=ctx0 + steps + 40, stream=stream)
    d.reserve(ctx0 + steps + 40)
    log(f"long: sidecar ready in {time.time() - t0:.1f}s")
    t0 = time.time()
    for c in range((ctx0 + 255) // 256):
        m = min(256, ctx0 - 256 * c)
        tp = synth.make_taps(g, m, seed=0, name=f"long_context.{c}", device=dev)
        d.settle(256 * c, m, tp.data_ptr())
    torch.cuda.synchronize()
    log(f"long: {ctx0} positions settled in {time.time() - t0:.1f}s")
    k, width, top = g["block"] - 1, g["vocab"], g["selector_top"]
    out = [torch.empty(k, width, device=dev), torch.empty(k, top, dtype=torch.int32, device=dev),
           torch.empty(k, top, device=dev), torch.empty(k, top, device=dev),
           torch.empty(k, dtype=torch.int32, device=dev)]
    ptrs = [t.data_ptr() for t in out]
    warm = 10
    total = warm + steps + 20
    taps = synth.make_taps(g, total, seed=0, name="long_stream", device=dev)
    anchors = synth.uniform_tokens(g, total, seed=1)
    pos = ctx0

    def step(i):
        nonlocal pos
        d.settle(pos, 1, taps[i:].data_ptr())
        pos += 1
        d.block(anchors[i], pos, k, width, *ptrs)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    a_first = pos + 1
    t0 = time.perf_counter()
    for i in range(warm, warm + steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    a_last = pos
    # blocks alone at the last anchor (no settle between)
    t0 = time.perf_counter()
    for i in range(20):
        d.block(anchors[i], pos, k, width, *ptrs)
    torch.cuda.synchronize()
    bo_us = (time.perf_counter() - t0) / 20 * 1e6
    d.set_timing(True)
    for i in range(warm + steps, total):
        step(i)
    st, nb, _ = d.stage_times()
    d.set_timing(False)
    d.close()
    del d
    bytes_mean = sum(block_bytes(g, 0, a, width, k) for a in range(a_first, a_last + 1)) / steps
    bo_bytes = block_bytes(g, 0, pos, width, k)
    step_us = dt / steps * 1e6
    kd = g["kv_heads"] * g["head_dim"]
    attn_us = st["attention"][0] / nb
    kv_bytes = g["layers"] * pos * kd * 8
    log(f"long: {steps / dt:.1f} steps/s, blocks alone {1e6 / bo_us:.1f}/s")
    res = {
        "workload": "27b_long: 27B sidecar, every window 0 (layer 4 no_rope), vocab 262144, "
                    "top 32, rank 128; 131071 positions settled, then per step 1 row settled "
                    "+ one block at a=131072+i (k=15, width=vocab)",
        "steps_per_s": round(steps / dt, 1), "us_per_step": round(step_us, 1), "steps": steps,
        "block_only": {"blocks_per_s": round(1e6 / bo_us, 1), "us_per_block": round(bo_us, 1),
                       "algorithmic_bytes": int(bo_bytes),
                       "hbm_frac": round(bo_bytes / (bo_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "step_hbm_frac": round(bytes_mean / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "attention": {"us_per_block": round(attn_us, 1), "kv_bytes": int(kv_bytes),
                      "hbm_frac": round(kv_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "note": "attention chunks + merge of all 5 layers over the whole context"},
        "stages_us": {s_: round(v[0] / nb, 2) for s_, v in st.items() if v[1]},
    }
    return res, (g, w)


HEAD_TRAFFIC = os.path.join(ROOT, "profiles", "k_head_27b_stream_traffic.txt")
KERNELS = os.path.join(ROOT, "block_drafter_settle_amd", "csrc", "kernels.hip")


def head_source_sha1():
    """sha1 of the head kernel's source text (its comment through the row
    kernels' section line), so a traffic figure taken from counters is only
    reported for the kernel it was taken on."""
    import hashlib

    src = open(KERNELS).read()
    a = src.find("// The head over rows 1..k")
    b = src.find("// ----------------------------------------------------------- row kernels")
    if a < 0 or b < a:
        return None
    return hashlib.sha1(src[a:b].encode()).hexdigest()


def _source_sha1(start, end):
    """sha1 of kernels.hip's text from the line `start` to the line `end`."""
    import hashlib

    src = open(KERNELS).read()
    a = src.find(start)
    b = src.find(end, a + 1)
    if a < 0 or b < a:
        return None
    return hashlib.sha1(src[a:b].encode()).hexdigest()


def _traffic(path, sha):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by the plain copy's reading), or None when there
    is none or the kernel changed since it was taken."""
    try:
        fields = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    if sha is None or fields.get("kernel_source_sha1", "").strip() != sha:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def head_traffic():
    return _traffic(HEAD_TRAFFIC, head_source_sha1())


FC_TRAFFIC = os.path.join(ROOT, "profiles", "k_gemm_big_f16_27b_settle_traffic.txt")


def fc_traffic():
    """The settle fc kernel's (k_gemm_big_f16 at 256 rows) counter traffic."""
    return _traffic(FC_TRAFFIC, _source_sha1(
        "// Many-row GEMM, f16 weights, two activation planes",
        "template <int R, int PL>\n__global__ __launch_bounds__(kThreads) void k_gemm_i4("))


def cpu_baseline(g, w, synth, steps):
    """The CPU oracle on a bounded sample of the stream: `steps` stream steps
    (8 tap rows settled + one block over a 32768-row context each) on the
    host cores."""
    from oracle import oracle

    oracle.build()
    log(f"cpu baseline: oracle, {steps} stream steps ...")
    m = oracle.Model(g, w)
    store = [(k.numpy(), v.numpy()) for k, v in synth.make_store(g, 32768, seed=0)]
    taps = synth.make_taps(g, 8 * steps, seed=0, name="stream").numpy()
    anchors = synth.uniform_tokens(g, steps, seed=0)
    t_settle = t_block = 0.0
    for i in range(steps):
        t0 = time.perf_counter()
        m.settle(taps[8 * i:8 * i + 8], 32768 + 8 * i)
        t1 = time.perf_counter()
        r = m.block(store, 0, 32768, anchors[i], 32768, g["block"] - 1, g["vocab"])
        m.select(r["logits"], r["hp"], anchors[i])
        t2 = time.perf_counter()
        t_settle += t1 - t0
        t_block += t2 - t1
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count()))
    log(f"cpu baseline: settle {t_settle:.1f}s, block {t_block:.1f}s over {steps} steps")
    res = {"value": round(steps / (t_settle + t_block), 4), "unit": "blocks/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{steps} stream steps of the same workload: 8 tap rows settled + one block "
                     "(32768-position synthetic context, k=15, width=vocab) + selection, each",
           "settle_s": round(t_settle, 2), "block_s": round(t_block, 2),
           "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}
    # the settle unit: one 256-row call of the settle workload's tap rows
    st4 = synth.make_taps(g, 256, seed=0, name="settle_taps", outliers=True).numpy()
    t0 = time.perf_counter()
    m.settle(st4, 0)
    t4 = time.perf_counter() - t0
    log(f"cpu baseline: one 256-row settle call in {t4:.2f}s")
    res["settle"] = {"value": round(256 / t4, 1), "unit": "rows/s", "cores": cores,
                     "sample": "one 256-row settle call of the 27b settle workload"}
    # one step more on one thread (the oracle's OpenMP runtime set to 1), and
    # 16 settle rows on one thread
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        t0 = time.perf_counter()
        m.settle(taps[:8], 32768)
        r = m.block(store, 0, 32768, anchors[0], 32768, g["block"] - 1, g["vocab"])
        m.select(r["logits"], r["hp"], anchors[0])
        t1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        m.settle(st4[:16], 0)
        t5 = time.perf_counter() - t0
        gomp.omp_set_num_threads(cores)
        log(f"cpu baseline: one thread, one step in {t1:.1f}s, 16 settle rows in {t5:.1f}s")
        res["one_thread"] = {"value": round(1.0 / t1, 4), "unit": "blocks/s", "cores": 1,
                             "sample": "1 stream step of the same workload"}
        res["settle"]["one_thread"] = {"value": round(16 / t5, 2), "unit": "rows/s", "cores": 1,
                                       "sample": "16 rows of the 256-row call"}
    except OSError as e:
        log(f"cpu baseline: one-thread run skipped ({e})")
    return res


def cpu_tiny(synth):
    """The oracle on the tiny sidecar whole: 128 tap rows settled, then one
    block at a = 128 over them (k = block - 1, width = vocab)."""
    from oracle import oracle

    g = synth.geometry("tiny")
    w = synth.make_weights(g, seed=0)
    m = oracle.Model(g, w)
    n = 128
    taps = synth.make_taps(g, n, seed=0).numpy()
    anchor = 17
    t0 = time.perf_counter()
    K, V = m.settle(taps, 0)
    r = m.block([(K[l], V[l]) for l in range(g["layers"])], 0, n, anchor, n, g["block"] - 1,
                g["vocab"])
    m.select(r["logits"], r["hp"], anchor)
    t = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count()))
    return {"value": round(1.0 / t, 2), "unit": "runs/s", "cores": cores,
            "sample": "the tiny sidecar whole: 128 rows settled + one block + selection"}


def cpu_4b(synth, gw, device="cuda:0"):
    """The oracle on the 4B-shaped sidecar's unit: one 256-row settle call,
    then 3 blocks at a = 4096 over a 4096-position synthetic context (drawn on
    the GPU, copied to the host), all cores."""
    import torch
    from oracle import oracle

    g, w = gw
    m = oracle.Model(g, w)
    taps = synth.make_taps(g, 256, seed=0, name="settle_taps", outliers=True).numpy()
    t0 = time.perf_counter()
    m.settle(taps, 0)
    ts = time.perf_counter() - t0
    ctx = 4096
    store = [(k_.cpu().numpy(), v_.cpu().numpy())
             for k_, v_ in synth.make_store(g, ctx, seed=0, device=torch.device(device))]
    anchors = synth.uniform_tokens(g, 3, seed=0)
    t0 = time.perf_counter()
    for anchor in anchors:
        r = m.block(store, 0, ctx, anchor, ctx, g["block"] - 1, g["vocab"])
        m.select(r["logits"], r["hp"], anchor)
    tb = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count()))
    log(f"cpu baseline: 4b settle call in {ts:.2f}s, 3 blocks in {tb:.1f}s")
    return {"value": round(3 / tb, 4), "unit": "blocks/s", "cores": cores,
            "sample": "3 blocks of the 4b workload at a=4096 (4096-position synthetic context, "
                      "k=15, width=vocab) + selection",
            "settle": {"value": round(256 / ts, 1), "unit": "rows/s", "cores": cores,
                       "sample": "one 256-row settle call of the 4b workload"}}


def cpu_long_block(synth, gw):
    """The oracle on one block of the long-context workload: a 131072-position
    synthetic context (drawn on the GPU, copied to the host), all cores."""
    import torch
    from oracle import oracle

    g, w = gw
    ctx = 131072
    store = [(k_.cpu().numpy(), v_.cpu().numpy())
             for k_, v_ in synth.make_store(g, ctx, seed=0, device=torch.device("cuda:0"))]
    m = oracle.Model(g, w)
    anchor = synth.uniform_tokens(g, 1, seed=1)[0]
    t0 = time.perf_counter()
    r = m.block(store, 0, ctx, anchor, ctx, g["block"] - 1, g["vocab"])
    m.select(r["logits"], r["hp"], anchor)
    t1 = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count()))
    log(f"cpu baseline: one long-context block in {t1:.1f}s")
    return {"value": round(1.0 / t1, 4), "unit": "blocks/s", "cores": cores,
            "sample": "one block of the 27b long workload (131072 positions) + selection"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
