#!/usr/bin/env python3
"""Benchmark of the SSA block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over the 8k prefill workload (batch 1,
32 query heads on 2 KV heads, N=8192, d=64, B=64, k=16): block summaries and
scores, top-k selection, block-sparse attention forward, and the full-attention
counterpart with per-row dropped mass.  The decode workload (64 sequences x 1
token against a 32768-entry cache, 16+1 blocks) is measured in the same run
and reported under "decode".

Prints ONE JSON line.  ``value`` is tokens/s of the whole step (inputs already
resident in HBM), from the timed steps, which run with no event between their
kernels; per-kernel timings come from HIP events recorded around each call on
the stream the kernels run on, over as many further steps (medians reported).
The 8k prefill step is also timed on the planted and tie 8k workloads (batch
4) and on the 32k extrapolation workload, and a peaks leg measures what the
matrix cores, HBM and the shader clock deliver on this GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from block_sparse_attention_kv_amd.profiling import source_hash
    e = t.get(kernel)
    if not e or e.get("source_sha256_16") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def sparse_useful_pairs(nqb: int, topk: int, block: int) -> int:
    """(query row, key) pairs the sparse pattern attends to per (b, h) when every
    block is full: per query block, (selected - 1) full tiles plus the causal
    half of the diagonal tile."""
    total = 0
    for i in range(nqb):
        n_sel = min(topk, i + 1)
        total += (n_sel - 1) * block * block + block * (block + 1) // 2
    return total


def full_useful_pairs(lo: int, hi: int) -> int:
    """Causal pairs of rows [lo, hi): sum of (r + 1)."""
    return (hi * (hi + 1) - lo * (lo + 1)) // 2


class KernelTimer:
    """Collects HIP-event durations of named calls on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.times = {}

    def run(self, name, fn, *args, **kw):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn(*args, **kw)
        e1.record()
        self.pending.append((name, e0, e1))
        return r

    def collect(self):
        for name, e0, e1 in self.pending:
            self.times.setdefault(name, []).append(e0.elapsed_time(e1))
        self.pending.clear()

    def median_ms(self, name):
        t = sorted(self.times[name])
        n = len(t)
        return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])

    def avg_ms(self, name):
        return sum(self.times[name]) / len(self.times[name])


class PlainRunner:
    """Same interface as KernelTimer, no events: the step timing runs through
    this, since an event record between kernels costs a few microseconds of
    GPU time by itself."""

    def run(self, name, fn, *args, **kw):
        return fn(*args, **kw)


def timed_steps(torch, step, n):
    """(ms per step, wall seconds) of ``n`` back-to-back plain steps, bracketed
    by synchronisations."""
    plain = PlainRunner()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(n):
        step(plain, i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, time.perf_counter() - t0


def kernel_pass(torch, timer, step, n):
    """Per-call HIP-event durations over ``n`` further steps."""
    torch.cuda.synchronize()
    timer.pending.clear()
    for i in range(n):
        step(timer, i)
    torch.cuda.synchronize()
    timer.collect()


def bench_prefill(args, torch, ssa, W, shared=False, workload=None, steps=None):
    """One step = summaries+scores, top-k, block-sparse forward, full forward
    with dropped mass; ``shared`` uses the group-shared selection."""
    w = W.BY_NAME[workload or args.workload]
    n_steps = steps or args.steps
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nqb, nkb = ssa.n_blocks(w.seq_q, w.block), ssa.n_blocks(w.seq_kv, w.block)
    if w.full_rows is None:
        fb0, fcnt = 0, nqb
    else:
        fb0 = w.full_rows[0] // w.block
        fcnt = ssa.n_blocks(w.full_rows[1], w.block) - fb0
    scores = torch.empty((w.batch, w.n_q_heads, nqb, nkb), dtype=torch.float32, device=dev)
    ksum = torch.empty((w.batch, w.n_kv_heads, nkb, w.head_dim), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_kv_heads if shared else w.n_q_heads, nqb, w.topk), dtype=torch.int32,
                      device=dev)
    select = ssa.ssa_select_topk_shared if shared else ssa.ssa_select_topk
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    rows = min(w.seq_q, (fb0 + fcnt) * w.block) - fb0 * w.block
    out_f = torch.empty((w.batch, w.n_q_heads, rows, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse_f = torch.empty((w.batch, w.n_q_heads, rows), dtype=torch.float32, device=dev)
    drop = torch.empty_like(lse_f)
    # work queues of the persistent attention launches (zeroed once, left zeroed by every call)
    ws_sp = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=dev)
    ws_full = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_FULL_FWD),), dtype=torch.uint8, device=dev)
    timer = KernelTimer(torch)

    def step(t, i=0):
        t.run("scores", ssa.ssa_block_scores, shape, q, k, summary_out=ksum, scores=scores)
        t.run("topk", select, shape, scores, idx)
        t.run("sparse_attn", ssa.ssa_block_sparse_attn_fwd, shape, q, k, v, idx, workspace=ws_sp, out=out, lse=lse,
              shared=shared)
        t.run("full_attn", ssa.ssa_full_attn_fwd_dropped_mass, shape, q, k, v, idx, fb0, fcnt,
              out=out_f, lse=lse_f, dropped=drop, shared=shared, workspace=ws_full)

    plain = PlainRunner()
    for i in range(args.warmup):
        step(plain, i)
    ms_step, wall = timed_steps(torch, step, n_steps)
    kernel_pass(torch, timer, step, n_steps)

    pairs_sp = w.batch * w.n_q_heads * sparse_useful_pairs(nqb, w.topk, w.block)
    pairs_full = w.batch * w.n_q_heads * full_useful_pairs(fb0 * w.block, fb0 * w.block + rows)
    flops = {"sparse_attn": 4.0 * w.head_dim * pairs_sp, "full_attn": 4.0 * w.head_dim * pairs_full}
    bytes_alg = {
        # summaries read K once and write K-bar; scores read Q once and write S
        "scores": (k.numel() * 2 + ksum.numel() * 4 + q.numel() * 2 + scores.numel() * 4),
        "topk": scores.numel() * 4 + idx.numel() * 4,
    }
    kernels = {}
    for name in ("scores", "topk", "sparse_attn", "full_attn"):
        ms = timer.median_ms(name)
        e = {"median_ms": round(ms, 5), "mean_ms": round(timer.avg_ms(name), 5)}
        if name in flops:
            tf = flops[name] / (ms * 1e-3) / 1e12
            e.update(bound="mfma", gflop_per_launch=round(flops[name] / 1e9, 3),
                     tflops=round(tf, 2), frac_of_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        else:
            gbs = bytes_alg[name] / (ms * 1e-3) / 1e9
            e.update(bound="hbm", mbytes_per_launch=round(bytes_alg[name] / 1e6, 3),
                     gbs=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
        kernels[name] = e
    # the metric's kernel: the block-sparse forward on selected-block flops
    counted = not shared and w.name == "prefill_8k"
    roof = roofline_entry("sparse_attn", kernels["sparse_attn"], flops, bytes_alg, counted)
    roof_full = roofline_entry("full_attn", kernels["full_attn"], flops, bytes_alg, counted)
    del q, k, v, scores, ksum, idx, out, lse, out_f, lse_f, drop, ws_sp, ws_full
    return dict(w=w, ms_step=ms_step, wall=wall, kernels=kernels, roofline=roof, roofline_full=roof_full,
                tokens_per_s=w.batch * w.seq_q / (ms_step * 1e-3))


def roofline_entry(name, e, flops, bytes_alg, counted=True):
    """Roofline object of one kernel.  The committed counter summary covers the
    per-head selection on the 8k prefill workload only: other launches get no
    traffic figure."""
    if e["bound"] == "mfma":
        ach = e["tflops"]
        r = {"kernel": name, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / PEAK_BF16_TFLOPS, 4), "algorithmic_per_launch": flops[name]}
    else:
        ach = e["gbs"]
        r = {"kernel": name, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(ach / PEAK_HBM_GBS, 4), "algorithmic_per_launch": bytes_alg[name]}
    r["traffic"] = measured_traffic(name) if counted else None
    return r


def prefill_leg(res):
    """Bench-line entry of a prefill run on another workload."""
    w = res["w"]
    return {"workload": w.name, "batch": w.batch, "seq_len": w.seq_q, "variant": w.variant,
            "full_rows": list(w.full_rows) if w.full_rows else None,
            "ms_per_step": round(res["ms_step"], 5), "tokens_per_s": round(res["tokens_per_s"], 1),
            "kernels": res["kernels"], "roofline": res["roofline"], "roofline_full": res["roofline_full"]}


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _event_ms(torch, fn, reps):
    """Median HIP-event time of ``reps`` single calls of ``fn``."""
    out = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return _median(out)


def _u32(t):
    """int32 tensor holding uint32 bit patterns -> int64 values on the CPU."""
    return t.long().cpu() & 0xFFFFFFFF


def bench_peaks(args, torch, ssa, W):
    """Measured peaks beside the nominal ones: a matrix-instruction loop with no
    memory traffic (bf16 32x32x16, 2 waves per SIMD), a compute-only replica
    of the attention tile, a streaming read and a streaming copy of 1 GiB, and
    the shader clock of an idle GPU (the clock under the attention kernels
    comes from their own timing records)."""
    from block_sparse_attention_kv_amd import peaks as P
    P.load_library()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"compute_units": cus}
    i32 = torch.int32

    def clock_ghz(out):
        c = _u32(out)
        return float(c[0]) / float(c[1]) * P.REALTIME_HZ / 1e9

    clk = torch.zeros(2, dtype=i32, device=dev)
    P.clock(20000, clk)
    torch.cuda.synchronize()
    res["clock_idle_ghz"] = round(clock_ghz(clk), 3)

    # matrix-instruction loop: 2 waves per SIMD, about 2 ms
    iters, nb = 4000, 2 * cus
    mo = torch.zeros(16 * nb, dtype=i32, device=dev)
    P.mfma(iters, nb, mo)
    torch.cuda.synchronize()
    ms = _event_ms(torch, lambda: P.mfma(iters, nb, mo), 5)
    per_wave = _u32(mo).view(-1, 4)
    ghz = float((per_wave[:, 1].double() / per_wave[:, 2].double()).median()) * P.REALTIME_HZ / 1e9
    fl = 4 * nb * iters * P.MFMA_PER_ITER * P.FLOP_PER_MFMA
    tf = fl / (ms * 1e-3) / 1e12
    res["mfma_bf16"] = {"tflops": round(tf, 1), "frac_of_nominal": round(tf / PEAK_BF16_TFLOPS, 4),
                        "clock_ghz": round(ghz, 3), "ms": round(ms, 4), "waves": 4 * nb,
                        "note": "v_mfma_f32_32x32x16_bf16 back to back on registers; the nominal peak assumes 2.4 GHz"}

    # compute-only replica of the attention tile, 2 waves per SIMD as the
    # attention kernels run: the cycles a tile's arithmetic needs with no LDS,
    # memory traffic or masking
    tiles = 500
    to = torch.zeros(16 * nb, dtype=i32, device=dev)
    P.tile(tiles, nb, to)
    torch.cuda.synchronize()
    ms = _event_ms(torch, lambda: P.tile(tiles, nb, to), 5)
    per_wave = _u32(to).view(-1, 4)
    cyc = per_wave[:, 1].double() / tiles
    ghz = float((per_wave[:, 1].double() / per_wave[:, 2].double()).median()) * P.REALTIME_HZ / 1e9
    fl = 4 * nb * tiles * P.MFMA_PER_TILE * P.FLOP_PER_MFMA
    tf = fl / (ms * 1e-3) / 1e12
    res["attention_tile_replica"] = {
        "cycles_per_tile_p10_50_90": [round(float(cyc.quantile(x)), 1) for x in (0.1, 0.5, 0.9)],
        "tflops": round(tf, 1), "frac_of_nominal": round(tf / PEAK_BF16_TFLOPS, 4), "clock_ghz": round(ghz, 3),
        "ms": round(ms, 4), "waves": 4 * nb,
        "note": "32 MFMAs + the fast-path softmax of one 64x64 tile per wave, operands in registers"}

    # streaming read and copy of 1 GiB (well above the 256 MB last-level cache)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=i32, device=dev)
    best_r, best_c = None, None
    for per_cu in (4, 8, 16, 64):
        nbr = per_cu * cus
        ro = torch.zeros(nbr, dtype=i32, device=dev)
        P.read(src, ro, nbr)
        ms = _event_ms(torch, lambda: P.read(src, ro, nbr), 7)
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best_r is None or gbs > best_r["gbs"]:
            best_r = {"gbs": round(gbs, 1), "frac_of_nominal": round(gbs / PEAK_HBM_GBS, 4), "blocks": nbr,
                      "ms": round(ms, 4)}
    half = nbytes // 2
    a, b = src[: half // 4], src[half // 4:]
    for per_cu in (4, 8, 16, 64):
        nbr = per_cu * cus
        P.copy(a, b, nbr)
        ms = _event_ms(torch, lambda: P.copy(a, b, nbr), 7)
        gbs = 2 * half / (ms * 1e-3) / 1e9
        if best_c is None or gbs > best_c["gbs"]:
            best_c = {"gbs": round(gbs, 1), "frac_of_nominal": round(gbs / PEAK_HBM_GBS, 4), "blocks": nbr,
                      "ms": round(ms, 4), "bytes_counted": "read + write"}
    res["hbm_read"] = best_r
    res["hbm_copy"] = best_c
    del src, a, b
    return res


def bench_decode(args, torch, ssa, W, shared=False):
    """One decode step = scores, top-k, attention over the selected blocks;
    ``shared`` uses the group-shared selection (then scores and top-k are one
    fused launch)."""
    w = W.DECODE_32K
    dev = torch.device("cuda:0")
    q0, k0, v0 = W.make_inputs(w)
    copies = []
    for c in range(args.decode_copies):      # distinct buffers defeat the 256 MB last-level cache
        q, k, v = q0.to(dev), k0.to(dev), v0.to(dev)
        ks = ssa.ssa_block_summaries(k, block=w.block)   # cached summaries (untimed, as in decoding)
        copies.append((q, k, v, ks))
    del q0, k0, v0
    shape = ssa.make_shape(copies[0][0], w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nkb = ssa.n_blocks(w.seq_kv, w.block)
    scores = torch.empty((w.batch, w.n_q_heads, 1, nkb), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_kv_heads if shared else w.n_q_heads, 1, w.topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(copies[0][0])
    lse = torch.empty((w.batch, w.n_q_heads, 1), dtype=torch.float32, device=dev)
    ws = torch.empty((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=dev)
    timer = KernelTimer(torch)

    def step(t, c):
        q, k, v, ks = copies[c % len(copies)]
        if shared:
            # one ranked row per KV group: scores and selection in one launch
            # (the scores are still written out)
            t.run("decode_scores_select", ssa.ssa_decode_scores_select, shape, q, ks, scores=scores, idx=idx,
                  shared=True)
        else:
            # per-head rows: the separate launches spread the fp64 scoring and
            # the 2048 selections over every compute unit
            t.run("decode_scores", ssa.ssa_block_scores, shape, q, None, ks, scores=scores)
            t.run("decode_topk", ssa.ssa_select_topk, shape, scores, idx)
        t.run("decode_attn", ssa.ssa_block_sparse_attn_fwd, shape, q, k, v, idx, workspace=ws, out=out, lse=lse,
              shared=shared)

    plain = PlainRunner()
    for i in range(args.warmup):
        step(plain, i)
    ms_step, _ = timed_steps(torch, step, args.decode_steps)
    kernel_pass(torch, timer, step, args.decode_steps)
    # Algorithmic bytes from the GPU's own selection (identical inputs in every copy):
    # the union over the query heads of each KV group of selected K and V blocks.
    G = 1 if shared else w.n_q_heads // w.n_kv_heads
    sel = torch.zeros((w.batch, w.n_kv_heads, nkb + 1), dtype=torch.bool, device=dev)
    ii = idx.view(w.batch, w.n_kv_heads, G * w.topk).long()
    sel.scatter_(2, torch.where(ii < 0, torch.full_like(ii, nkb), ii), True)
    union_blocks = int(sel[..., :nkb].sum())
    kv_bytes = union_blocks * w.block * w.head_dim * 2 * 2
    attn_bytes = kv_bytes + copies[0][0].numel() * 2 * 2 + idx.numel() * 4 + lse.numel() * 4
    # summaries and queries read, scores written; the selection reads the scores and writes the indices
    score_bytes = copies[0][3].numel() * 4 + copies[0][0].numel() * 2 + scores.numel() * 4
    topk_bytes = scores.numel() * 4 + idx.numel() * 4
    select_bytes = score_bytes + idx.numel() * 4
    legs = ((("decode_scores_select", select_bytes),) if shared else
            (("decode_scores", score_bytes), ("decode_topk", topk_bytes)))
    kern = {}
    for name, b in legs + (("decode_attn", attn_bytes),):
        ms = timer.median_ms(name)
        gbs = b / (ms * 1e-3) / 1e9
        kern[name] = {"median_ms": round(ms, 5), "mean_ms": round(timer.avg_ms(name), 5), "bound": "hbm",
                      "mbytes_per_launch": round(b / 1e6, 3),
                      "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    step_bytes = attn_bytes + (select_bytes if shared else score_bytes + topk_bytes)
    return {
        "workload": w.name, "tokens_per_s": round(w.batch / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 5),
        "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "union_blocks_per_group": round(union_blocks / (w.batch * w.n_kv_heads), 2),
        "kernels": kern,
        "roofline": {"kernel": "decode_attn", "bound": "hbm", "achieved": kern["decode_attn"]["gbs"],
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": kern["decode_attn"]["frac_of_peak"],
                     "algorithmic_per_launch": attn_bytes,
                     # counters were taken on the per-head selection (a different union)
                     "traffic": None if shared else measured_traffic("decode_attn")},
        "cache_copies_rotated": len(copies), "steps": args.decode_steps,
    }


def bench_early_stop(args, torch, ssa, W, taus=(0.05, 1.0)):
    """Block-sparse forward with early stopping on the bench workload, for a
    few thresholds: time, blocks visited per query block, and the useful
    (visited, unmasked) work rate."""
    w = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    scores, _ = ssa.ssa_block_scores(shape, q, k)
    idx = ssa.ssa_select_topk(shape, scores)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    nqb = ssa.n_blocks(w.seq_q, w.block)
    used = torch.empty((w.batch, w.n_q_heads, nqb), dtype=torch.int32, device=dev)
    listed = float((idx >= 0).sum(-1).float().mean())
    res = {"workload": w.name, "blocks_listed_per_query_block": round(listed, 3), "thresholds": {}}
    n = max(1, args.steps // 2)
    for tau in taus:
        for _ in range(3):
            ssa.ssa_block_sparse_attn_fwd_early_stop(shape, q, k, v, scores, idx, tau, out, lse, used)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            ssa.ssa_block_sparse_attn_fwd_early_stop(shape, q, k, v, scores, idx, tau, out, lse, used)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        # useful pairs: the diagonal block's causal half plus every other visited block
        # (every query block of this workload is complete)
        u = used.double()
        pairs = float((w.block * (w.block + 1) / 2 + (u - 1).clamp(min=0) * w.block * w.block).sum())
        tf = 4.0 * w.head_dim * pairs / (ms * 1e-3) / 1e12
        res["thresholds"][str(tau)] = {"avg_ms": round(ms, 5), "blocks_visited_per_query_block": round(float(u.mean()), 3),
                                       "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    return res


def bench_backward(args, torch, ssa, W):
    """Backward of the block-sparse forward and of the full counterpart on the
    bench workload, for a synthetic output gradient: time per call (all its
    kernels) and the useful rate, counting 5 products of 2*d flops per
    attended (query row, key) pair (score recomputation, dP, dV, dQ, dK)."""
    w = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nqb = ssa.n_blocks(w.seq_q, w.block)
    if w.full_rows is None:
        fb0, fcnt = 0, nqb
    else:
        fb0 = w.full_rows[0] // w.block
        fcnt = ssa.n_blocks(w.full_rows[1], w.block) - fb0
    rows = (fb0 * w.block, min(w.seq_q, (fb0 + fcnt) * w.block))
    scores, _ = ssa.ssa_block_scores(shape, q, k)
    idx = ssa.ssa_select_topk(shape, scores)
    o, lse = ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx)
    of, lf, _ = ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, fb0, fcnt)
    dout = W.make_output_grad(w, device=dev)
    dout_f = W.make_output_grad(w, rows, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_f = torch.empty_like(dout_f)
    ws = torch.empty((max(ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_BWD),
                          ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_FULL_BWD)),), dtype=torch.uint8, device=dev)
    calls = {
        "sparse": lambda: ssa.ssa_block_sparse_attn_bwd(shape, q, k, v, idx, o, lse, dout, dq, dk, dv, ws),
        "full": lambda: ssa.ssa_full_attn_bwd(shape, q, k, v, of, lf, dout_f, fb0, fcnt, dq_f, dk, dv, ws),
    }
    pairs = {"sparse": w.batch * w.n_q_heads * sparse_useful_pairs(nqb, w.topk, w.block),
             "full": w.batch * w.n_q_heads * full_useful_pairs(*rows)}
    res = {"workload": w.name, "flops_per_pair": 10 * w.head_dim}
    n = max(1, args.steps // 2)
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        gf = 10.0 * w.head_dim * pairs[name] / 1e9
        tf = gf / (ms * 1e-3) / 1e3
        res[name] = {"avg_ms": round(ms, 5), "gflop_per_call": round(gf, 3), "tflops": round(tf, 2),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    return res


def bench_dash(args, torch, ssa, W, alpha=1.5, gamma=800.0, sigma=1.0, cap=64):
    """DashAttention-style stages on the bench workload with a synthetic learned
    query: learned-query summaries, scores against them, alpha-entmax routing
    (group-shared support, capped at ``cap`` blocks), prior-biased block-sparse
    forward.  Time per stage (HIP events), list length, useful attention rate."""
    w = W.BY_NAME[args.workload].scaled(topk=cap)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    qbar = W.make_learned_query(w, device=dev)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nqb, nkb = ssa.n_blocks(w.seq_q, w.block), ssa.n_blocks(w.seq_kv, w.block)
    ks = torch.empty((w.batch, w.n_kv_heads, nkb, w.head_dim), dtype=torch.float32, device=dev)
    scores = torch.empty((w.batch, w.n_q_heads, nqb, nkb), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_kv_heads, nqb, w.topk), dtype=torch.int32, device=dev)
    bias = torch.empty((w.batch, w.n_kv_heads, nqb, w.topk), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    timer = KernelTimer(torch)

    def step(t, i=0):
        t.run("summaries", ssa.ssa_block_summaries_learned, k, qbar, out=ks)
        t.run("scores", ssa.ssa_block_scores, shape, q, None, ks, scores=scores)
        t.run("route", ssa.ssa_entmax_route, shape, scores, alpha, gamma, sigma, idx, bias, None, False)
        t.run("attn", ssa.ssa_block_sparse_attn_fwd_biased, shape, q, k, v, idx, bias, out, lse)

    plain = PlainRunner()
    for i in range(3):
        step(plain, i)
    n = max(1, args.steps // 2)
    ms, _ = timed_steps(torch, step, n)
    kernel_pass(torch, timer, step, n)
    # useful pairs: every listed block whole, the diagonal block's causal half
    listed = (idx >= 0).sum(-1).double()                       # [b, Hkv, nqb]
    pairs = float(((listed - 1) * w.block * w.block + w.block * (w.block + 1) / 2).sum()) * (w.n_q_heads // w.n_kv_heads)
    attn_ms = timer.median_ms("attn")
    tf = 4.0 * w.head_dim * pairs / (attn_ms * 1e-3) / 1e12
    return {"workload": w.name, "alpha": alpha, "gamma": gamma, "sigma": sigma, "list_cap": cap,
            "blocks_listed_per_query_block": round(float(listed.mean()), 3), "ms_per_step": round(ms, 5),
            "tokens_per_s": round(w.batch * w.seq_q / (ms * 1e-3), 1),
            "kernels_median_ms": {kk: round(timer.median_ms(kk), 5) for kk in ("summaries", "scores", "route", "attn")},
            "attn_tflops": round(tf, 2), "attn_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def bench_trace(args, torch, ssa, W, workloads=("prefill_8k", "structured_8k")):
    """One launch each of the block-sparse and the full forward with per-workgroup
    timing records (workspace past the work queue): the shader clock each
    workgroup ran at, how evenly the persistent workgroups finished, and the
    rate against the matrix peak at the measured clock."""
    from block_sparse_attention_kv_amd.profiling import TRACE_WORDS, trace_summary
    dev = torch.device("cuda:0")
    res = {}
    for name in workloads:
        w = W.BY_NAME[name]
        q, k, v = (t.to(dev) for t in W.make_inputs(w))
        shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
        nqb = ssa.n_blocks(w.seq_q, w.block)
        fb0 = 0 if w.full_rows is None else w.full_rows[0] // w.block
        fcnt = nqb - fb0
        scores, _ = ssa.ssa_block_scores(shape, q, k)
        idx = ssa.ssa_select_topk(shape, scores)
        qbytes = ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD)
        cap = 8192
        ws = torch.zeros((qbytes + cap * TRACE_WORDS * 4,), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        rows = fcnt * w.block
        of = torch.empty((w.batch, w.n_q_heads, rows, w.head_dim), dtype=torch.bfloat16, device=dev)
        lf = torch.empty((w.batch, w.n_q_heads, rows), dtype=torch.float32, device=dev)
        dm = torch.empty_like(lf)
        pairs_sp = w.batch * w.n_q_heads * sparse_useful_pairs(nqb, w.topk, w.block)
        pairs_full = w.batch * w.n_q_heads * full_useful_pairs(fb0 * w.block, fb0 * w.block + rows)
        calls = {
            "sparse_attn": (lambda: ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws, out=out, lse=lse),
                            4.0 * w.head_dim * pairs_sp),
            "full_attn": (lambda: ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, fb0, fcnt, out=of, lse=lf,
                                                                     dropped=dm, workspace=ws),
                          4.0 * w.head_dim * pairs_full),
        }
        res[name] = {}
        for kname, (fn, fl) in calls.items():
            for _ in range(4):          # the last launch's records are kept
                fn()
            torch.cuda.synchronize()
            recs = ws[qbytes:].view(torch.int32).cpu().numpy().view("uint32")
            res[name][kname] = trace_summary(recs, fl, PEAK_BF16_TFLOPS)
            ws[qbytes:].zero_()
        del q, k, v, scores, idx, ws, out, lse, of, lf, dm
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_decode_baseline(args, W, seconds):
    """The fp64 oracle on whole sequences of the decode workload (scores, top-k
    and attention, cached summaries computed outside the timing), until about
    ``seconds`` elapse."""
    from oracle import ssa_oracle as O
    w = W.DECODE_32K
    q, k, v = W.make_inputs(w)
    seqs, spent = 0, 0.0
    while seqs < w.batch and spent < seconds:
        qs, ks, vs = (t[seqs:seqs + 1].double().numpy() for t in (q, k, v))
        ksum = O.key_summaries(ks, w.block)
        t0 = time.perf_counter()
        O.hot_path(qs, ks, vs, w.block, w.topk, q_offset=w.q_offset, k_summary=ksum, with_full=False)
        spent += time.perf_counter() - t0
        seqs += 1
    return {"value": round(seqs / spent, 3), "unit": "tokens/s", "kind": "oracle",
            "sample": f"{seqs} of {w.batch} sequences of {w.name} (1 token each against {w.seq_kv} keys): "
                      f"scores+top-k+sparse attention in fp64 NumPy ({spent:.1f} s)"}


def cpu_baseline(args, W):
    """The fp64 oracle, as it stands, on a bounded sample of the prefill workload:
    whole query heads (all rows, all five steps) until ~target seconds elapse."""
    import numpy as np
    from oracle import ssa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    affinity = len(os.sched_getaffinity(0))
    w = W.BY_NAME[args.workload]
    q, k, v = W.make_inputs(w)
    G = w.n_q_heads // w.n_kv_heads
    t0 = time.perf_counter()
    heads = 0
    while heads < w.n_q_heads:
        h = heads
        g = h // G
        qh = q[:1, h:h + 1].double().numpy()
        kh = k[:1, g:g + 1].double().numpy()
        vh = v[:1, g:g + 1].double().numpy()
        O.hot_path(qh, kh, vh, w.block, w.topk, full_row_range=w.full_rows)
        heads += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    tokens = w.seq_q * heads / w.n_q_heads   # fraction of one batch row's work
    return {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": affinity, "kind": "oracle",
            "cpu_model": _cpu_model(), "affinity_cpus": affinity, "blas_threads": blas_threads,
            "sample": f"{heads} of {w.n_q_heads} query heads of batch row 0 of {w.name}, all {w.seq_q} rows, "
                      f"summaries+scores+top-k+sparse+full+dropped mass in fp64 NumPy ({dt:.1f} s; "
                      f"matrix products on {blas_threads} BLAS threads, elementwise ops on one); "
                      f"tokens/s scaled by the head fraction",
            "decode": None if args.no_decode else cpu_decode_baseline(args, W, args.cpu_seconds / 2)}


def counter_pass(args, torch, ssa, W):
    """Dispatches for a rocprofv3 --pmc run: a plain copy of known size (the
    counter calibration), then the prefill and decode attention kernels."""
    from block_sparse_attention_kv_amd.profiling import COPY_BYTES
    dev = torch.device("cuda:0")
    src = torch.empty((COPY_BYTES // 2,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    args.warmup, args.steps, args.decode_steps, args.decode_copies = 0, 3, 3, 1
    bench_prefill(args, torch, ssa, W)
    bench_decode(args, torch, ssa, W)
    torch.cuda.synchronize()
    print("counter pass done", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_8k")
    ap.add_argument("--decode-steps", type=int, default=60)
    ap.add_argument("--decode-copies", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the extra legs (group-shared selection, early stopping, DashAttention stages)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the other prefill workloads (structured_8k, structured_8k_tie, extrap_32k)")
    ap.add_argument("--leg-steps", type=int, default=10)
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peaks leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--counter-pass", action="store_true",
                    help="only issue the dispatches a rocprofv3 --pmc run needs (no JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard over sequences and KV heads with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_kv_amd import ssa
    from block_sparse_attention_kv_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (there is no CPU fallback)", file=sys.stderr)
        sys.exit(1)
    ssa.load_library()
    if args.counter_pass:
        counter_pass(args, torch, ssa, W)
        return

    pre = bench_prefill(args, torch, ssa, W)
    dec = None if args.no_decode else bench_decode(args, torch, ssa, W)
    shared = None
    if not args.no_shared:
        # the same steps with the group-shared selection (one list per KV group)
        sp = bench_prefill(args, torch, ssa, W, shared=True)
        shared = {"prefill": {"workload": sp["w"].name, "ms_per_step": round(sp["ms_step"], 5),
                              "tokens_per_s": round(sp["tokens_per_s"], 1), "kernels": sp["kernels"]}}
        if not args.no_decode:
            sd = bench_decode(args, torch, ssa, W, shared=True)
            shared["decode"] = {k2: sd[k2] for k2 in ("workload", "tokens_per_s", "ms_per_step",
                                                       "union_blocks_per_group", "kernels", "roofline")}
    legs = None
    if not args.no_legs:
        legs = {}
        for name in ("structured_8k", "structured_8k_tie", "extrap_32k"):
            legs[name] = prefill_leg(bench_prefill(args, torch, ssa, W, workload=name, steps=args.leg_steps))
    peaks = None if args.no_peaks else bench_peaks(args, torch, ssa, W)
    trace = None if args.no_peaks else bench_trace(args, torch, ssa, W)
    if peaks is not None and trace is not None:
        # each kernel's median tile-loop cycles against the compute-only replica's
        rep = peaks["attention_tile_replica"]["cycles_per_tile_p10_50_90"][1]
        for per_kernel in trace.values():
            for tr in per_kernel.values():
                tr["replica_over_loop_cycles_per_tile"] = round(rep / tr["loop_cycles_per_tile_p10_50_90"][1], 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, W)
    w = pre["w"]
    line = {
        "metric": "block-sparse attn fwd tokens/s + % bf16 MFMA peak at N=8k; decode HBM GB/s",
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V cast to bf16)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "seq_len": w.seq_q, "head_dim": w.head_dim, "block": w.block, "topk": w.topk,
                   "step": "summaries+scores, top-k, block-sparse fwd, full fwd + dropped mass"},
        "roofline": pre["roofline"],
        "roofline_full": pre["roofline_full"],
        "kernels": pre["kernels"],
        "sparse_fwd": {"tokens_per_s": round(w.batch * w.seq_q / (pre["kernels"]["sparse_attn"]["median_ms"] * 1e-3), 1),
                       "tflops": pre["kernels"]["sparse_attn"]["tflops"],
                       "frac_of_bf16_peak": pre["kernels"]["sparse_attn"]["frac_of_peak"],
                       "traffic": measured_traffic("sparse_attn")},
        "targets": {"sparse_fwd_frac_of_bf16_peak": pre["kernels"]["sparse_attn"]["frac_of_peak"],
                    "decode_step_frac_of_hbm_peak": None if dec is None else dec["step_frac_of_hbm_peak"]},
        "decode": dec,
        "workload_legs": legs,
        "peaks": peaks,
        "workgroup_trace": trace,
        "shared_selection": shared,
        "early_stop": None if args.no_shared else bench_early_stop(args, torch, ssa, W),
        "backward": None if args.no_backward else bench_backward(args, torch, ssa, W),
        "dash": None if args.no_shared else bench_dash(args, torch, ssa, W),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
