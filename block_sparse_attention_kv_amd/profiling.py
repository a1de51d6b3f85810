"""Summaries of rocprofv3 output for the kernels of libssa.

  python -m block_sparse_attention_kv_amd.profiling stats <rocprof_dir> [--title T] [--command C]
      -> markdown table of per-kernel dispatch counts and durations (kernel_stats.csv)
  python -m block_sparse_attention_kv_amd.profiling traffic <fetch_dir> <write_dir> --out profiles/traffic.json
      -> HBM bytes per dispatch of the attention kernels from FETCH_SIZE / WRITE_SIZE
         counter runs, scaled by what the same counters read for a plain copy of
         known size (the calibration dispatch in the same run)
  python -m block_sparse_attention_kv_amd.profiling waits <counter_dir> [--title T] [--command C]
      -> markdown table of where the waves' cycles go per kernel (SQ cycle counters)
  python -m block_sparse_attention_kv_amd.profiling mfma <counter_dir> [--title T] [--command C]
      -> markdown table of matrix-core utilisation per kernel from one counter run
         (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_BF16,
         SQ_INSTS_MFMA, SQ_INSTS_VALU)

Kernel names are matched by substring: attn_group_kernel<NW, true> is the
full counterpart, attn_group_kernel<NW, false> the block-sparse forward with a
group-shared selection, attn_sparse_kernel the block-sparse forward, attn_sparse_early_stop_kernel its
early-stopping variant, attn_decode_partial_kernel the decode gather.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

KERNEL_SOURCES = {
    "full_attn": ["ssa_attn.hip", "ssa_tiles.hpp", "ssa_common.hpp", "ssa_internal.hpp"],
    "sparse_attn": ["ssa_attn.hip", "ssa_tiles.hpp", "ssa_common.hpp", "ssa_internal.hpp"],
    "decode_attn": ["ssa_decode.hip", "ssa_tiles.hpp", "ssa_common.hpp", "ssa_internal.hpp"],
}
# calibration copy: bench.py --counter-pass copies this many bytes (read + write) per dispatch
COPY_BYTES = 512 * 1024 * 1024


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def classify(name: str):
    if "attn_group_kernel" in name:
        # attn_group_kernel<NW, FULL, BIAS>: demangled "<4, true, false>", mangled "ILi4ELb1ELb0E"
        m = re.search(r"attn_group_kernel<\s*\d+,\s*(true|false)(?:,\s*(true|false))?", name)
        if m:
            full, bias = m.group(1) == "true", m.group(2) == "true"
        else:
            m = re.search(r"attn_group_kernelILi\d+ELb([01])E(?:Lb([01])E)?", name)
            full, bias = (m.group(1) == "1", m.group(2) == "1") if m else (False, False)
        if full:
            return "full_attn"
        return "sparse_attn_biased" if bias else "sparse_attn_shared"
    if "attn_sparse_kernel" in name and ("<true>" in name or "ILb1E" in name):
        return "sparse_attn_biased"
    if "attn_bwd_dkv_kernel" in name:
        return "bwd_dkv"
    if "attn_bwd_dq_kernel" in name:
        return "bwd_dq"
    if "attn_bwd_reduce_kernel" in name:
        return "bwd_reduce"
    if "bwd_mask_kernel" in name:
        return "bwd_mask"
    if "bwd_count_kernel" in name:
        return "bwd_count"
    if "bwd_pair_scan_kernel" in name:
        return "bwd_pair_scan"
    if "bwd_fill_zero_kernel" in name:
        return "bwd_clear"
    if "attn_sparse_early_stop_kernel" in name:
        return "sparse_attn_early_stop"
    if "attn_sparse_kernel" in name:
        return "sparse_attn"
    if "attn_decode_partial_kernel" in name:
        return "decode_attn"
    if "attn_decode_combine_kernel" in name:
        return "decode_combine"
    if "prefill_scores_kernel" in name:
        return "prefill_scores"
    if "decode_select_kernel" in name:
        return "decode_scores_select"
    if "decode_scores_kernel" in name:
        return "decode_scores"
    if "block_summaries_kernel" in name:
        return "block_summaries"
    if "learned_summaries_kernel" in name:
        return "learned_summaries"
    if "entmax_route_kernel" in name:
        return "entmax_route"
    if "select_topk_shared_kernel" in name:
        return "select_topk_shared"
    if "select_topk_kernel" in name:
        return "select_topk"
    if "copyBuffer" in name:
        return "copy"
    return None


def _csvs(d: str, pattern: str):
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))


def _bench_line(path: str):
    """The JSON line bench.py printed (the last line of the log that parses)."""
    line = None
    with open(path) as f:
        for raw in f:
            raw = raw.strip()
            if raw.startswith("{"):
                try:
                    line = json.loads(raw)
                except ValueError:
                    pass
    return line


def bench_comparison(path: str, ref_path: str = "") -> str:
    """Markdown rows: the same run's HIP-event medians and means from bench.py
    for the kernels the trace also times, and (``ref_path``) the event medians
    of a run of bench.py without the profiler."""
    b = _bench_line(path)
    if not b:
        return ""
    ref = _bench_line(ref_path) if ref_path else None

    def calls(line):
        k = line["kernels"]
        rows = [("sparse_attn", k["sparse_attn"]), ("full_attn", k["full_attn"])]
        if line.get("decode"):
            rows.append(("decode_attn (decode_attn + decode_combine)", line["decode"]["kernels"]["decode_attn"]))
        return rows

    out = ["", "The same run's bench.py HIP-event timings (prefill_8k, decode_32k): each event pair brackets",
           "one call of the event-timed pass, the last of the run's three passes (warm-up, back-to-back",
           "timed steps, event-timed calls).  The trace above covers the dispatches of all three, whose",
           "shader clocks differ by a few percent.  Under the profiler every launch is held for about",
           "10 us (the gaps between consecutive dispatches in the trace), so an event pair whose call",
           "follows a short kernel also times the wait for its own launch: the decode call comes right",
           "after the 6 us selection and reads about 20 us above its two kernels' durations.  The last",
           "column is the same calls in the default bench.py run without the profiler, which the bench",
           "line's rooflines use.", ""]
    if ref:
        rmap = dict(calls(ref))
        out += ["| call | event median us | event mean us | event median us, default run |", "|---|---|---|---|"]
        out += [f"| {n} | {e['median_ms'] * 1e3:.2f} | {e['mean_ms'] * 1e3:.2f} | "
                f"{rmap[n]['median_ms'] * 1e3:.2f} |" for n, e in calls(b) if n in rmap]
    else:
        out += ["| call | event median us | event mean us |", "|---|---|---|"]
        out += [f"| {n} | {e['median_ms'] * 1e3:.2f} | {e['mean_ms'] * 1e3:.2f} |" for n, e in calls(b)]
    return "\n".join(out) + "\n"


SHAPE_KERNELS = ("sparse_attn", "sparse_attn_shared", "full_attn", "decode_attn", "decode_combine", "bwd_dq",
                 "bwd_dkv")


def shape_markdown(d: str) -> str:
    """Per kernel and launch shape (workgroups x threads per workgroup), from
    the per-dispatch trace: a kernel launched at different sizes (the sparse
    and the full dK/dV backward) gets a row per size."""
    files = _csvs(d, "*kernel_trace.csv")
    if not files:
        return ""
    per = defaultdict(list)
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            cls = classify(r.get("Kernel_Name", ""))
            if cls not in SHAPE_KERNELS:
                continue
            wg = int(r.get("Workgroup_Size_X", 1) or 1)
            grid = int(r.get("Grid_Size_X", 0) or 0)
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            per[(cls, grid // max(wg, 1), wg)].append(dur)
    out = ["", "Per launch shape (workgroups x threads per workgroup):", "",
           "| kernel | workgroups x threads | calls | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for (cls, nwg, wg), v in sorted(per.items(), key=lambda kv: (kv[0][0], -kv[0][1])):
        v = sorted(v)
        med = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
        out.append(f"| {cls} | {nwg} x {wg} | {len(v)} | {sum(v) / len(v):.2f} | {med:.2f} | {min(v):.2f} | "
                   f"{max(v):.2f} |")
    return "\n".join(out) + "\n"


def stats_markdown(d: str, title: str = "", command: str = "") -> str:
    files = _csvs(d, "*kernel_stats.csv")
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            rows.append(r)
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    out += ["| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name", "")
        short = classify(name) or name[:60]
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        out.append(f"| {short} | {r.get('Calls')} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {float(r.get('Percentage', 0)):.2f} |")
    return "\n".join(out) + "\n" + shape_markdown(d)


def _counter_per_kernel(d: str, counter: str):
    """kernel class -> list of per-dispatch counter values (summed over the
    per-dimension rows a dispatch may have)."""
    per = defaultdict(lambda: defaultdict(float))
    for fpath in _csvs(d, "*counter_collection.csv"):
        with open(fpath) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                cls = classify(r.get("Kernel_Name", ""))
                if cls is None:
                    continue
                per[cls][r.get("Dispatch_Id")] += float(r.get("Counter_Value", 0))
    return {k: list(v.values()) for k, v in per.items()}


def traffic(fetch_dir: str, write_dir: str, out_json: str, command: str = ""):
    fetch = _counter_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _counter_per_kernel(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("calibration copy dispatch not found in the counter output")
    copy_f = max(fetch["copy"])   # KiB per dispatch
    copy_w = max(write["copy"])
    f_scale = (COPY_BYTES / 2) / (copy_f * 1024.0)   # a copy reads half and writes half of COPY_BYTES
    w_scale = (COPY_BYTES / 2) / (copy_w * 1024.0)
    res = {"_about": "HBM bytes per dispatch = FETCH_SIZE*1024*f_scale + WRITE_SIZE*1024*w_scale; "
                     "scales from a plain copy of known size measured in the same runs",
           "_command": command, "_copy_fetch_kib": copy_f, "_copy_write_kib": copy_w,
           "_f_scale": f_scale, "_w_scale": w_scale}
    for k in ("full_attn", "sparse_attn", "decode_attn"):
        if k not in fetch or k not in write:
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        res[k] = {"fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                  "bytes_per_launch": round(fk * 1024 * f_scale + wk * 1024 * w_scale),
                  "source_sha256_16": source_hash(k), "dispatches": len(fetch[k])}
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    return res


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU")
SIMD_NUM = 256 * 4  # compute units x SIMDs per compute unit
XCD_NUM = 8         # GRBM_GUI_ACTIVE comes summed over the accelerator dies


def _counters_per_dispatch(d: str):
    """kernel class -> dispatch id -> (counter -> summed value, duration ns)."""
    per = defaultdict(dict)
    for fpath in _csvs(d, "*counter_collection.csv"):
        with open(fpath) as f:
            for r in csv.DictReader(f):
                cls = classify(r.get("Kernel_Name", ""))
                if cls is None:
                    continue
                ent = per[cls].setdefault(r.get("Dispatch_Id"), [defaultdict(float), 0.0])
                ent[0][r.get("Counter_Name")] += float(r.get("Counter_Value", 0))
                ent[1] = float(r.get("End_Timestamp", 0)) - float(r.get("Start_Timestamp", 0))
    return per


def mfma_markdown(d: str, title: str = "", command: str = "") -> str:
    """Per kernel, averaged over its dispatches: matrix-core busy fraction
    (busy cycles summed over the SIMDs / (active cycles of one die x SIMDs)),
    executed bf16 matrix flops (MOPS x 512), matrix instructions, and vector
    instructions issued per matrix instruction.  GRBM_GUI_ACTIVE spans the
    counting window, which adds some 20-30 thousand cycles to every dispatch,
    so the busy fraction of a short dispatch reads low; no clock is derived
    from it (the attention launches' own timing records give the clock)."""
    per = _counters_per_dispatch(d)
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    out += ["| kernel | dispatches | matrix-core busy % | executed bf16 GFLOP | MFMA instr (M) | "
            "VALU instr per MFMA instr |",
            "|---|---|---|---|---|---|"]
    for cls in sorted(per):
        util, gflop, nmf, ratio = [], [], [], []
        for ctr, dur in per[cls].values():
            if not all(c in ctr for c in MFMA_COUNTERS) or ctr["SQ_INSTS_MFMA"] <= 0:
                continue
            gui = ctr["GRBM_GUI_ACTIVE"] / XCD_NUM
            if gui <= 0 or dur <= 0:
                continue
            util.append(100.0 * ctr["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM))
            gflop.append(ctr["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9)
            nmf.append(ctr["SQ_INSTS_MFMA"] / 1e6)
            ratio.append(ctr["SQ_INSTS_VALU"] / ctr["SQ_INSTS_MFMA"])
        if not util:
            continue
        avg = lambda v: sum(v) / len(v)
        out.append(f"| {cls} | {len(util)} | {avg(util):.1f} | {avg(gflop):.2f} | {avg(nmf):.3f} | "
                   f"{avg(ratio):.2f} |")
    return "\n".join(out) + "\n"


VALU_MIX_COUNTERS = ("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_ADD_F32",
                     "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_CVT", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA")


def valu_mix_markdown(d: str, title: str = "", command: str = "") -> str:
    """Per kernel, averaged over its dispatches: instructions of each class
    (summed over all waves) per matrix instruction -- transcendental (exp,
    log), fp32 fma, add and mul, conversions, scalar, LDS."""
    per = _counters_per_dispatch(d)
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    cols = VALU_MIX_COUNTERS[:-1]
    out += ["Instructions per v_mfma instruction (wave-level instruction counts):", "",
            "| kernel | dispatches | MFMA instr (M) | " + " | ".join(c.replace("SQ_INSTS_", "") for c in cols) + " |",
            "|---|---|---|" + "---|" * len(cols)]
    for cls in sorted(per):
        rows = [ctr for ctr, _ in per[cls].values()
                if all(c in ctr for c in VALU_MIX_COUNTERS) and ctr["SQ_INSTS_MFMA"] > 0]
        if not rows:
            continue
        avg = lambda f: sum(f(r) for r in rows) / len(rows)
        out.append(f"| {cls} | {len(rows)} | {avg(lambda r: r['SQ_INSTS_MFMA']) / 1e6:.3f} | " +
                   " | ".join(f"{avg(lambda r, c=c: r[c] / r['SQ_INSTS_MFMA']):.2f}" for c in cols) + " |")
    return "\n".join(out) + "\n"


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS")


def lds_markdown(d: str, title: str = "", command: str = "") -> str:
    """Per kernel, averaged over its dispatches: LDS bank-conflict cycles as a
    fraction of the cycles the LDS was indexing, and LDS instructions."""
    per = _counters_per_dispatch(d)
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    out += ["| kernel | dispatches | bank-conflict cycles | LDS active cycles | conflict / active | LDS instr (M) |",
            "|---|---|---|---|---|---|"]
    for cls in sorted(per):
        rows = [ctr for ctr, _ in per[cls].values() if all(c in ctr for c in LDS_COUNTERS)]
        if not rows:
            continue
        avg = lambda c: sum(r[c] for r in rows) / len(rows)
        act = avg("SQ_LDS_IDX_ACTIVE")
        out.append(f"| {cls} | {len(rows)} | {avg('SQ_LDS_BANK_CONFLICT'):.0f} | {act:.0f} | "
                   f"{(avg('SQ_LDS_BANK_CONFLICT') / act if act else 0.0):.4f} | {avg('SQ_INSTS_LDS') / 1e6:.3f} |")
    return "\n".join(out) + "\n"


WAIT_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                 "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY")


def waits_markdown(d: str, title: str = "", command: str = "") -> str:
    """Where the waves' time goes, per kernel: each SQ cycle counter as a
    fraction of SQ_WAVE_CYCLES (all in the same quad-cycle units), averaged
    over the kernel's dispatches."""
    per = _counters_per_dispatch(d)
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    out += ["Fractions of the waves' cycles (SQ_WAVE_CYCLES):", "",
            "| kernel | dispatches | executing any | executing VALU | executing LDS | waiting on a dependency "
            "(SQ_WAIT_ANY) | ready, waiting to issue (SQ_WAIT_INST_ANY) |",
            "|---|---|---|---|---|---|---|"]
    for cls in sorted(per):
        fr = defaultdict(list)
        for ctr, _dur in per[cls].values():
            if not all(c in ctr for c in WAIT_COUNTERS) or ctr["SQ_WAVE_CYCLES"] <= 0:
                continue
            for c in WAIT_COUNTERS[1:]:
                fr[c].append(ctr[c] / ctr["SQ_WAVE_CYCLES"])
        if not fr:
            continue
        avg = lambda v: sum(v) / len(v)
        out.append(f"| {cls} | {len(fr['SQ_WAIT_ANY'])} | " +
                   " | ".join(f"{avg(fr[c]):.3f}" for c in WAIT_COUNTERS[1:]) + " |")
    return "\n".join(out) + "\n"


TRACE_WORDS = 8  # words per workgroup timing record of a persistent attention launch


def trace_summary(records, flops: float = 0.0, peak_tflops: float = 2516.6, nominal_ghz: float = 2.4) -> dict:
    """Summary of the per-workgroup timing records of one persistent launch
    (uint32 [n, 8]: real-time start/end in 10 ns ticks, shader cycles, cycles
    in the tile loops, units, tiles, hardware id, XCC id; unused rows zero).
    The shader clock of a workgroup is its cycles over its real time; with
    ``flops`` the launch's rate is also given against the matrix peak scaled
    to the median measured clock."""
    import numpy as np
    r = np.asarray(records, dtype=np.uint64).reshape(-1, TRACE_WORDS).astype(np.int64)
    r = r[r[:, 4] > 0]
    if len(r) == 0:
        return {}
    rt0, rt1 = r[:, 0], r[:, 1]
    rt1 = np.where(rt1 < rt0, rt1 + (1 << 32), rt1)
    base = rt0.min()
    start_us, end_us = (rt0 - base) * 1e-2, (rt1 - base) * 1e-2
    busy_us = end_us - start_us
    ghz = r[:, 2] / np.maximum(rt1 - rt0, 1) * 0.1
    span = float(end_us.max())
    q = lambda x: [round(float(np.percentile(x, p)), 3) for p in (0, 10, 50, 90, 100)]
    out = {
        "workgroups": int(len(r)),
        "span_us": round(span, 2),
        "start_us_p0_10_50_90_100": q(start_us),
        "end_us_p0_10_50_90_100": q(end_us),
        "clock_ghz_p0_10_50_90_100": q(ghz),
        "busy_fraction": round(float(busy_us.sum() / (len(r) * span)), 4) if span > 0 else None,
        "loop_fraction_of_cycles": round(float(r[:, 3].sum() / max(r[:, 2].sum(), 1)), 4),
        "tiles_per_workgroup_p0_50_100": [int(r[:, 5].min()), int(np.median(r[:, 5])), int(r[:, 5].max())],
        "units": int(r[:, 4].sum()),
        "tiles": int(r[:, 5].sum()),
        "loop_cycles_per_tile_p10_50_90": [round(float(np.percentile(r[:, 3] / np.maximum(r[:, 5], 1), p)), 1)
                                           for p in (10, 50, 90)],
    }
    if flops and span > 0:
        clk = float(np.median(ghz))
        tf = flops / (span * 1e-6) / 1e12
        out["tflops_over_span"] = round(tf, 2)
        out["frac_of_peak_at_measured_clock"] = round(tf / (peak_tflops * clk / nominal_ghz), 4)
    return out


def workgroup_trace_markdown(bench_log: str, title: str = "", command: str = "") -> str:
    """The bench line's measured peaks and per-workgroup timing summaries of
    the persistent attention launches, as tables."""
    b = _bench_line(bench_log)
    if not b:
        raise SystemExit(f"no bench line in {bench_log}")
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    pk = b.get("peaks") or {}
    if pk:
        m, r, c = pk["mfma_bf16"], pk["hbm_read"], pk["hbm_copy"]
        out += ["Measured peaks (libssa_peaks):", "",
                "| quantity | measured | nominal | fraction |", "|---|---|---|---|",
                f"| bf16 32x32x16 matrix loop | {m['tflops']} TFLOP/s at {m['clock_ghz']} GHz | 2516.6 TFLOP/s at 2.4 GHz "
                f"| {m['frac_of_nominal']} |",
                f"| streaming read, 1 GiB | {r['gbs']} GB/s | 8000 GB/s | {r['frac_of_nominal']} |",
                f"| streaming copy, 2 x 512 MiB | {c['gbs']} GB/s | 8000 GB/s | {c['frac_of_nominal']} |",
                f"| shader clock, idle | {pk['clock_idle_ghz']} GHz | 2.4 GHz | |", ""]
        rp = pk.get("attention_tile_replica")
        if rp:
            cy = rp["cycles_per_tile_p10_50_90"]
            out += ["Compute-only replica of the attention tile (32 matrix instructions and the fast-path softmax",
                    "of one 64 x 64 tile per wave, operands in registers, 2 waves per SIMD): "
                    f"{cy[0]} / {cy[1]} / {cy[2]} cycles per tile (p10 / p50 / p90), {rp['tflops']} TFLOP/s at "
                    f"{rp['clock_ghz']} GHz ({rp['frac_of_nominal']} of the nominal peak).", ""]
    tr = b.get("workgroup_trace") or {}
    if tr:
        out += ["One traced launch per kernel (records in the workspace past the work queue).  Clock = a",
                "workgroup's shader cycles over its real time; busy = summed workgroup time over",
                "(workgroups x span); the last column is the launch's useful rate against the bf16 peak",
                "scaled to the median measured clock.", "",
                "| workload | kernel | workgroups | span us | clock GHz p10 / p50 / p90 | busy | end us p50 / max | "
                "tiles per workgroup min / med / max | loop cycles per tile p10 / p50 / p90 | TFLOP/s over span | "
                "fraction of peak at measured clock | replica / loop cycles per tile |",
                "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for wl, ks in tr.items():
            for kn, x in ks.items():
                cg, en = x["clock_ghz_p0_10_50_90_100"], x["end_us_p0_10_50_90_100"]
                out.append(f"| {wl} | {kn} | {x['workgroups']} | {x['span_us']} | {cg[1]} / {cg[2]} / {cg[3]} | "
                           f"{x['busy_fraction']} | {en[2]} / {en[4]} | "
                           f"{' / '.join(str(t) for t in x['tiles_per_workgroup_p0_50_100'])} | "
                           f"{' / '.join(str(t) for t in x['loop_cycles_per_tile_p10_50_90'])} | "
                           f"{x.get('tflops_over_span')} | {x.get('frac_of_peak_at_measured_clock')} | "
                           f"{x.get('replica_over_loop_cycles_per_tile', '')} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", default="")
    s.add_argument("--command", default="")
    s.add_argument("--bench-log", default="", help="output of the profiled bench.py run, for its own timings")
    s.add_argument("--ref-bench-log", default="", help="output of a bench.py run without the profiler")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--out", required=True)
    t.add_argument("--command", default="")
    w = sub.add_parser("waits")
    w.add_argument("dir")
    w.add_argument("--title", default="")
    w.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--title", default="")
    m.add_argument("--command", default="")
    vm = sub.add_parser("valu")
    vm.add_argument("dir")
    vm.add_argument("--title", default="")
    vm.add_argument("--command", default="")
    wt = sub.add_parser("wgtrace")
    wt.add_argument("bench_log")
    wt.add_argument("--title", default="")
    wt.add_argument("--command", default="")
    ld = sub.add_parser("lds")
    ld.add_argument("dir")
    ld.add_argument("--title", default="")
    ld.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats_markdown(a.dir, a.title, a.command))
        if a.bench_log:
            sys.stdout.write(bench_comparison(a.bench_log, a.ref_bench_log))
    elif a.cmd == "mfma":
        sys.stdout.write(mfma_markdown(a.dir, a.title, a.command))
    elif a.cmd == "waits":
        sys.stdout.write(waits_markdown(a.dir, a.title, a.command))
    elif a.cmd == "valu":
        sys.stdout.write(valu_mix_markdown(a.dir, a.title, a.command))
    elif a.cmd == "wgtrace":
        sys.stdout.write(workgroup_trace_markdown(a.bench_log, a.title, a.command))
    elif a.cmd == "lds":
        sys.stdout.write(lds_markdown(a.dir, a.title, a.command))
    else:
        print(json.dumps(traffic(a.fetch_dir, a.write_dir, a.out, a.command), indent=1))


if __name__ == "__main__":
    main()
