"""Host logic of the rocprofv3 summaries (block_sparse_attention_kv_amd.profiling)
on small synthetic CSV directories: kernel-name classification, the trace
tables, the copy-calibrated HBM traffic, and the matrix-core busy fraction."""
import csv
import json
import os

import pytest

from block_sparse_attention_kv_amd import profiling as P

SPARSE = "ssa::(anonymous namespace)::attn_sparse_kernel<false>(ssa::AttnArgs, ssa::Geometry)"
FULL = "void ssa::(anonymous namespace)::attn_group_kernel<4, true, false>(ssa::AttnArgs, ssa::Geometry)"
DKV = "void ssa::(anonymous namespace)::attn_bwd_dkv_kernel<1, 2>(ssa::BwdArgs, ssa::Geometry)"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=header)
        w.writeheader()
        for r in rows:
            w.writerow(r)


@pytest.mark.parametrize("name,cls", [
    (SPARSE, "sparse_attn"),
    ("ssa::(anonymous namespace)::attn_sparse_kernel<true>(ssa::AttnArgs, ssa::Geometry)", "sparse_attn_biased"),
    (FULL, "full_attn"),
    ("void ssa::(anonymous namespace)::attn_group_kernel<4, false, false>(ssa::AttnArgs)", "sparse_attn_shared"),
    ("void ssa::(anonymous namespace)::attn_group_kernel<4, false, true>(ssa::AttnArgs)", "sparse_attn_biased"),
    ("_ZN3ssa12_GLOBAL__N_117attn_group_kernelILi4ELb1ELb0EEEvNS_8AttnArgsENS_8GeometryE", "full_attn"),
    ("_ZN3ssa12_GLOBAL__N_117attn_group_kernelILi4ELb0ELb0EEEvNS_8AttnArgsENS_8GeometryE", "sparse_attn_shared"),
    ("ssa::(anonymous namespace)::attn_sparse_early_stop_kernel(ssa::AttnArgs)", "sparse_attn_early_stop"),
    ("void ssa::(anonymous namespace)::attn_decode_partial_kernel<1>(ssa::AttnArgs, float*)", "decode_attn"),
    (DKV, "bwd_dkv"),
    ("ssa::(anonymous namespace)::bwd_pair_scan_kernel(ssa::BwdArgs, ssa::Geometry)", "bwd_pair_scan"),
    (COPY, "copy"),
    ("void at::native::vectorized_elementwise_kernel<4>", None),
])
def test_classify(name, cls):
    assert P.classify(name) == cls


def test_stats_and_shapes(tmp_path):
    d = str(tmp_path / "trace")
    _write_csv(os.path.join(d, "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [{"Name": FULL, "Calls": 2, "TotalDurationNs": 600000, "AverageNs": 300000, "Percentage": 75.0,
                 "MinNs": 290000, "MaxNs": 310000},
                {"Name": DKV, "Calls": 3, "TotalDurationNs": 200000, "AverageNs": 66666.7, "Percentage": 25.0,
                 "MinNs": 10000, "MaxNs": 120000}])
    trace_rows = []
    for k, (name, grid, wg, dur) in enumerate([(FULL, 1024 * 256, 256, 290000), (FULL, 1024 * 256, 256, 310000),
                                               (DKV, 100 * 128, 128, 10000), (DKV, 100 * 128, 128, 70000),
                                               (DKV, 50 * 256, 256, 120000)]):
        trace_rows.append({"Kernel_Name": name, "Start_Timestamp": 1000 * k, "End_Timestamp": 1000 * k + dur,
                           "Workgroup_Size_X": wg, "Grid_Size_X": grid})
    _write_csv(os.path.join(d, "run_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"], trace_rows)
    md = P.stats_markdown(d, title="t", command="rocprofv3 ...")
    assert "| full_attn | 2 | 300.00 | 290.00 | 310.00 | 75.00 |" in md
    # one row per launch shape; durations averaged per shape
    assert "| bwd_dkv | 100 x 128 | 2 | 40.00 | 40.00 | 10.00 | 70.00 |" in md
    assert "| bwd_dkv | 50 x 256 | 1 | 120.00 | 120.00 | 120.00 | 120.00 |" in md
    assert "| full_attn | 1024 x 256 | 2 | 300.00 | 300.00 | 290.00 | 310.00 |" in md


def _counter_rows(counter, values):
    """values: [(kernel name, dispatch id, value)], each split over two
    per-dimension rows as rocprofv3 may report them."""
    rows = []
    for name, disp, v in values:
        for half in (0.25, 0.75):
            rows.append({"Kernel_Name": name, "Dispatch_Id": disp, "Counter_Name": counter,
                         "Counter_Value": v * half, "Start_Timestamp": 0, "End_Timestamp": 1000})
    return rows


def test_traffic_calibration(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    # the copy moves COPY_BYTES/2 each way; its counters read half of that on
    # fetch (factor 2) and exactly it on write (factor 1)
    copy_kib = P.COPY_BYTES / 2 / 1024
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    _write_csv(os.path.join(fd, "x_counter_collection.csv"), hdr,
               _counter_rows("FETCH_SIZE", [(COPY, 1, copy_kib / 2), (SPARSE, 2, 1000.0), (SPARSE, 3, 3000.0)]))
    _write_csv(os.path.join(wd, "x_counter_collection.csv"), hdr,
               _counter_rows("WRITE_SIZE", [(COPY, 1, copy_kib), (SPARSE, 2, 10.0), (SPARSE, 3, 30.0)]))
    out = str(tmp_path / "traffic.json")
    res = P.traffic(fd, wd, out, command="c")
    assert res["_f_scale"] == pytest.approx(2.0)
    assert res["_w_scale"] == pytest.approx(1.0)
    e = res["sparse_attn"]
    assert e["dispatches"] == 2
    assert e["fetch_kib_per_dispatch"] == pytest.approx(2000.0)
    assert e["bytes_per_launch"] == round(2000.0 * 1024 * 2 + 20.0 * 1024)
    assert e["source_sha256_16"] == P.source_hash("sparse_attn")
    with open(out) as f:
        assert json.load(f)["sparse_attn"]["bytes_per_launch"] == e["bytes_per_launch"]


def test_traffic_needs_calibration(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    _write_csv(os.path.join(fd, "x_counter_collection.csv"), hdr, _counter_rows("FETCH_SIZE", [(SPARSE, 2, 1.0)]))
    _write_csv(os.path.join(wd, "x_counter_collection.csv"), hdr, _counter_rows("WRITE_SIZE", [(SPARSE, 2, 1.0)]))
    with pytest.raises(SystemExit):
        P.traffic(fd, wd, str(tmp_path / "t.json"))


def test_mfma_busy_fraction(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    # 2000 active cycles on each of the 8 dies over a 1000 ns dispatch (2 GHz);
    # the matrix cores of all SIMDs busy for a quarter of them
    gui = 2000.0 * P.XCD_NUM
    busy = 0.25 * 2000.0 * P.SIMD_NUM
    rows = []
    for ctr, v in (("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                   ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6), ("SQ_INSTS_MFMA", 2e6), ("SQ_INSTS_VALU", 2.2e7)):
        rows += _counter_rows(ctr, [(FULL, 7, v)])
    d = str(tmp_path / "m")
    _write_csv(os.path.join(d, "x_counter_collection.csv"), hdr, rows)
    md = P.mfma_markdown(d)
    assert "| full_attn | 1 | 25.0 | 0.51 | 2.000 | 11.00 |" in md


def test_trace_summary_hand_case():
    """Two workgroup records (third row unused): clock = cycles / ticks x 0.1 GHz,
    span from the earliest start to the latest end, busy fraction = summed
    busy time / (workgroups x span)."""
    import numpy as np
    from block_sparse_attention_kv_amd.profiling import trace_summary
    r = np.zeros((3, 8), dtype=np.uint32)
    # ticks of 10 ns: wg0 runs 0..1000 (10 us), wg1 runs 500..1500 (10 us)
    r[0, :6] = [5000, 6000, 20000, 15000, 2, 32]   # 20000 cycles / 10 us = 2.0 GHz
    r[1, :6] = [5500, 6500, 15000, 9000, 1, 16]    # 15000 cycles / 10 us = 1.5 GHz
    s = trace_summary(r, flops=1e9, peak_tflops=1000.0, nominal_ghz=2.0)
    assert s["workgroups"] == 2 and s["units"] == 3 and s["tiles"] == 48
    assert s["span_us"] == 15.0
    assert s["clock_ghz_p0_10_50_90_100"][0] == 1.5 and s["clock_ghz_p0_10_50_90_100"][-1] == 2.0
    assert abs(s["busy_fraction"] - 20.0 / 30.0) < 1e-4
    assert abs(s["loop_fraction_of_cycles"] - 24000 / 35000) < 1e-4
    # 1e9 flop over 15 us = 66.67 TFLOP/s; peak at the median clock 1.75 GHz = 875 TFLOP/s
    assert abs(s["tflops_over_span"] - 66.67) < 0.01
    assert abs(s["frac_of_peak_at_measured_clock"] - 66.6667 / 875.0) < 1e-4


def test_trace_summary_wraps_the_tick_counter():
    import numpy as np
    from block_sparse_attention_kv_amd.profiling import trace_summary
    r = np.zeros((1, 8), dtype=np.uint32)
    r[0, :6] = [0xFFFFFF00, 0x00000100, 1024 * 16, 0, 1, 1]   # 512 ticks across the wrap
    s = trace_summary(r)
    assert s["span_us"] == 5.12
    assert abs(s["clock_ghz_p0_10_50_90_100"][2] - 3.2) < 1e-6


def test_valu_mix_and_lds_summaries(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    vals = {"SQ_INSTS_VALU_TRANS_F32": 4e6, "SQ_INSTS_VALU_FMA_F32": 4e6, "SQ_INSTS_VALU_ADD_F32": 3e6,
            "SQ_INSTS_VALU_MUL_F32": 1e6, "SQ_INSTS_VALU_CVT": 2e6, "SQ_INSTS_SALU": 5e5, "SQ_INSTS_LDS": 1e6,
            "SQ_INSTS_MFMA": 2e6}
    rows = []
    for ctr, v in vals.items():
        rows += _counter_rows(ctr, [(FULL, 7, v)])
    d = str(tmp_path / "v")
    _write_csv(os.path.join(d, "x_counter_collection.csv"), hdr, rows)
    md = P.valu_mix_markdown(d)
    assert "| full_attn | 1 | 2.000 | 2.00 | 2.00 | 1.50 | 0.50 | 1.00 | 0.25 | 0.50 |" in md
    rows = []
    for ctr, v in (("SQ_LDS_BANK_CONFLICT", 50.0), ("SQ_LDS_IDX_ACTIVE", 1000.0), ("SQ_INSTS_LDS", 2e6)):
        rows += _counter_rows(ctr, [(FULL, 7, v)])
    d2 = str(tmp_path / "l")
    _write_csv(os.path.join(d2, "x_counter_collection.csv"), hdr, rows)
    assert "| full_attn | 1 | 50 | 1000 | 0.0500 | 2.000 |" in P.lds_markdown(d2)


def test_workgroup_trace_markdown_with_replica(tmp_path):
    """The summary of a bench line carries the measured peaks, the attention-tile
    replica and each traced kernel's replica-to-loop cycle ratio."""
    trace = {"workgroups": 2, "span_us": 15.0, "clock_ghz_p0_10_50_90_100": [1.5, 1.5, 1.75, 2.0, 2.0],
             "busy_fraction": 0.6667, "end_us_p0_10_50_90_100": [10.0, 10.0, 12.5, 15.0, 15.0],
             "tiles_per_workgroup_p0_50_100": [16, 24, 32], "loop_cycles_per_tile_p10_50_90": [1500.0, 2000.0, 2500.0],
             "tflops_over_span": 66.67, "frac_of_peak_at_measured_clock": 0.0762,
             "replica_over_loop_cycles_per_tile": 0.75}
    line = {"metric": "m", "value": 1.0,
            "peaks": {"clock_idle_ghz": 2.4,
                      "mfma_bf16": {"tflops": 1858.0, "clock_ghz": 1.93, "frac_of_nominal": 0.738},
                      "attention_tile_replica": {"cycles_per_tile_p10_50_90": [1400.0, 1500.0, 3000.0],
                                                 "tflops": 900.0, "clock_ghz": 2.1, "frac_of_nominal": 0.3576},
                      "hbm_read": {"gbs": 5830.0, "frac_of_nominal": 0.7288},
                      "hbm_copy": {"gbs": 5160.0, "frac_of_nominal": 0.645}},
            "workgroup_trace": {"prefill_8k": {"sparse_attn": trace}}}
    log = tmp_path / "bench.log"
    log.write_text("noise\n" + json.dumps(line) + "\n")
    md = P.workgroup_trace_markdown(str(log), title="t", command="c")
    assert "1400.0 / 1500.0 / 3000.0 cycles per tile" in md
    assert "| prefill_8k | sparse_attn | 2 |" in md
    assert md.rstrip().endswith("| 0.0762 | 0.75 |")


def test_bench_comparison_with_default_run(tmp_path):
    def line(sp, fu, de):
        k = lambda ms: {"median_ms": ms, "mean_ms": ms * 1.05}
        return json.dumps({"kernels": {"sparse_attn": k(sp), "full_attn": k(fu)},
                           "decode": {"kernels": {"decode_attn": k(de)}}})
    prof, ref = tmp_path / "prof.log", tmp_path / "ref.log"
    prof.write_text("noise\n" + line(0.0979, 0.3187, 0.0954) + "\n")
    ref.write_text(line(0.0897, 0.2982, 0.0749) + "\n")
    md = P.bench_comparison(str(prof), str(ref))
    assert "| sparse_attn | 97.90 | 102.80 | 89.70 |" in md
    assert "| decode_attn (decode_attn + decode_combine) | 95.40 | 100.17 | 74.90 |" in md
    # without a default run: three columns only
    md2 = P.bench_comparison(str(prof))
    assert "| full_attn | 318.70 | 334.63 |" in md2 and "default run |" not in md2
