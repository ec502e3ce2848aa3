"""Host logic of the rocprofv3 harness and of bench.py's clock figures (no GPU, no profiler):
the timed launches are picked in dispatch order after the warm-up, the clock median keeps
only samples inside bench.py's timed region, and the summary names its commands."""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import attn_inputs  # noqa: E402
import bench  # noqa: E402
from flash_attention_amd import rocprof_harness as rh  # noqa: E402


def _write_trace(d, rows):
    os.makedirs(os.path.join(d, "trace", "host"), exist_ok=True)
    with open(os.path.join(d, "trace", "host", "k_kernel_trace.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for did, name, t0, t1 in rows:
            f.write('%d,"%s",%d,%d\n' % (did, name, t0, t1))


def test_timed_launches_follow_dispatch_order(tmp_path):
    d = str(tmp_path)
    k = "_ZN12_GLOBAL__N_115attn_fwd_kernelILi256ELi0EDF16_Lb0EEEvNS_6ParamsE"
    m = "void (anonymous namespace)::attn_merge_kernel<0, 2>(MergeParams)"
    rows = []
    # rows written out of order; durations 10*id
    for did in (5, 1, 3, 2, 4, 6):
        rows.append((did, k if did % 2 else m, 1000 * did, 1000 * did + 10 * did))
    _write_trace(d, rows)
    assert rh.kernel_durations(d) == [10, 30, 50]
    assert rh.kernel_durations(d, rh.MERGE_TAG) == [20, 40, 60]
    assert rh.kernel_name(d) == k


def test_clock_median_inside_timed_region():
    c = rh.ClockSampler.__new__(rh.ClockSampler)
    c.samples = [(1.0, 2400), (2.0, 1800), (2.5, 1850), (3.0, 1900), (9.0, 2400)]
    assert c.median_between(1.5, 3.5) == (1850, 3)
    assert c.median_between(4.0, 5.0) == (None, 0)


def test_bench_stderr_and_line(tmp_path):
    log = tmp_path / "trace.log"
    log.write_text("rocprofv3 noise\n[bench] timed region epoch 100.250 101.500\n")
    assert rh._timed_region(str(log)) == (100.25, 101.5)
    out = tmp_path / "b.json"
    out.write_text("noise\n" + json.dumps({"value": 1.0}) + "\n")
    assert rh._bench_line(str(out)) == {"value": 1.0}


def test_sclk_parser():
    text = "device,sclk clock level:,sclk clock speed:,mclk\ncard0,1,(1883Mhz),(2000Mhz)\n"
    assert bench.sclk_from_csv(text) == 1883
    assert bench.sclk_from_csv("no csv here") is None


def test_markdown_names_commands():
    w = attn_inputs.WORKLOADS["gqa16k_d256"]
    a = argparse.Namespace(workload="gqa16k_d256", steps=3, command="python -m x --workload y")
    s = {"kernel_sha": "abc", "launches_traced": 205, "timed_launches": 100,
         "warmup_ms": [8.5, 7.7], "kernel_avg_ms": 6.9, "kernel_min_ms": 6.8,
         "kernel_max_ms": 7.1, "merge_avg_ms": None, "bench_kernel_ms_mean": 6.9,
         "trace_frac": 0.5, "sclk_mhz_timed_region": 1880, "sclk_samples": 4,
         "mfma_util_pct": 60.0, "lds_bank_conflicts_per_access": 0.0,
         "fetch_calibration": 2.0, "fetch_bytes_per_launch": 6e8,
         "algorithmic_read_bytes": 3e8, "write_calibration": 1.0,
         "write_bytes_per_launch": 2.7e8, "bench_frac": 0.5}
    line = {"value": 1266.0, "unit": "TFLOPS", "ms_per_step": 6.94,
            "config": {"kernel": "attn_fwd_d256_f16"},
            "roofline": {"unit": "TFLOP/s", "frac": 0.5}}
    md = rh.markdown(a, w, s, line, "attn_fwd_kernel<...>",
                     ["rocprofv3", "--kernel-trace", "--", sys.executable,
                      os.path.join(ROOT, "bench.py")])
    assert "python -m x --workload y" in md
    assert "rocprofv3 --kernel-trace -- python3 bench.py" in md
    assert "1880 MHz" in md and "2.00 x" in md


def test_kernel_stats_and_index(tmp_path):
    d = str(tmp_path)
    os.makedirs(os.path.join(d, "trace", "h"))
    with open(os.path.join(d, "trace", "h", "k_kernel_stats.csv"), "w") as f:
        f.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n")
        f.write('"attn_fwd_kernel<x>",10,100,10.0,90,9,11,0.5\n')
        f.write('"__amd_rocclr_copyBuffer",3,30,10.0,10,9,11,0.5\n')
    assert rh.kernel_stats(d) == [("attn_fwd_kernel<x>", 10, 10.0, 9.0, 11.0)]
    t = {"w1": {"kernel_sha": "abc", "timed_launches": 100, "kernel_avg_ms": 7.0,
                "bench_frac": 0.5, "trace_frac": 0.5, "sclk_mhz_timed_region": 1800,
                "mfma_util_pct": 63.0, "lds_bank_conflicts_per_access": 0.0,
                "fetch_bytes_per_launch": 6e8, "algorithmic_read_bytes": 3e8,
                "write_bytes_per_launch": 2e8},
         "old": {"kernel_sha": "x", "bytes_per_launch": 1}}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(t))
    text = rh.index_table(str(p), "python -m x")
    assert "| w1 | abc | 100 | 7.0000 | 0.5 | 0.5000 | 1800 | 63.0 | 0.0000 | 600.0 (2.00) | 200.0 |" in text
    assert "| old |" not in text


def _write_sq_pass(d, name, rows, engines=32, simds=1024):
    """A --pmc pass directory: agent table and counter rows (dispatch, kernel, counter,
    value, start, end)."""
    base = os.path.join(d, name, "host")
    os.makedirs(base, exist_ok=True)
    with open(os.path.join(base, "p_agent_info.csv"), "w") as f:
        f.write("Agent_Type,Num_Shader_Banks,Simd_Count\n")
        f.write('"CPU",0,0\n"GPU",%d,%d\n' % (engines, simds))
    with open(os.path.join(base, "p_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,"
                "End_Timestamp\n")
        for r in rows:
            f.write('%d,"%s","%s",%f,%d,%d\n' % r)


def test_sq_figures(tmp_path):
    """Cycles per launch are the busy cycles over the shader engines, matrix-core busy the
    MFMA busy cycles over SIMDs and cycles, the clock cycles over duration; other kernels'
    rows are ignored."""
    d = str(tmp_path)
    k = "_ZN12_GLOBAL__N_115attn_fwd_kernelILi256ELi0EDF16_Lb0EEEvNS_6ParamsE"
    flops = 1000 * rh.MFMA_FLOP  # 1000 algorithmic MFMAs
    rows = []
    for disp, t0 in ((2, 0), (3, 10_000)):  # two launches of 2 us each
        vals = {"SQ_BUSY_CYCLES": 32 * 3000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 2400.0,
                "SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 250.0, "SQ_WAIT_INST_ANY": 100.0,
                "SQ_ACTIVE_INST_VALU": 400.0, "SQ_INSTS_MFMA": 1000.0, "SQ_INSTS_VALU": 3000.0,
                "SQ_INSTS_LDS": 750.0}
        rows += [(disp, k, c, v, t0, t0 + 2000) for c, v in vals.items()]
    rows.append((1, "copy_kernel", "SQ_BUSY_CYCLES", 1e9, 0, 10))
    _write_sq_pass(d, "sq1", rows)
    assert rh.gpu_agent(d, "sq1") == (32, 1024)
    launches = rh.sq_launches(d, "sq1")
    assert len(launches) == 2 and launches[0][1] == 2000
    med, fig = rh.sq_figures(launches, 32, 1024, flops)
    assert fig["cycles_per_launch"] == 3000.0
    assert abs(fig["mfma_busy_pct"] - 80.0) < 1e-9
    assert abs(fig["clock_mhz_min"] - 1500.0) < 1e-9  # 3000 cycles in 2 us
    assert fig["mfma_per_algorithmic"] == 1.0 and fig["valu_per_mfma"] == 2.0
    assert fig["lds_per_mfma"] == 0.75 and fig["wait_any_pct"] == 25.0
