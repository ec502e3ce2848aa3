"""rocprofv3 harness for the attention kernel: launch durations next to a bench line of the
same run, MFMA utilisation, LDS bank conflicts and HBM traffic of one workload, from
separate profiler runs of bench.py.

    python -m flash_attention_amd.rocprof_harness --workload gqa16k_d256 \
        [--outdir rocprof_out] [--traffic-json traffic.json] [--md summary.md]
    python -m flash_attention_amd.rocprof_harness --workload all --traffic-json traffic.json \
        [--md-dir profiles]

Runs, each as its own child process (this process never touches the GPU):
  1. rocprofv3 --kernel-trace --stats  -- bench.py (W warm-up + K timed launches)
     -> every launch's duration and bench.py's own JSON line from the same process; the
        average over the K timed launches (dispatch order: the first W launches of the
        attention kernel are the warm-up) is set beside the bench line's event-timed mean.
        Meanwhile this process samples the shader clock with rocm-smi; the median of the
        samples inside the timed region (bench.py prints its wall-clock bounds) is recorded.
  2. rocprofv3 --pmc MfmaUtil LdsBankConflict  -> matrix-core busy %, LDS conflicts/access
  3. rocprofv3 --pmc FETCH_SIZE                -> KiB read from HBM per dispatch
  4. rocprofv3 --pmc WRITE_SIZE                -> KiB written to HBM per dispatch
Passes 3 and 4 also time a plain 1 GiB device copy (bench.py --copy-calib-mib); the ratio
of its known byte count to what the counter reads for it calibrates the counter, and the
kernel's reading is scaled by that ratio.  Counter passes run under a hard kill timeout
so that a refused counter request cannot leave a hung profiler behind.

With --sq it instead runs three passes of SQ (sequencer) counters per workload (cycles,
matrix-core busy cycles, wait and issue counters, instruction counts) and writes one
summary of where a launch's cycles go and at what average clock it ran.

Prints a markdown summary (also written to --md, or to <md-dir>/<kernel>__<workload>.md)
and, with --traffic-json, records the calibrated bytes per launch under the workload's name
together with the hash of the kernel sources, so that bench.py reports them only while the
kernel is unchanged.
"""
import argparse
import csv
import glob
import json
import os
import shutil
import statistics
import subprocess
import sys
import threading
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_TAG = "attn_fwd_kernel"
MERGE_TAG = "attn_merge_kernel"
COPY_MIB = 1024


def _bench_cmd(workload, steps, warmup, calib):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload,
           "--steps", str(steps), "--warmup", str(warmup), "--no-cpu", "--no-clock"]
    if calib:
        cmd += ["--copy-calib-mib", str(COPY_MIB)]
    return cmd


def _run(cmd, log, kill_after, out=None):
    """Run one profiler pass from /tmp (TMPDIR=/tmp); return its exit status.  stdout goes
    to `out` when given (bench.py's JSON line), else with stderr to `log`."""
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(kill_after)] + cmd
    print("[harness] " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        if out is None:
            r = subprocess.run(full, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT)
        else:
            with open(out, "w") as g:
                r = subprocess.run(full, cwd="/tmp", env=env, stdout=g, stderr=f)
    # rocprofv3 may end with SIGSEGV after the program finished and wrote its results
    print("[harness]   exit %d (log %s)" % (r.returncode, log), flush=True)
    return r.returncode


def _rows(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def counters(outdir, name):
    """{dispatch id: (kernel name, {counter: summed value})} of one --pmc pass."""
    res = {}
    for r in _rows(os.path.join(outdir, name, "**", "*counter_collection.csv")):
        d = int(r["Dispatch_Id"])
        kname, vals = res.setdefault(d, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return res


def kernel_durations(outdir, tag=KERNEL_TAG):
    """Durations (ns) of the launches whose name contains `tag`, in dispatch order."""
    rows = [r for r in _rows(os.path.join(outdir, "trace", "**", "*kernel_trace.csv"))
            if tag in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def kernel_stats(outdir):
    """Rows of rocprofv3's --stats summary (k_kernel_stats.csv) for the attention and
    merge kernels: (name, calls, average ns, min ns, max ns)."""
    rows = []
    for r in _rows(os.path.join(outdir, "trace", "**", "*kernel_stats.csv")):
        if KERNEL_TAG in r["Name"] or MERGE_TAG in r["Name"]:
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]),
                         float(r["MinNs"]), float(r["MaxNs"])))
    return rows


def kernel_name(outdir, tag=KERNEL_TAG):
    for r in _rows(os.path.join(outdir, "trace", "**", "*kernel_trace.csv")):
        if tag in r["Kernel_Name"]:
            return r["Kernel_Name"]
    return None


def calibrated_bytes(outdir, name, counter):
    """(median KiB per kernel dispatch, copy-calibration factor)."""
    disp = counters(outdir, name)
    kern = [v[counter] for k, v in disp.values() if KERNEL_TAG in k]
    # the calibration copy is the largest copy dispatch in the run
    copies = [v[counter] for k, v in disp.values() if "copy" in k.lower()]
    if not kern or not copies:
        raise RuntimeError("%s: kernel or calibration copy dispatch missing" % name)
    factor = COPY_MIB * 1024.0 / max(copies)
    return statistics.median(kern), factor


class ClockSampler:
    """Samples the shader clock with rocm-smi from a thread of this (GPU-free) process:
    a list of (wall-clock time, MHz)."""

    def __init__(self):
        sys.path.insert(0, ROOT)
        import bench  # noqa: E402  (the CSV parser; imports no GPU code)
        self._parse = bench.sclk_from_csv
        self._exe = shutil.which("rocm-smi")
        self._stop = threading.Event()
        self.samples = []
        self._thread = threading.Thread(target=self._loop, daemon=True)

    def _loop(self):
        while self._exe and not self._stop.is_set():
            t0 = time.time()
            try:
                r = subprocess.run([self._exe, "--showclocks", "--csv"], capture_output=True,
                                   text=True, timeout=20)
            except (OSError, subprocess.SubprocessError):
                return
            mhz = self._parse(r.stdout)
            if mhz:
                self.samples.append(((t0 + time.time()) / 2, mhz))
            self._stop.wait(0.05)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=30)

    def median_between(self, t0, t1):
        inside = sorted(m for t, m in self.samples if t0 <= t <= t1)
        return (inside[len(inside) // 2], len(inside)) if inside else (None, 0)


def _timed_region(log):
    """Wall-clock bounds of bench.py's timed region, from its stderr."""
    with open(log) as f:
        for line in f:
            if line.startswith("[bench] timed region epoch"):
                a, b = line.split()[-2:]
                return float(a), float(b)
    return None


def _bench_line(path):
    with open(path) as f:
        lines = [x for x in f.read().splitlines() if x.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="gqa16k_d256",
                    help="a name of attn_inputs.WORKLOADS, or 'all' (every one but 'tiny', "
                         "each into its own subdirectory of --outdir)")
    ap.add_argument("--outdir", default="rocprof_out")
    ap.add_argument("--traffic-json", default=None)
    ap.add_argument("--md", default=None, help="write the markdown summary here")
    ap.add_argument("--md-dir", default=None,
                    help="write each workload's summary to <md-dir>/<kernel>__<workload>.md")
    ap.add_argument("--steps", type=int, default=3, help="timed launches of the counter passes")
    ap.add_argument("--trace-steps", type=int, default=100,
                    help="timed launches of the trace pass (bench.py's default)")
    ap.add_argument("--trace-warmup", type=int, default=5)
    ap.add_argument("--kill-after", type=int, default=90)
    ap.add_argument("--sq", action="store_true",
                    help="SQ counter passes instead (--workload may list several, comma-"
                         "separated); the summary goes to --md")
    ap.add_argument("--index", default=None,
                    help="only write a table of every workload in this --traffic-json file "
                         "(to --md) and exit")
    a = ap.parse_args()
    # (paths inside the repository are shown relative to its root)
    a.command = "python -m flash_attention_amd.rocprof_harness " + " ".join(
        os.path.relpath(x, ROOT) if x.startswith(ROOT + os.sep) else x for x in sys.argv[1:])
    if a.sq:
        return sq_profile(a.workload.split(","), os.path.abspath(a.outdir), a)
    if a.index:
        text = index_table(a.index, a.command)
        print(text)
        if a.md:
            with open(a.md, "w") as f:
                f.write(text)
        return 0
    if a.workload != "all":
        return profile(a.workload, os.path.abspath(a.outdir), a)
    sys.path.insert(0, ROOT)
    import attn_inputs  # noqa: E402  (shapes only; imports no GPU code)
    for name in attn_inputs.WORKLOADS:
        if name == "tiny":
            continue
        rc = profile(name, os.path.join(os.path.abspath(a.outdir), name), a)
        if rc != 0:
            return rc
    return 0


def profile(workload, out, a):
    """The four passes over one workload; 0, or the exit status of the pass that failed."""
    a = argparse.Namespace(**dict(vars(a), workload=workload))
    os.makedirs(out, exist_ok=True)
    rp = "rocprofv3"

    def ok(rc):
        return rc in (0, 139)

    trace_cmd = ([rp, "--kernel-trace", "--stats", "-f", "csv", "-d", os.path.join(out, "trace"),
                  "-o", "k", "--"] +
                 _bench_cmd(a.workload, a.trace_steps, a.trace_warmup, False))
    with ClockSampler() as clock:
        rc = _run(trace_cmd, os.path.join(out, "trace.log"), 300,
                  out=os.path.join(out, "trace_bench.json"))
    if not ok(rc):
        print("[harness] pass trace failed (exit %d); stopping" % rc, flush=True)
        return rc
    passes = [
        ("util", [rp, "--pmc", "MfmaUtil", "LdsBankConflict", "-f", "csv", "-d",
                  os.path.join(out, "util"), "-o", "p", "--"] +
         _bench_cmd(a.workload, a.steps, 1, False), a.kill_after),
        ("fetch", [rp, "--pmc", "FETCH_SIZE", "-f", "csv", "-d", os.path.join(out, "fetch"),
                   "-o", "p", "--"] + _bench_cmd(a.workload, a.steps, 1, True), a.kill_after),
        ("write", [rp, "--pmc", "WRITE_SIZE", "-f", "csv", "-d", os.path.join(out, "write"),
                   "-o", "p", "--"] + _bench_cmd(a.workload, a.steps, 1, True), a.kill_after),
    ]
    for name, cmd, kill in passes:
        rc = _run(cmd, os.path.join(out, name + ".log"), kill)
        if not ok(rc):
            print("[harness] pass %s failed (exit %d); stopping" % (name, rc), flush=True)
            return rc

    # trace pass: the timed launches are the attention kernel's launches W .. W+K-1 (one
    # per step; a split step also launches the merge once)
    dur = kernel_durations(out)
    mdur = kernel_durations(out, MERGE_TAG)
    W, K = a.trace_warmup, a.trace_steps
    timed = dur[W:W + K]
    mtimed = mdur[W:W + K]
    line = _bench_line(os.path.join(out, "trace_bench.json"))
    region = _timed_region(os.path.join(out, "trace.log"))
    sclk, nsamp = clock.median_between(*region) if region else (None, 0)
    avg_ns = statistics.mean(timed)
    merge_ns = statistics.mean(mtimed) if mtimed else 0.0
    util = [v for k, v in counters(out, "util").values() if KERNEL_TAG in k]
    mfma = statistics.median(v["MfmaUtil"] for v in util)
    lds = statistics.median(v["LdsBankConflict"] for v in util)
    fetch_kib, ffac = calibrated_bytes(out, "fetch", "FETCH_SIZE")
    write_kib, wfac = calibrated_bytes(out, "write", "WRITE_SIZE")
    fetch_b = fetch_kib * 1024 * ffac
    write_b = write_kib * 1024 * wfac
    gbs = (fetch_b + write_b) / avg_ns
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (source hash of the kernel; imports no GPU code)
    import attn_inputs  # noqa: E402
    w = attn_inputs.WORKLOADS[a.workload]
    roof = line["roofline"] if line else None
    step_ns = avg_ns + merge_ns
    # the bench line's roofline recomputed from the trace's timed launches (attention +
    # merge per step, as the bench line's events bracket both)
    frac_trace = None
    if roof:
        if roof["unit"] == "TFLOP/s":
            frac_trace = roof["algorithmic_flops_per_launch"] / step_ns * 1e-3 / roof["peak"]
        else:
            frac_trace = roof["algorithmic_bytes_per_launch"] / step_ns / roof["peak"]
    summary = {
        "kernel_sha": bench.kernel_source_hash(), "launches_traced": len(dur),
        "timed_launches": len(timed), "kernel_avg_ms": avg_ns / 1e6,
        "kernel_min_ms": min(timed) / 1e6, "kernel_max_ms": max(timed) / 1e6,
        "merge_avg_ms": merge_ns / 1e6 if mtimed else None,
        "warmup_ms": [round(x / 1e6, 4) for x in dur[:W]],
        "sclk_mhz_timed_region": sclk, "sclk_samples": nsamp,
        "bench_kernel_ms_mean": line.get("kernel_ms_mean") if line else None,
        "bench_value": line.get("value") if line else None,
        "bench_frac": roof["frac"] if roof else None, "trace_frac": frac_trace,
        "mfma_util_pct": mfma, "lds_bank_conflicts_per_access": lds,
        "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
        "fetch_calibration": ffac, "write_calibration": wfac,
        "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b, "hbm_gbs": gbs,
        "algorithmic_read_bytes":
            bench.algorithmic_bytes(w) - w.B * w.Hq * w.Lq * (2 * w.D + 4),
    }
    print(json.dumps(summary, indent=1))
    summary["stats"] = kernel_stats(out)
    md = markdown(a, w, summary, line, kernel_name(out), trace_cmd)
    print(md)
    path = a.md
    if path is None and a.md_dir:
        short = line["config"]["kernel"] if line else "attn_fwd"
        path = os.path.join(a.md_dir, "%s__%s.md" % (short, a.workload))
    if path:
        with open(path, "w") as f:
            f.write(md)
    if a.traffic_json:
        try:
            with open(a.traffic_json) as f:
                t = json.load(f)
        except (OSError, ValueError):
            t = {}
        t[a.workload] = summary
        with open(a.traffic_json, "w") as f:
            json.dump(t, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


def index_table(traffic_json, command):
    """One line per workload of a --traffic-json file (what each per-workload summary
    holds, side by side)."""
    with open(traffic_json) as f:
        t = json.load(f)
    out = ["# rocprofv3 summaries of every workload (attention kernel)", "",
           "Made by (repository root):", "", "    " + command, "",
           "from the figures each workload's own summary records (its trace pass: W warm-up "
           "and K timed launches beside the bench line of the same process; its counter "
           "passes: MfmaUtil and LdsBankConflict, FETCH_SIZE, WRITE_SIZE, each calibrated "
           "by a plain device copy of known size).", "",
           "| workload | kernel source hash | timed launches | trace average ms | bench "
           "`roofline.frac` | same from the trace | shader clock MHz | MFMA busy % | "
           "LDS conflicts / access | HBM read MB (x algorithmic) | HBM write MB |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(t):
        s = t[name]
        if "trace_frac" not in s:
            continue
        out.append("| %s | %s | %d | %.4f | %s | %.4f | %s | %.1f | %.4f | %.1f (%.2f) | %.1f |" % (
            name, s["kernel_sha"], s["timed_launches"], s["kernel_avg_ms"], s["bench_frac"],
            s["trace_frac"], s["sclk_mhz_timed_region"], s["mfma_util_pct"],
            s["lds_bank_conflicts_per_access"], s["fetch_bytes_per_launch"] / 1e6,
            s["fetch_bytes_per_launch"] / s["algorithmic_read_bytes"],
            s["write_bytes_per_launch"] / 1e6))
    out.append("")
    return "\n".join(out)


# SQ counters of the three --sq passes (at most 8 SQ counters per pass).
SQ_PASSES = [
    ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
     "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES"],
    ["SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_INST_LEVEL_LDS", "SQ_LDS_IDX_ACTIVE",
     "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL", "SQ_IFETCH", "SQ_ACTIVE_INST_VMEM"],
    ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_SCA",
     "SQ_ACTIVE_INST_MISC", "SQ_INSTS_VMEM", "SQ_IFETCH_LEVEL"],
]
MFMA_FLOP = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_{f16,bf16}


def gpu_agent(outdir, name):
    """(shader engines, SIMDs) of the GPU in a pass's agent table."""
    for r in _rows(os.path.join(outdir, name, "**", "*agent_info.csv")):
        if r.get("Agent_Type") == "GPU":
            return int(r["Num_Shader_Banks"]), int(r["Simd_Count"])
    raise RuntimeError("%s: no GPU agent in the agent table" % name)


def sq_launches(outdir, name):
    """[(counter values, duration ns)] of the attention launches of one pass."""
    res = {}
    for r in _rows(os.path.join(outdir, name, "**", "*counter_collection.csv")):
        if KERNEL_TAG not in r["Kernel_Name"]:
            continue
        vals, _ = res.setdefault(int(r["Dispatch_Id"]), ({}, None))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        res[int(r["Dispatch_Id"])] = (vals, int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return [res[d] for d in sorted(res)]


def sq_figures(launches, engines, simds, flops):
    """Medians of every counter over the launches, and what follows from them: SQ cycle
    counters are summed over the shader engines, the matrix-core busy cycles over the
    SIMDs."""
    names = sorted({k for v, _ in launches for k in v})
    med = {k: statistics.median(v[k] for v, _ in launches if k in v) for k in names}
    cyc = med["SQ_BUSY_CYCLES"] / engines
    clocks = [v["SQ_BUSY_CYCLES"] / engines / (ns * 1e-9) / 1e6
              for v, ns in launches if "SQ_BUSY_CYCLES" in v and ns > 0]
    fig = {
        "mfma_per_algorithmic": med["SQ_INSTS_MFMA"] / (flops / MFMA_FLOP),
        "valu_per_mfma": (med["SQ_INSTS_VALU"] - med["SQ_INSTS_MFMA"]) / med["SQ_INSTS_MFMA"],
        "lds_per_mfma": med["SQ_INSTS_LDS"] / med["SQ_INSTS_MFMA"],
        "cycles_per_mfma": med["SQ_VALU_MFMA_BUSY_CYCLES"] / med["SQ_INSTS_MFMA"],
        "cycles_per_launch": cyc,
        "mfma_busy_pct": 100 * med["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cyc,
        "clock_mhz_min": min(clocks), "clock_mhz_max": max(clocks),
        "wait_any_pct": 100 * med["SQ_WAIT_ANY"] / med["SQ_WAVE_CYCLES"],
        "wait_inst_any_pct": 100 * med["SQ_WAIT_INST_ANY"] / med["SQ_WAVE_CYCLES"],
        "active_valu_pct": 100 * med["SQ_ACTIVE_INST_VALU"] / med["SQ_WAVE_CYCLES"],
    }
    return med, fig


def sq_profile(workloads, out, a):
    """The three SQ passes over each workload, then one summary of them all."""
    sys.path.insert(0, ROOT)
    import attn_inputs  # noqa: E402  (shapes only; imports no GPU code)
    import bench  # noqa: E402
    cmds, sections = [], []
    for wl in workloads:
        w = attn_inputs.WORKLOADS[wl]
        wout = os.path.join(out, wl)
        os.makedirs(wout, exist_ok=True)
        for i, ctrs in enumerate(SQ_PASSES, 1):
            cmd = (["rocprofv3", "--pmc"] + ctrs + ["-f", "csv", "-d",
                   os.path.join(wout, "sq%d" % i), "-o", "p", "--"] +
                   _bench_cmd(wl, a.steps, 1, False))
            if wl == workloads[0]:
                cmds.append(cmd)
            rc = _run(cmd, os.path.join(wout, "sq%d.log" % i), a.kill_after)
            if rc not in (0, 139):
                print("[harness] SQ pass %d failed (exit %d); stopping" % (i, rc), flush=True)
                return rc
        engines, simds = gpu_agent(wout, "sq1")
        launches = []
        for i in range(1, len(SQ_PASSES) + 1):
            launches += sq_launches(wout, "sq%d" % i)
        med, fig = sq_figures(launches, engines, simds, bench.flops_workload(w))
        sections.append((wl, w, med, fig, engines, simds))
    md = sq_markdown(a, cmds, sections, bench.kernel_source_hash())
    print(md)
    if a.md:
        with open(a.md, "w") as f:
            f.write(md)
    return 0


def sq_markdown(a, cmds, sections, sha):
    def rel(c):
        return " ".join("python3" if x == sys.executable else
                        os.path.relpath(x, ROOT) if x.startswith(ROOT) else x for x in c)

    out = ["# attn_fwd: issue and stall counters (SQ block), %s" %
           ", ".join(wl for wl, *_ in sections), "",
           "Made by (repository root on the MI355X box; every pass is a child process, run "
           "from /tmp with TMPDIR=/tmp):", "", "    " + a.command, "",
           "which runs, for each workload (here the first):", ""]
    out += ["    " + rel(c) for c in cmds]
    out += ["", "Kernel source hash: `%s`.  Values are medians over the attention launches of "
            "the passes (1 warm-up + %d timed each).  SQ cycle counters are summed over the "
            "GPU's shader engines, the matrix-core busy cycles over its SIMDs (both from the "
            "profiler's agent table); a launch's duration comes from the same rows' "
            "timestamps." % (sha, a.steps), ""]
    for wl, w, med, fig, engines, simds in sections:
        out += ["## %s (%s)" % (wl, w.describe()), "", "| counter | median per launch |",
                "|---|---|"]
        out += ["| `%s` | %.4g |" % (k, med[k]) for k in sorted(med)]
        out += ["", "Derived (%d shader engines, %d SIMDs):" % (engines, simds), "",
                "| figure | value |", "|---|---|",
                "| MFMA instructions / (algorithmic flops / %d per v_mfma_f32_32x32x16) | %.4f |"
                % (MFMA_FLOP, fig["mfma_per_algorithmic"]),
                "| other VALU instructions per MFMA | %.2f |" % fig["valu_per_mfma"],
                "| LDS instructions per MFMA | %.2f |" % fig["lds_per_mfma"],
                "| matrix-core busy cycles per MFMA | %.2f |" % fig["cycles_per_mfma"],
                "| cycles per launch (`SQ_BUSY_CYCLES` / shader engines) | %.4gM |"
                % (fig["cycles_per_launch"] / 1e6),
                "| matrix-core busy per SIMD (`SQ_VALU_MFMA_BUSY_CYCLES` / SIMDs / cycles per "
                "launch) | %.1f %% |" % fig["mfma_busy_pct"],
                "| average clock of the profiled launches (cycles / duration) | %.0f-%.0f MHz |"
                % (fig["clock_mhz_min"], fig["clock_mhz_max"]),
                "| wave time in dependency waits (`SQ_WAIT_ANY` / `SQ_WAVE_CYCLES`) | %.1f %% |"
                % fig["wait_any_pct"],
                "| wave time waiting to issue (`SQ_WAIT_INST_ANY` / `SQ_WAVE_CYCLES`) | %.1f %% |"
                % fig["wait_inst_any_pct"],
                "| wave time issuing VALU (`SQ_ACTIVE_INST_VALU` / `SQ_WAVE_CYCLES`) | %.1f %% |"
                % fig["active_valu_pct"], ""]
    return "\n".join(out)


def markdown(a, w, s, line, kname, trace_cmd):
    """The summary of one workload, with the commands that made it."""
    rel = [os.path.relpath(x, ROOT) if x.startswith(ROOT) else x for x in trace_cmd]
    rel = ["python3" if x == sys.executable else x for x in rel]
    frac = s["bench_frac"]
    unit = line["roofline"]["unit"] if line else ""
    out = []
    out.append("# %s: %s (%s)" % (line["config"]["kernel"] if line else "attn_fwd", a.workload,
                                  w.describe() if hasattr(w, "describe") else a.workload))
    out.append("")
    out.append("Made by (repository root on the MI355X box; every pass is a child process, "
               "run from /tmp with TMPDIR=/tmp):")
    out.append("")
    out.append("    " + a.command)
    out.append("")
    out.append("Trace pass (the bench line below is this same process's output):")
    out.append("")
    out.append("    " + " ".join(rel))
    out.append("")
    out.append("Kernel source hash: `%s`.  Kernel: `%s`." % (s["kernel_sha"], kname))
    out.append("")
    out.append("| figure | value |")
    out.append("|---|---|")
    out.append("| attention launches traced | %d (%d warm-up, %d timed, then bench.py's "
               "one-by-one launches) |" % (s["launches_traced"], len(s["warmup_ms"]),
                                          s["timed_launches"]))
    out.append("| warm-up launches, ms | %s |" % ", ".join("%.4f" % x for x in s["warmup_ms"]))
    out.append("| **timed launches, trace average ms** | **%.4f** (min %.4f, max %.4f) |" % (
        s["kernel_avg_ms"], s["kernel_min_ms"], s["kernel_max_ms"]))
    if s["merge_avg_ms"] is not None:
        out.append("| merge launches (timed steps), trace average ms | %.4f |" %
                   s["merge_avg_ms"])
    out.append("| bench line `kernel_ms_mean` (HIP events over the same timed steps) | %s |" %
               s["bench_kernel_ms_mean"])
    if line:
        out.append("| bench line `value` | %s %s (`ms_per_step` %s) |" % (
            line["value"], line["unit"], line["ms_per_step"]))
        out.append("| bench line `roofline.frac` (%s) | %s |" % (unit, frac))
    if s["trace_frac"] is not None:
        out.append("| the same fraction from the trace's timed launches | %.4f |" %
                   s["trace_frac"])
    out.append("| shader clock in the timed region (rocm-smi, median) | %s MHz (%d samples) |"
               % (s["sclk_mhz_timed_region"], s["sclk_samples"]))
    out.append("| MFMA busy, %% of cycles (MfmaUtil) | %.1f |" % s["mfma_util_pct"])
    out.append("| LDS bank conflicts per access | %.4f |" % s["lds_bank_conflicts_per_access"])
    out.append("| HBM read per launch, MB (FETCH_SIZE x %.3f) | %.1f (%.2f x the algorithmic "
               "Q + K + V) |" % (s["fetch_calibration"], s["fetch_bytes_per_launch"] / 1e6,
                                 s["fetch_bytes_per_launch"] / s["algorithmic_read_bytes"]))
    out.append("| HBM write per launch, MB (WRITE_SIZE x %.3f) | %.1f |" % (
        s["write_calibration"], s["write_bytes_per_launch"] / 1e6))
    if s.get("stats"):
        out.append("")
        out.append("rocprofv3 `--stats` summary of the trace pass (`k_kernel_stats.csv`: every "
                   "launch of the run, the warm-up and bench.py's one-by-one launches after the "
                   "timed region included; the timed-launch average above is taken from the "
                   "same run's `k_kernel_trace.csv`):")
        out.append("")
        out.append("| kernel | calls | average ns | min ns | max ns |")
        out.append("|---|---|---|---|---|")
        for name, calls, avg, lo, hi in s["stats"]:
            out.append("| `%s` | %d | %.0f | %.0f | %.0f |" % (name[:90], calls, avg, lo, hi))
    out.append("")
    out.append("Counter passes: `rocprofv3 --pmc MfmaUtil LdsBankConflict`, `--pmc FETCH_SIZE`, "
               "`--pmc WRITE_SIZE`, each of `bench.py --workload %s --steps %d --warmup 1 "
               "--no-cpu --no-clock` (the last two with `--copy-calib-mib %d`: a plain device "
               "copy of known size calibrates the counter); medians over the attention "
               "launches." % (a.workload, a.steps, COPY_MIB))
    if line:
        out.append("")
        out.append("Bench line of the trace pass:")
        out.append("")
        out.append("    " + json.dumps(line))
    out.append("")
    return "\n".join(out)


if __name__ == "__main__":
    sys.exit(main())
