"""rocprofv3 harness for the attention kernel: MFMA utilisation, LDS bank conflicts, HBM
traffic and bandwidth of one workload, from separate profiler runs of bench.py.

    python -m flash_attention_amd.rocprof_harness --workload gqa16k_d256 \
        [--outdir rocprof_out] [--traffic-json traffic.json]
    python -m flash_attention_amd.rocprof_harness --workload all --traffic-json traffic.json

Runs, each as its own child process (this process never touches the GPU):
  1. rocprofv3 --kernel-trace --stats          -> launch durations of the kernel
  2. rocprofv3 --pmc MfmaUtil LdsBankConflict  -> matrix-core busy %, LDS conflicts/access
  3. rocprofv3 --pmc FETCH_SIZE                -> KiB read from HBM per dispatch
  4. rocprofv3 --pmc WRITE_SIZE                -> KiB written to HBM per dispatch
Passes 3 and 4 also time a plain 1 GiB device copy (bench.py --copy-calib-mib); the ratio
of its known byte count to what the counter reads for it calibrates the counter, and the
kernel's reading is scaled by that ratio.  Counter passes run under a hard kill timeout
so that a refused counter request cannot leave a hung profiler behind.

Prints a markdown summary and, with --traffic-json, records the calibrated bytes per
launch under the workload's name together with the hash of the kernel sources, so that
bench.py reports them only while the kernel is unchanged.
"""
import argparse
import csv
import glob
import json
import os
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_TAG = "attn_fwd_kernel"
COPY_MIB = 1024


def _bench_cmd(workload, steps, warmup, calib):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload,
           "--steps", str(steps), "--warmup", str(warmup), "--no-cpu", "--no-clock"]
    if calib:
        cmd += ["--copy-calib-mib", str(COPY_MIB)]
    return cmd


def _run(cmd, log, kill_after):
    """Run one profiler pass from /tmp (TMPDIR=/tmp); return its exit status."""
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(kill_after)] + cmd
    print("[harness] " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(full, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT)
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


def kernel_durations(outdir):
    ns = []
    for r in _rows(os.path.join(outdir, "trace", "**", "*kernel_trace.csv")):
        if KERNEL_TAG in r["Kernel_Name"]:
            ns.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return ns


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="gqa16k_d256",
                    help="a name of attn_inputs.WORKLOADS, or 'all' (every one but 'tiny', "
                         "each into its own subdirectory of --outdir)")
    ap.add_argument("--outdir", default="rocprof_out")
    ap.add_argument("--traffic-json", default=None)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--kill-after", type=int, default=90)
    a = ap.parse_args()
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

    passes = [
        ("trace", [rp, "--kernel-trace", "--stats", "-f", "csv", "-d", os.path.join(out, "trace"),
                   "-o", "k", "--"] + _bench_cmd(a.workload, a.steps, 1, False), 300),
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

    dur = kernel_durations(out)
    util = [v for k, v in counters(out, "util").values() if KERNEL_TAG in k]
    mfma = statistics.median(v["MfmaUtil"] for v in util)
    lds = statistics.median(v["LdsBankConflict"] for v in util)
    fetch_kib, ffac = calibrated_bytes(out, "fetch", "FETCH_SIZE")
    write_kib, wfac = calibrated_bytes(out, "write", "WRITE_SIZE")
    fetch_b = fetch_kib * 1024 * ffac
    write_b = write_kib * 1024 * wfac
    avg_ns = statistics.mean(dur)
    gbs = (fetch_b + write_b) / avg_ns
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (source hash of the kernel; imports no GPU code)
    sha = bench.kernel_source_hash()
    summary = {
        "kernel_sha": sha, "launches_traced": len(dur), "kernel_avg_ms": avg_ns / 1e6,
        "kernel_min_ms": min(dur) / 1e6, "mfma_util_pct": mfma,
        "lds_bank_conflicts_per_access": lds,
        "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
        "fetch_calibration": ffac, "write_calibration": wfac,
        "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b, "hbm_gbs": gbs,
    }
    print(json.dumps(summary, indent=1))
    print()
    print("| workload | kernel avg ms | MFMA util % | LDS conflicts/access | HBM read MB | "
          "HBM write MB | HBM GB/s |")
    print("|---|---|---|---|---|---|---|")
    print("| %s | %.3f | %.1f | %.4f | %.1f | %.1f | %.1f |" % (
        a.workload, avg_ns / 1e6, mfma, lds, fetch_b / 1e6, write_b / 1e6, gbs))
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


if __name__ == "__main__":
    sys.exit(main())
