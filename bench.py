"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one attention forward over the whole workload (every step of the method in the
one kernel), inputs resident in HBM.  Prints ONE JSON line.  The default workload is the
16K x 16K, 32 query / 2 key-value heads, HD=256, fp16 case; other names are listed in
attn_inputs.WORKLOADS.

The metric is attention TFLOPS = 4*B*Hq*Lq*Lk*D / time (the two matrix products) and its
fraction of MI355X's dense fp16/bf16 MFMA peak.  The "Xe2 ... Flash Attention -- HD=256"
page's formula (section "Performance Testing"), which adds 2*Lq*Lk*Hq for the softmax, is
reported beside it.  The fp64 CPU oracle is timed on a seeded sample of query rows on the
host cores (cpu_baseline) and checks the GPU output on those rows.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense fp16/bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU (AMD's 2.5 PFLOP/s).
PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
METRIC = "attn fwd TFLOPS & % of MFMA peak, GQA 32Q/2KV HD=256 16Kx16K fp16"
# The pages' own figure for the same workload (16K x 16K, 32 query / 2 key-value heads,
# HD=256, fp16): 88 TFLOPS for the best kernel of the "Xe2 (Lunar Lake/LNL, Battlemage/BMG)
# ESIMD Flash Attention -- HD=256" page (header, and section "Performance Ladder"), measured
# on Intel Xe2 hardware.  Context, not a target: vs_baseline = value / that figure.
PAGES_TFLOPS = {"gqa16k_d256": 88.0}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "flash_attention_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "attn_config.h")]


def flops_headline(B, Hq, Lq, Lk, D):
    return 4 * B * Hq * Lq * Lk * D


def visible_pairs(Lq, Lk, causal):
    """(query row, key) pairs per head that enter the products: all of them, or under the
    causal mask (row i sees key j iff j <= i + Lk - Lq) the lower triangle."""
    if not causal:
        return Lq * Lk
    import numpy as np
    return int(np.clip(np.arange(Lq) + Lk - Lq + 1, 0, Lk).sum())


def flops_workload(w):
    """4*D flops per visible (row, key) pair: 4*B*Hq*Lq*Lk*D without a mask."""
    return 4 * w.B * w.Hq * visible_pairs(w.Lq, w.Lk, w.causal) * w.D


def algorithmic_bytes(w):
    """Q and O (16-bit), K and V (16-bit, once per key/value head), LSE (fp32)."""
    q = w.B * w.Hq * w.Lq * w.D * 2
    return 2 * q + 2 * (w.B * w.Hkv * w.Lk * w.D * 2) + w.B * w.Hq * w.Lq * 4


def flops_pages(q_len, kv_len, hd, heads_q, batch=1):
    """The pages' count: both matrix products plus 2 flops per score for the softmax."""
    return batch * (4 * q_len * kv_len * hd * heads_q + 2 * q_len * kv_len * heads_q)


def kernel_source_hash():
    """Hash of the kernel sources with // comments and blank space removed, so that editing
    a comment does not invalidate counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = re.sub(r"//[^\n]*", "", f.read())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None when the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("kernel_sha") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def compare_rows(o_gpu, lse_gpu, rows, o_ref, lse_ref):
    """Error metrics of the GPU output on the oracle's rows (NaN count first)."""
    import numpy as np
    import torch
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64))
    og = o_gpu.reshape(-1, o_gpu.shape[-1])[idx].double().numpy()
    lg = lse_gpu.reshape(-1)[idx].double().numpy()
    err = og - o_ref
    # rows that see no key (causal, Lq > Lk) have LSE -inf on both sides
    empty = np.isneginf(lse_ref)
    bad_empty = int((lg[empty] != -np.inf).sum() + (og[empty] != 0).sum())
    lg_f, lr_f = lg[~empty], lse_ref[~empty]
    return {"rows": int(len(rows)),
            "nonfinite": int((~np.isfinite(og)).sum() + (~np.isfinite(lg_f)).sum()) + bad_empty,
            "rel_rms": float(np.sqrt((err ** 2).sum() / (o_ref ** 2).sum())),
            "max_abs": float(np.abs(err).max()),
            "lse_abs": float(np.abs(lg_f - lr_f).max()) if lg_f.size else 0.0}


# Shader-clock poller, run as a separate process that is started before this process touches
# the GPU: it calls rocm-smi itself (a program started from a process that has initialised
# the GPU would inherit that state).  Protocol: "start" on stdin begins polling, "stop" (or
# end of input) ends it; the median MHz of the samples (or "null") comes back on stdout.
_SCLK_POLLER = r"""
import json, shutil, subprocess, sys, threading
sys.path.insert(0, sys.argv[1])
from bench import sclk_from_csv
exe = shutil.which("rocm-smi")
if sys.stdin.readline().strip() != "start" or exe is None:
    print("null", flush=True)
    sys.exit(0)
stop = threading.Event()
threading.Thread(target=lambda: (sys.stdin.readline(), stop.set()), daemon=True).start()
samples = []
while not stop.is_set():
    try:
        r = subprocess.run([exe, "--showclocks", "--csv"], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.SubprocessError):
        break
    mhz = sclk_from_csv(r.stdout)
    if mhz:
        samples.append(mhz)
    stop.wait(0.2)
print(json.dumps(sorted(samples)[len(samples) // 2] if samples else None), flush=True)
"""


def sclk_from_csv(text):
    """Shader clock (MHz) of the first GPU from `rocm-smi --showclocks --csv`, or None."""
    lines = [x for x in text.splitlines() if "," in x]
    if len(lines) < 2:
        return None
    head = lines[0].split(",")
    if "sclk clock speed:" not in head:
        return None
    cell = lines[1].split(",")[head.index("sclk clock speed:")]
    digits = "".join(ch for ch in cell if ch.isdigit())
    return int(digits) if digits else None


def start_sclk_poller():
    """The poller process (see above), or None; call before any GPU work.  None under a
    profiler, whose preloaded library has initialised the GPU before this program began."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        return subprocess.Popen([sys.executable, "-c", _SCLK_POLLER, ROOT],
                                stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)
    except OSError:
        return None


def sample_sclk(poller, busy, seconds=1.5):
    """Shader clock (MHz) under load: busy() runs back to back for about `seconds` while the
    poller samples rocm-smi; None without a poller or samples."""
    if poller is None:
        return None
    busy()  # the clock settles under load before the first sample
    poller.stdin.write("start\n")
    poller.stdin.flush()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        busy()
    poller.stdin.write("stop\n")
    poller.stdin.flush()
    try:
        out, _ = poller.communicate(timeout=30)
        return json.loads(out.strip().splitlines()[-1])
    except Exception:  # the poller failed: no clock figure
        poller.kill()
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sampling window after the timed region")
    ap.add_argument("--cpu-rows", type=int, default=65536,
                    help="random query rows in the oracle sample")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    poller = None if args.no_clock else start_sclk_poller()  # before any GPU work
    import numpy as np
    import torch

    import attn_inputs
    import flash_attention_amd as fa

    name = args.workload or attn_inputs.HEADLINE
    w = attn_inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    t0 = time.time()
    q, k, v = attn_inputs.workload_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(w.scale))
    stream = torch.cuda.current_stream(dev)
    code = fa.dtype_code(q)
    flags = fa.ATTN_CAUSAL if w.causal else 0
    # the launch: the planner's (splits and tile shape: attn_fwd_ex with nsplit = 0), unless
    # the workload fixes the split count (then the default tile shape)
    if w.nsplit:
        plan = fa.attn_plan(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, code)
        plan.grid *= w.nsplit
        plan.nsplit = w.nsplit
    else:
        plan = fa.attn_plan_ex(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, code, flags)
    nsplit = plan.nsplit
    # the workspace of a split launch is allocated once, outside the timed region
    ws_bytes = fa.attn_workspace_bytes(w.B, w.Hq, w.Lq, w.D, nsplit)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if not w.causal and nsplit == 1:
        args_c = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                  w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, scale, code, stream.cuda_stream)
        launch = fa.attn_fwd_stream
    else:
        args_c = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                  w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, scale, code, flags, w.nsplit,
                  ws.data_ptr(), ws_bytes, stream.cuda_stream)
        launch = fa.attn_fwd_ex
    torch.cuda.synchronize()
    print("[bench] %s inputs ready in %.1fs; plan %s grid=%d block_m=%d block_n=%d nsplit=%d" %
          (w.describe(), time.time() - t0, plan.kernel.decode(), plan.grid, plan.block_m,
           plan.block_n, nsplit), file=sys.stderr, flush=True)

    def step():
        rc = launch(*args_c)
        if rc != 0:
            raise fa.AttnError(rc, fa.attn_strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    # Timed region: K back-to-back launches between two HIP events on the launch stream
    # (per-launch events would put their own packets between the kernels).
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    epoch0 = time.time()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # (wall-clock bounds of the timed region, for a clock sampler outside this process)
    print("[bench] timed region epoch %.3f %.3f" % (epoch0, epoch0 + wall), file=sys.stderr,
          flush=True)
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = e0.elapsed_time(e1) / args.steps
    flops = flops_workload(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg * 1e-3) / 1e12
    print("[bench] kernel ms (events, mean over %d launches) %.4f; wall/step %.4f ms" %
          (args.steps, kern_avg, ms_per_step), file=sys.stderr, flush=True)

    # Per-launch distribution, outside the timed region: each launch between its own pair
    # of events (the events' own packets sit between the kernels here).
    per = []
    for _ in range(min(args.steps, 100)):
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        step()
        a1.record(stream)
        torch.cuda.synchronize()
        per.append(a0.elapsed_time(a1))
    per.sort()
    try:
        peak_rt, cus, khz = fa.attn_device_peak()
    except fa.AttnError:
        peak_rt, cus, khz = None, None, None

    sclk = None
    if not args.no_clock:
        def busy():
            for _ in range(10):
                step()
            torch.cuda.synchronize()
        sclk = sample_sclk(poller, busy)

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: %d bytes read, %d bytes written" % (2 * n, 2 * n),
              file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_TFLOPS[name], 2) if name in PAGES_TFLOPS else None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq,
                   "Lk": w.Lk, "D": w.D, "in_dtype": w.dtype, "k_mult": w.k_mult,
                   "scale": scale, "causal": w.causal, "nsplit": nsplit,
                   "kernel": plan.kernel.decode(), "block_m": plan.block_m,
                   "block_n": plan.block_n, "grid": plan.grid},
        "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
        "kernel_ms_mean": round(kern_avg, 4),
        "kernel_ms_median": round(per[len(per) // 2], 4),
        "kernel_ms_min": round(per[0], 4),
        "peak_runtime_tflops": round(peak_rt, 1) if peak_rt else None,
        "device": {"compute_units": cus, "peak_clock_mhz": khz / 1000 if khz else None,
                   "sclk_mhz_under_load": sclk},
        # the same kernel time against the MFMA peak at the clock measured under this load
        "frac_at_measured_clock": (round(achieved / (cus * sclk * 1e6 * 4096 / 1e12), 4)
                                   if sclk and cus else None),
        "tflops_pages_formula": (round(flops_pages(w.Lq, w.Lk, w.D, w.Hq, w.B) /
                                       (ms_per_step * 1e-3) / 1e12, 2)
                                 if not w.causal else None),
        "roofline": None,
        "cpu_baseline": None,
    }
    traffic = measured_traffic(name)
    # The bound follows the arithmetic intensity over the algorithmic bytes (Q, K, V, O and
    # LSE once; a split's partial results are not the method's bytes): below the machine
    # balance (peak flop/s over HBM bytes/s) HBM bounds the step, above it the MFMAs.
    abytes = algorithmic_bytes(w)
    if flops / abytes < PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        gbs = abytes / (kern_avg * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                           "traffic": traffic, "algorithmic_bytes_per_launch": abytes,
                           "algorithmic_flops_per_launch": flops}
    else:
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2),
                           "peak": round(PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                           "algorithmic_flops_per_launch": flops,
                           "algorithmic_bytes_per_launch": abytes}

    if not args.no_cpu:
        import oracle
        rows = attn_inputs.sample_rows(w, n_random=min(args.cpu_rows, w.B * w.Hq * w.Lq))
        threads = len(os.sched_getaffinity(0))
        orc = oracle.default()
        c0 = time.perf_counter()
        o_ref, lse_ref = orc.attention(q, k, v, scale, rows=rows, nthreads=threads,
                                       causal=w.causal)
        csec = time.perf_counter() - c0
        i_rows = np.asarray(rows) % w.Lq
        nvis = (np.clip(i_rows + w.Lk - w.Lq + 1, 0, w.Lk) if w.causal
                else np.full(len(rows), w.Lk))
        cpu_flops = 4 * w.D * int(nvis.sum())
        cm = compare_rows(o.cpu(), lse.cpu(), rows, o_ref, lse_ref)
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        out["cpu_baseline"] = {
            "value": round(cpu_flops / csec / 1e12, 6), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model,
            "ms_per_row": round(csec * 1e3 / len(rows), 4),
            "sample": "%d query rows of this workload (seeded: %d random + first/last tiles "
                      "and end rows of every head), fp64, %.1f s; extrapolated full oracle "
                      "%.0f s" % (len(rows), min(args.cpu_rows, w.B * w.Hq * w.Lq), csec,
                                  csec * flops / cpu_flops)}
        out["parity_on_sample"] = cm
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
