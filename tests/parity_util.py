"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle on the
same 16-bit inputs, and compare with the tolerances of the attention contract.

Tolerances (fixed for this method: fp32 accumulation, 16-bit inputs):
  fp16 inputs: relative RMS error <= 2e-3 and max |error| <= 1e-2
  bf16 inputs: relative RMS error <= 1e-2 (and max |error| <= 0.15, the bf16 threshold of
               "Xe2 Sdp Bf16", section "Correctness Testing")
  LSE: |error| <= 1e-3
Any NaN/Inf in O or LSE for finite inputs fails before the error metrics are looked at
(NaN count first: "Xe2 ... Flash Attention -- HD=256", section "Performance Testing").
The one exception is a row that sees no key under the causal mask (Lq > Lk): there the
oracle's LSE is -inf and its O is 0, and the GPU must give exactly those values.
"""
import math

import numpy as np
import torch

import flash_attention_amd as fa
import oracle

TOL = {"f16": dict(rel_rms=2e-3, max_abs=1e-2), "bf16": dict(rel_rms=1e-2, max_abs=0.15)}
LSE_ABS = 1e-3


def gpu_fwd(q, k, v, scale, with_lse=True, causal=False, nsplit=1):
    """Run the HIP path on CPU 16-bit tensors; outputs are NaN-poisoned first so any
    element the kernel fails to write shows up.  Returns CPU tensors (o, lse)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev) if with_lse else None
    fa.fwd(qd, kd, vd, scale=scale, out=o, lse=lse, return_lse=with_lse, causal=causal,
           nsplit=nsplit)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if with_lse else None)


def metrics(o_gpu_rows, lse_gpu_rows, o_ref, lse_ref):
    og = o_gpu_rows.to(torch.float64).numpy()
    nan_o = int((~np.isfinite(og)).sum())
    lg = lse_gpu_rows.to(torch.float64).numpy() if lse_gpu_rows is not None else None
    empty = np.isneginf(lse_ref)  # rows that see no key: exact values required
    nan_l = int((~np.isfinite(lg[~empty])).sum()) if lg is not None else 0
    err = og - o_ref
    out = dict(nan_o=nan_o, nan_lse=nan_l, empty_rows=int(empty.sum()),
               empty_wrong=int((og[empty] != 0).sum()) + (int((lg[empty] != -np.inf).sum())
                                                          if lg is not None else 0),
               rel_rms=float(np.sqrt((err ** 2).sum() / max((o_ref ** 2).sum(), 1e-300))),
               max_abs=float(np.abs(err).max()) if err.size else 0.0)
    if lg is not None:
        d = lg[~empty] - lse_ref[~empty]
        out["lse_abs"] = float(np.abs(d).max()) if d.size else 0.0
    return out


def check(m, dtype, what=""):
    assert m["nan_o"] == 0 and m["nan_lse"] == 0, ("non-finite outputs", what, m)
    assert m.get("empty_wrong", 0) == 0, ("empty rows not O = 0, LSE = -inf", what, m)
    tol = TOL[dtype]
    assert m["rel_rms"] <= tol["rel_rms"], ("rel_rms", what, m)
    assert m["max_abs"] <= tol["max_abs"], ("max_abs", what, m)
    if "lse_abs" in m:
        assert m["lse_abs"] <= LSE_ABS, ("lse_abs", what, m)


def parity(q, k, v, scale, dtype, rows=None, what="", causal=False, nsplit=1):
    """GPU vs oracle on all rows (rows=None) or on the given flat rows.  The oracle gets
    the float32 value of scale, the value the kernel receives."""
    scale = float(np.float32(scale))
    o, lse = gpu_fwd(q, k, v, scale, causal=causal, nsplit=nsplit)
    B, Hq, Lq, D = q.shape
    of = o.reshape(-1, D)
    lf = lse.reshape(-1)
    if rows is None:
        o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
        m = metrics(of, lf, o_ref, lse_ref)
    else:
        idx = torch.from_numpy(np.asarray(rows, dtype=np.int64))
        o_ref, lse_ref = oracle.attention(q, k, v, scale, rows=rows, causal=causal)
        m = metrics(of[idx], lf[idx], o_ref, lse_ref)
        # every row, sampled or not, must be written: no NaN poison left (empty causal rows
        # hold LSE -inf, which is not NaN)
        m["nan_o"] += int(torch.isnan(of.float()).sum())
        m["nan_lse"] += int(torch.isnan(lf).sum())
    print("[parity] %s %s" % (what, {kk: (round(vv, 7) if isinstance(vv, float) else vv)
                                     for kk, vv in m.items()}), flush=True)
    check(m, dtype, what)
    return o, lse, m


def scale_of(D):
    return 1.0 / math.sqrt(D)
