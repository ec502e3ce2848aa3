"""fp64 CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may import this package.  The HIP library never does, and this
package imports nothing from it: the two share no code.

Two independent implementations live here:

* ``liboracle.so`` (attn_oracle.c): the plain definition -- scores, row
  softmax, weighted sum of V, natural-log LSE, optionally causal or over a
  slice of the keys -- in fp64 with OpenMP over query rows, and the merge of
  partial results by their LSE.  This is the oracle the GPU path is judged
  against.
* ``numpy_ref.attention`` (numpy_ref.py): the same definition written with
  NumPy array operations, used only on tiny shapes to cross-check the C code.

Inputs are fp16/bf16 tensors (widened exactly to fp64 inside the oracle) or
float64 arrays.  Layouts: Q [B,Hq,Lq,D]; K, V [B,Hkv,Lk,D]; outputs are
float64 O rows [n, D] and LSE [n].
"""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F16, BF16 = 0, 1

_I64 = ctypes.c_int64
_PTR = ctypes.c_void_p


class Oracle:
    """ctypes wrapper around one build of attn_oracle.c."""

    def __init__(self, path=LIB_PATH):
        if not os.path.exists(path):
            # built on first use, but never from a process that already drives the GPU (the
            # compiler would start from it): build the oracle before any GPU work instead
            torch = sys.modules.get("torch")
            if torch is not None and torch.cuda.is_initialized():
                raise RuntimeError("%s is not built; run `python -m oracle.build` (or "
                                   "__graft_entry__.build()) before using the GPU" % path)
            from . import build as _b
            _b.build(out=path, quiet=True)
        self.path = path
        self.lib = ctypes.CDLL(path)
        lib = self.lib
        common = [_I64] * 6 + [ctypes.c_double, ctypes.c_int, _I64, _I64, _PTR, _I64, _PTR, _PTR,
                               ctypes.c_int]
        lib.oracle_attn_rows_f64.argtypes = [_PTR, _PTR, _PTR] + common
        lib.oracle_attn_rows_f64.restype = ctypes.c_int
        lib.oracle_attn_rows_u16.argtypes = [_PTR, _PTR, _PTR, ctypes.c_int] + common
        lib.oracle_attn_rows_u16.restype = ctypes.c_int
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [_PTR, _PTR, _I64, _I64, _I64, _PTR, _PTR]
        lib.oracle_merge.restype = ctypes.c_int

    def max_threads(self):
        return int(self.lib.oracle_max_threads())

    def widen(self, bits, dtype):
        fn = self.lib.oracle_bf16_to_double if dtype == BF16 else self.lib.oracle_f16_to_double
        return fn(int(bits))

    def attention(self, q, k, v, scale, rows=None, nthreads=0, causal=False, key_begin=0,
                  lk_total=None):
        """Attention rows from the plain definition, in fp64.

        q, k, v: torch tensors (float16 / bfloat16 / float64, CPU) or numpy
        arrays (float16 / float64), layouts [B,Hq,Lq,D] and [B,Hkv,Lk,D].
        scale: the softmax scale (pass the float32 value the GPU receives).
        rows: optional int64 array of flat row indices (b*Hq + h)*Lq + i;
        None means every row in order.
        causal: row i sees global key j only if j <= i + lk_total - Lq.
        key_begin, lk_total: k and v hold keys [key_begin, key_begin + Lk) of a
        sequence of lk_total keys (default: the whole sequence, lk_total = Lk);
        the result is then the partial attention over that slice.
        Returns (O [n, D] float64, LSE [n] float64) as numpy arrays; a row that
        sees no key has O = 0 and LSE = -inf.
        """
        qa, dtype = _as_array(q)
        ka, kd = _as_array(k)
        va, vd = _as_array(v)
        if not (dtype == kd == vd):
            raise TypeError("q, k, v must share one dtype")
        if qa.ndim != 4 or ka.ndim != 4 or va.ndim != 4:
            raise ValueError("q, k, v must be 4-D [B,H,L,D]")
        B, Hq, Lq, D = qa.shape
        Bk, Hkv, Lk, Dk = ka.shape
        if (Bk, Dk) != (B, D) or va.shape != ka.shape:
            raise ValueError("shape mismatch: q %s k %s v %s" % (qa.shape, ka.shape, va.shape))
        if rows is None:
            n = B * Hq * Lq
            rows_arr = None
            rows_ptr = None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            n = rows_arr.size
            rows_ptr = rows_arr.ctypes.data
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        lk_total = Lk if lk_total is None else int(lk_total)
        args = (B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)), int(key_begin), lk_total,
                rows_ptr, n, o.ctypes.data, lse.ctypes.data, int(nthreads))
        if dtype == "f64":
            rc = self.lib.oracle_attn_rows_f64(qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
                                               *args)
        else:
            code = F16 if dtype == "f16" else BF16
            rc = self.lib.oracle_attn_rows_u16(qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
                                               code, *args)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (code %d)" % rc)
        return o, lse

    def merge(self, o_parts, lse_parts):
        """Merge partial results over disjoint key ranges (fp64).

        o_parts [P, n, D] and lse_parts [P, n] (array-likes, any float type):
        part g of row r is the attention of row r over key range g alone.
        Returns (O [n, D], LSE [n]) float64 with LSE = ln sum_g exp(LSE_g) and
        O = sum_g exp(LSE_g - LSE) O_g.
        """
        op = np.ascontiguousarray(np.asarray(o_parts, dtype=np.float64))
        lp = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
        if op.ndim != 3 or lp.shape != op.shape[:2]:
            raise ValueError("o_parts must be [P,n,D] and lse_parts [P,n]")
        P, n, D = op.shape
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self.lib.oracle_merge(op.ctypes.data, lp.ctypes.data, P, n, D, o.ctypes.data,
                                   lse.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (code %d)" % rc)
        return o, lse


def _as_array(x):
    """Return (contiguous numpy array, dtype tag); 16-bit data as raw uint16 bits."""
    try:
        import torch
    except ImportError:  # pragma: no cover - torch is always present here
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.float16:
            return x.view(torch.int16).numpy().view(np.uint16), "f16"
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), "bf16"
        if x.dtype == torch.float64:
            return x.numpy(), "f64"
        raise TypeError("unsupported tensor dtype %s" % x.dtype)
    a = np.ascontiguousarray(x)
    if a.dtype == np.float16:
        return a.view(np.uint16), "f16"
    if a.dtype == np.float64:
        return a, "f64"
    raise TypeError("unsupported array dtype %s" % a.dtype)


_default = None


def default():
    """The oracle built from oracle/attn_oracle.c (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(q, k, v, scale, rows=None, nthreads=0, causal=False, key_begin=0, lk_total=None):
    return default().attention(q, k, v, scale, rows=rows, nthreads=nthreads, causal=causal,
                               key_begin=key_begin, lk_total=lk_total)


def merge(o_parts, lse_parts):
    return default().merge(o_parts, lse_parts)
