"""MI355X (gfx950) fused attention forward: a thin ctypes binding over libattn.so.

The functions here only marshal arguments into the C ABI declared in
include/attn.h; every step of the computation runs in the HIP kernels of
libattn.so.  There is no fallback: if the library is missing or fails to
load, every call raises.

    o, lse = flash_attention_amd.fwd(q, k, v)          # torch tensors on the GPU

Layouts: q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D], contiguous, fp16 or bf16,
D in {128, 256}, Hq a multiple of Hkv.  o has q's dtype; lse is float32
[B,Hq,Lq] (natural log).
"""
import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F16, ATTN_BF16 = 0, 1
ATTN_OK = 0
ERROR_CODES = {
    -1: "ATTN_E_NULLPTR", -2: "ATTN_E_SHAPE", -3: "ATTN_E_HEADDIM", -4: "ATTN_E_GQA",
    -5: "ATTN_E_DTYPE", -6: "ATTN_E_SCALE", -7: "ATTN_E_ALIGN", -8: "ATTN_E_ALIAS",
    -9: "ATTN_E_LAUNCH",
}

_I64 = ctypes.c_int64
_VP = ctypes.c_void_p


class AttnPlan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("kernel", ctypes.c_char * 64)]


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERROR_CODES.get(code, "?"), code, msg))
        self.code = code


_lib = None


def lib():
    """Load libattn.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libattn.so is not built (%s); run `python -m "
                              "flash_attention_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        shape = [_I64] * 6
        L.attn_fwd.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape + [ctypes.c_float, ctypes.c_int]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_fwd_stream.argtypes = L.attn_fwd.argtypes + [_VP]
        L.attn_fwd_stream.restype = ctypes.c_int
        L.attn_validate.argtypes = L.attn_fwd.argtypes
        L.attn_validate.restype = ctypes.c_int
        L.attn_strerror.argtypes = [ctypes.c_int]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_plan.argtypes = shape + [ctypes.c_int, ctypes.POINTER(AttnPlan)]
        L.attn_plan.restype = ctypes.c_int
        L.attn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


# --- the C ABI, one Python function per entry point (same names, same arguments) ---

def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype):
    return lib().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype)


def attn_fwd_stream(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, stream):
    return lib().attn_fwd_stream(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype,
                                 stream)


def attn_validate(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype):
    return lib().attn_validate(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype)


def attn_strerror(code):
    return lib().attn_strerror(code).decode()


def attn_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype):
    """Return the planner's AttnPlan for a problem, or raise AttnError."""
    p = AttnPlan()
    rc = lib().attn_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, ctypes.byref(p))
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return p


def attn_version():
    return lib().attn_version().decode()


# --- torch convenience wrapper (marshalling only) ---

def dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError("q, k, v must be float16 or bfloat16, got %s" % t.dtype)


def fwd(q, k, v, scale=None, out=None, lse=None, return_lse=True, stream=None):
    """Attention forward on torch GPU tensors; returns (o, lse) (lse None if not asked).

    scale defaults to 1/sqrt(D).  out / lse may be preallocated ([B,Hq,Lq,D] of q's
    dtype, [B,Hq,Lq] float32).  Runs on `stream` (a torch.cuda.Stream) or the current
    stream.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dim() != 4:
            raise ValueError("%s must be 4-D [B,H,L,D]" % name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = attn_fwd_stream(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Lq, Lk, D,
                         float(scale), dtype_code(q), s.cuda_stream)
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return out, lse
