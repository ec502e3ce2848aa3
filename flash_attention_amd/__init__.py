"""MI355X (gfx950) fused attention forward: a thin ctypes binding over libattn.so.

The functions here only marshal arguments into the C ABI declared in
include/attn.h; every step of the computation runs in the HIP kernels of
libattn.so.  There is no fallback: if the library is missing or fails to
load, every call raises.

    o, lse = flash_attention_amd.fwd(q, k, v)          # torch tensors on the GPU
    o, lse = flash_attention_amd.fwd(q, k, v, causal=True, nsplit=0)

Layouts: q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D], contiguous, fp16 or bf16,
D in {128, 256}, Hq a multiple of Hkv.  o has q's dtype; lse is float32
[B,Hq,Lq] (natural log).  Partial results over key splits are float32
[nsplit,B,Hq,Lq,D] and [nsplit,B,Hq,Lq].
"""
import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F16, ATTN_BF16, ATTN_F32 = 0, 1, 2
ATTN_CAUSAL = 1
ATTN_MAX_SPLITS = 256
ATTN_NOALLOC_WORKSPACE_BYTES = 64 << 20
ATTN_OK = 0
ERROR_CODES = {
    -1: "ATTN_E_NULLPTR", -2: "ATTN_E_SHAPE", -3: "ATTN_E_HEADDIM", -4: "ATTN_E_GQA",
    -5: "ATTN_E_DTYPE", -6: "ATTN_E_SCALE", -7: "ATTN_E_ALIGN", -8: "ATTN_E_LAUNCH",
    -9: "ATTN_E_ALIAS", -10: "ATTN_E_FLAGS", -11: "ATTN_E_SPLIT", -12: "ATTN_E_WORKSPACE",
}

_I64 = ctypes.c_int64
_VP = ctypes.c_void_p


class AttnPlan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("kernel", ctypes.c_char * 64),
                ("nsplit", ctypes.c_int32), ("split_len", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


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
        U32 = ctypes.c_uint32
        L.attn_fwd_ex.argtypes = L.attn_fwd.argtypes + [U32, _I64, _VP, _I64, _VP]
        L.attn_fwd_ex.restype = ctypes.c_int
        L.attn_validate_ex.argtypes = L.attn_fwd.argtypes + [U32, _I64]
        L.attn_validate_ex.restype = ctypes.c_int
        L.attn_fwd_partial.argtypes = L.attn_fwd.argtypes + [U32, _I64, _VP]
        L.attn_fwd_partial.restype = ctypes.c_int
        L.attn_validate_partial.argtypes = L.attn_fwd.argtypes + [U32, _I64]
        L.attn_validate_partial.restype = ctypes.c_int
        L.attn_merge.argtypes = [_VP, _VP, _I64, _I64, _I64, _VP, _VP, ctypes.c_int, _VP]
        L.attn_merge.restype = ctypes.c_int
        L.attn_validate_merge.argtypes = [_VP, _VP, _I64, _I64, _I64, _VP, _VP, ctypes.c_int]
        L.attn_validate_merge.restype = ctypes.c_int
        L.attn_split_range.argtypes = [_I64, _I64, _I64, ctypes.POINTER(_I64),
                                       ctypes.POINTER(_I64)]
        L.attn_split_range.restype = ctypes.c_int
        L.attn_workspace_bytes.argtypes = [_I64] * 5
        L.attn_workspace_bytes.restype = _I64
        L.attn_plan_ex.argtypes = shape + [ctypes.c_int, U32, ctypes.POINTER(AttnPlan)]
        L.attn_plan_ex.restype = ctypes.c_int
        L.attn_fwd_ex_noalloc.argtypes = L.attn_fwd.argtypes + [U32, _I64, _VP]
        L.attn_fwd_ex_noalloc.restype = ctypes.c_int
        L.attn_device_peak.argtypes = [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_int32)]
        L.attn_device_peak.restype = ctypes.c_int
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


def attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags, nsplit,
                workspace, workspace_bytes, stream):
    return lib().attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags,
                             nsplit, workspace, workspace_bytes, stream)


def attn_fwd_ex_noalloc(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags,
                        nsplit, stream):
    return lib().attn_fwd_ex_noalloc(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype,
                                     flags, nsplit, stream)


def attn_validate_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags, nsplit):
    return lib().attn_validate_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype,
                                  flags, nsplit)


def attn_fwd_partial(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags,
                     nsplit, stream):
    return lib().attn_fwd_partial(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, D, scale,
                                  in_dtype, flags, nsplit, stream)


def attn_validate_partial(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype,
                          flags, nsplit):
    return lib().attn_validate_partial(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, D, scale,
                                       in_dtype, flags, nsplit)


def attn_merge(o_part, lse_part, nsplit, rows, D, o, lse, out_dtype, stream):
    return lib().attn_merge(o_part, lse_part, nsplit, rows, D, o, lse, out_dtype, stream)


def attn_validate_merge(o_part, lse_part, nsplit, rows, D, o, lse, out_dtype):
    return lib().attn_validate_merge(o_part, lse_part, nsplit, rows, D, o, lse, out_dtype)


def attn_split_range(Lk, nsplit, s):
    """(begin, end) of key split s, or raise AttnError."""
    b, e = _I64(), _I64()
    rc = lib().attn_split_range(Lk, nsplit, s, ctypes.byref(b), ctypes.byref(e))
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return b.value, e.value


def attn_workspace_bytes(B, Hq, Lq, D, nsplit):
    return lib().attn_workspace_bytes(B, Hq, Lq, D, nsplit)


def attn_device_peak():
    """(peak TFLOP/s, compute units, clock kHz) of the current device, or raise AttnError."""
    t, cu, khz = ctypes.c_double(), ctypes.c_int32(), ctypes.c_int32()
    rc = lib().attn_device_peak(ctypes.byref(t), ctypes.byref(cu), ctypes.byref(khz))
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return t.value, cu.value, khz.value


def attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, in_dtype, flags):
    """Return the planner's AttnPlan for attn_fwd_ex with nsplit = 0, or raise AttnError."""
    p = AttnPlan()
    rc = lib().attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, in_dtype, flags, ctypes.byref(p))
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return p


# --- torch convenience wrapper (marshalling only) ---

def dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError("q, k, v must be float16 or bfloat16, got %s" % t.dtype)


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dim() != 4:
            raise ValueError("%s must be 4-D [B,H,L,D]" % name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    return B, Hq, Hkv, Lq, Lk, D


def _check_out(name, t, shape, dtype, device):
    """A caller-provided output must match exactly what the kernel writes."""
    if t.device != device:
        raise ValueError("%s must be on %s, not %s" % (name, device, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, not %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def fwd(q, k, v, scale=None, out=None, lse=None, return_lse=True, stream=None, causal=False,
        nsplit=1, workspace=None):
    """Attention forward on torch GPU tensors; returns (o, lse) (lse None if not asked).

    scale defaults to 1/sqrt(D).  out / lse may be preallocated ([B,Hq,Lq,D] of q's
    dtype, [B,Hq,Lq] float32).  Runs on `stream` (a torch.cuda.Stream) or the current
    stream.  causal: row i sees key j only if j <= i + Lk - Lq.  nsplit: key splits (1: one
    pass; 0: the planner's choice; >1: split keys and merge).  A split run needs a
    workspace (a uint8 GPU tensor of at least attn_workspace_bytes bytes); one is allocated
    with torch when none is given.
    """
    import torch
    B, Hq, Hkv, Lq, Lk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out("out", out, tuple(q.shape), q.dtype, q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    if workspace is not None:
        _check_out("workspace", workspace, tuple(workspace.shape), torch.uint8, q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    flags = ATTN_CAUSAL if causal else 0
    lse_ptr = lse.data_ptr() if lse is not None else None
    if nsplit == 1 and not causal and workspace is None:
        rc = attn_fwd_stream(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                             B, Hq, Hkv, Lq, Lk, D, float(scale), dtype_code(q), s.cuda_stream)
    else:
        # nsplit = 0 goes to the library as is: its planner picks the splits (and, for
        # key/value groups of 129-256 rows, the tile shape); the workspace is sized from the
        # same plan
        need = (attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, dtype_code(q), flags).workspace_bytes
                if nsplit == 0 else attn_workspace_bytes(B, Hq, Lq, D, nsplit))
        if need < 0:
            raise AttnError(need, attn_strerror(need))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        rc = attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B,
                         Hq, Hkv, Lq, Lk, D, float(scale), dtype_code(q), flags, nsplit, ws_ptr,
                         ws_bytes, s.cuda_stream)
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return out, lse


def fwd_partial(q, k, v, nsplit, scale=None, causal=False, stream=None):
    """Partial results over nsplit key ranges: (o_part [nsplit,B,Hq,Lq,D] fp32,
    lse_part [nsplit,B,Hq,Lq] fp32); split s covers attn_split_range(Lk, nsplit, s)."""
    import torch
    B, Hq, Hkv, Lq, Lk, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o_part = torch.empty((nsplit, B, Hq, Lq, D), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((nsplit, B, Hq, Lq), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = attn_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                          lse_part.data_ptr(), B, Hq, Hkv, Lq, Lk, D, float(scale),
                          dtype_code(q), ATTN_CAUSAL if causal else 0, nsplit, s.cuda_stream)
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return o_part, lse_part


def merge(o_part, lse_part, out_dtype=None, lse=True, stream=None):
    """Merge partial results o_part [P,...,D] fp32, lse_part [P,...] fp32 into
    (o [...,D] of out_dtype (torch dtype, default float32), lse [...] float32 or None)."""
    import torch
    if not (o_part.is_cuda and lse_part.is_cuda):
        raise ValueError("o_part and lse_part must be GPU tensors")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise TypeError("partial results must be float32")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("partial results must be contiguous")
    if tuple(o_part.shape[:-1]) != tuple(lse_part.shape):
        raise ValueError("o_part %s and lse_part %s disagree" % (tuple(o_part.shape),
                                                                 tuple(lse_part.shape)))
    P, D = o_part.shape[0], o_part.shape[-1]
    rows = lse_part.numel() // P
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    code = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}[out_dtype]
    o = torch.empty(tuple(o_part.shape[1:]), dtype=out_dtype, device=o_part.device)
    lse_t = torch.empty(tuple(lse_part.shape[1:]), dtype=torch.float32,
                        device=o_part.device) if lse else None
    s = stream if stream is not None else torch.cuda.current_stream(o_part.device)
    rc = attn_merge(o_part.data_ptr(), lse_part.data_ptr(), P, rows, D, o.data_ptr(),
                    lse_t.data_ptr() if lse_t is not None else None, code, s.cuda_stream)
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))
    return o, lse_t
