"""The C ABI on the CPU: the library loads, exports every function include/attn.h
declares, and the host-side validation and planner behave as documented.  No
compute call is made (no GPU here)."""
import ctypes
import math
import os
import re

import pytest

import flash_attention_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(attn_[a-z_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def declared_codes():
    text = open(HEADER).read()
    return {name: int(val) for name, val in re.findall(r"(ATTN_E_[A-Z]+|ATTN_OK)\s*=\s*(-?\d+)",
                                                       text)}


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("attn_fwd", "attn_fwd_stream", "attn_validate", "attn_strerror", "attn_plan",
                 "attn_version"):
        assert must in names, names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), "libattn.so does not export %s" % name


def test_python_binding_mirrors_the_c_names():
    for name in declared_functions():
        assert callable(getattr(fa, name)), name


def test_error_codes_match_header():
    codes = declared_codes()
    assert codes["ATTN_OK"] == fa.ATTN_OK == 0
    for name, val in codes.items():
        if name != "ATTN_OK":
            assert fa.ERROR_CODES[val] == name
            assert fa.attn_strerror(val) and fa.attn_strerror(val) != "unknown error code"
    assert fa.attn_strerror(12345) == "unknown error code"


# Fake, well-separated, 256-byte aligned device addresses: validation only compares them.
GB = 1 << 30
Q, K, V, O, L = 1 * GB, 3 * GB, 5 * GB, 7 * GB, 9 * GB
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, Hq=32, Hkv=2, Lq=4096, Lk=4096, D=256,
            scale=1 / 16, in_dtype=fa.ATTN_F16)


def validate(**over):
    a = dict(GOOD)
    a.update(over)
    return fa.attn_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Lq"], a["Lk"], a["D"], a["scale"], a["in_dtype"])


def test_validate_accepts_good_arguments():
    assert validate() == 0
    assert validate(lse=None) == 0
    assert validate(D=128, in_dtype=fa.ATTN_BF16, Hkv=8) == 0
    assert validate(Lq=1, Lk=1, Hq=1, Hkv=1) == 0
    assert validate(Lq=17, Lk=33) == 0  # ragged sizes are supported
    assert validate(scale=0.0) == 0 and validate(scale=-0.5) == 0


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(Lq=0), -2), (dict(Lk=-1), -2),
    (dict(Lq=(1 << 31) // 256 + 1), -2), (dict(Lk=1 << 24), -2),
    (dict(D=64), -3), (dict(D=192), -3), (dict(D=512), -3),
    (dict(Hq=32, Hkv=3), -4), (dict(Hq=2, Hkv=4), -4),
    (dict(in_dtype=2), -5), (dict(in_dtype=-1), -5),
    (dict(scale=math.inf), -6), (dict(scale=math.nan), -6), (dict(scale=-math.inf), -6),
    (dict(q=Q + 8), -7), (dict(k=K + 2), -7), (dict(v=V + 4), -7), (dict(o=O + 1), -7),
    (dict(lse=L + 2), -7),
    (dict(o=Q), -8), (dict(o=K + 4096), -8), (dict(o=V), -8), (dict(lse=O + 256), -8),
    (dict(lse=Q), -8), (dict(lse=K), -8),
])
def test_validate_rejects(over, code):
    assert validate(**over) == code


def test_validate_grid_limit():
    # a grid of 2^31 or more workgroups is refused, not truncated
    assert validate(B=1 << 20, Hq=1 << 11, Hkv=1, Lq=128, Lk=128) == -2


def test_lse_may_follow_o_directly():
    qbytes = 1 * 32 * 4096 * 256 * 2
    assert validate(lse=O + qbytes) == 0
    assert validate(lse=O + qbytes - 4) == -8


@pytest.mark.parametrize("D,dtype", [(128, fa.ATTN_F16), (128, fa.ATTN_BF16),
                                     (256, fa.ATTN_F16), (256, fa.ATTN_BF16)])
def test_plan(D, dtype):
    p = fa.attn_plan(2, 8, 2, 1000, 777, D, dtype)
    assert p.waves >= 1 and p.block_m % 32 == 0 and p.block_n % 32 == 0
    assert p.grid == math.ceil(1000 / p.block_m) * 8 * 2
    assert 0 < p.lds_bytes <= 160 * 1024
    assert p.kernel.decode().startswith("attn_fwd_d%d" % D)


def test_plan_rejects_like_validate():
    with pytest.raises(fa.AttnError) as e:
        fa.attn_plan(1, 4, 3, 64, 64, 128, fa.ATTN_F16)
    assert e.value.code == -4


def test_version():
    assert re.match(r"^\d+\.\d+\.\d+$", fa.attn_version())
