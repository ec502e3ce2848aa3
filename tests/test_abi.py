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
                 "attn_version", "attn_fwd_ex", "attn_validate_ex", "attn_fwd_partial",
                 "attn_validate_partial", "attn_merge", "attn_validate_merge",
                 "attn_split_range", "attn_workspace_bytes", "attn_plan_ex"):
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
    (dict(B=-1), -2), (dict(Hq=-1), -2), (dict(Hkv=0), -2), (dict(Hkv=-2), -2), (dict(Lq=-1), -2),
    (dict(Lk=-1), -2), (dict(k=None), -1), (dict(v=None), -1),
    (dict(Lq=(1 << 31) // 256 + 1), -2), (dict(Lk=1 << 24), -2),
    (dict(D=64), -3), (dict(D=192), -3), (dict(D=512), -3),
    (dict(Hq=32, Hkv=3), -4), (dict(Hq=2, Hkv=4), -4),
    (dict(in_dtype=2), -5), (dict(in_dtype=-1), -5),
    (dict(scale=math.inf), -6), (dict(scale=math.nan), -6), (dict(scale=-math.inf), -6),
    (dict(q=Q + 8), -7), (dict(k=K + 2), -7), (dict(v=V + 4), -7), (dict(o=O + 1), -7),
    (dict(lse=L + 2), -7),
    (dict(o=Q), -9), (dict(o=K + 4096), -9), (dict(o=V), -9), (dict(lse=O + 256), -9),
    (dict(lse=Q), -9), (dict(lse=K), -9),
])
def test_validate_rejects(over, code):
    assert validate(**over) == code


def test_validate_grid_limit():
    # a grid of 2^31 or more workgroups is refused, not truncated: 2^21 batches of one
    # key/value head with 2048 query heads x 128 rows (1024 tiles of 256 rows)
    assert validate(B=1 << 21, Hq=1 << 11, Hkv=1, Lq=128, Lk=128) == -2
    # the query rows of one key/value group (Hq/Hkv * Lq) * D stay below 2^31
    assert validate(Hq=256, Hkv=1, Lq=(1 << 31) // 256 // 256 + 1, Lk=64) == -2


def test_validate_exact_length_limits():
    # per-head offsets are 32-bit: Lk*D and (Hq/Hkv)*Lq*D up to 2^31 - 1 are accepted, one
    # more row or key is refused (addresses far apart: the tensors span gigabytes here)
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, lse=5 << 40)
    for D in (128, 256):
        lim = ((1 << 31) - 1) // D
        assert validate(**far, D=D, Hq=2, Hkv=1, Lq=40, Lk=lim) == 0
        assert validate(**far, D=D, Hq=2, Hkv=1, Lq=40, Lk=lim + 1) == -2
        assert validate(**far, D=D, Hq=1, Hkv=1, Lq=lim, Lk=33) == 0
        assert validate(**far, D=D, Hq=1, Hkv=1, Lq=lim + 1, Lk=33) == -2
        assert validate(**far, D=D, Hq=16, Hkv=1, Lq=lim // 16, Lk=33) == 0
        assert validate(**far, D=D, Hq=16, Hkv=1, Lq=lim // 16 + 1, Lk=33) == -2


def test_empty_sizes():
    # No query rows (B, Hq or Lq = 0): nothing to compute.  No keys (Lk = 0): every row's
    # softmax is over an empty set, O = 0 and LSE = -inf.  Both are valid calls.
    assert validate(B=0) == 0 and validate(Hq=0) == 0 and validate(Lq=0) == 0
    assert validate(Lk=0) == 0 and validate(Lk=0, Lq=0) == 0
    # a tensor of no elements may be NULL; one with elements may not
    assert validate(q=None, o=None, lse=None, Lq=0) == 0
    assert validate(q=None, k=None, v=None, o=None, lse=None, B=0) == 0
    assert validate(k=None, v=None, Lk=0) == 0
    assert validate(q=None, Lk=0) == -1 and validate(o=None, Lk=0) == -1
    assert validate(Hq=0, Hkv=0) == -2
    assert fa.attn_plan(1, 32, 2, 0, 4096, 256, fa.ATTN_F16).grid == 0
    assert fa.attn_plan(0, 32, 2, 64, 4096, 256, fa.ATTN_F16).grid == 0
    assert fa.attn_plan_ex(1, 32, 2, 16, 0, 256, fa.ATTN_F16, fa.ATTN_CAUSAL).nsplit == 1
    assert fa.attn_plan_ex(1, 32, 2, 0, 16384, 256, fa.ATTN_F16, 0).nsplit == 1
    assert [fa.attn_split_range(0, 4, s) for s in range(4)] == [(0, 0)] * 4
    assert fa.attn_split_range(0, 1, 0) == (0, 0)
    assert validate_partial(Lq=0, o_part=None, lse_part=None) == 0
    assert validate_partial(Lk=0, k=None, v=None) == 0
    assert validate_partial(Lk=0, o_part=None) == -1


def test_calls_without_query_rows_launch_nothing():
    # with no query row the entry points return ATTN_OK before any HIP call, so this runs
    # without a GPU (and with NULL tensors)
    args = (None, None, None, None, None)
    kv = (None, K, V, None, None)  # keys exist (never read here): their pointers are checked
    assert fa.attn_fwd(*args, 0, 32, 2, 128, 128, 256, 0.0625, fa.ATTN_F16) == 0
    assert fa.attn_fwd_stream(*kv, 1, 32, 2, 0, 128, 128, 0.1, fa.ATTN_BF16, None) == 0
    assert fa.attn_fwd_stream(*args, 1, 32, 2, 0, 128, 128, 0.1, fa.ATTN_BF16, None) == -1
    assert fa.attn_fwd_ex(*args, 1, 0, 2, 16, 0, 256, 0.1, fa.ATTN_F16, fa.ATTN_CAUSAL, 4,
                          None, 0, None) == 0
    assert fa.attn_fwd_ex(*kv, 1, 32, 2, 0, 4096, 256, 0.1, fa.ATTN_F16, 0, 0, None, 0,
                          None) == 0
    assert fa.attn_fwd_partial(*kv, 1, 32, 2, 0, 64, 128, 0.1, fa.ATTN_F16, 0, 3, None) == 0
    assert fa.attn_merge(None, None, 5, 0, 256, None, None, fa.ATTN_F32, None) == 0
    # the checks still run first
    assert fa.attn_fwd(*args, 0, 32, 2, 128, 128, 64, 0.0625, fa.ATTN_F16) == -3
    assert fa.attn_fwd(*args, -1, 32, 2, 128, 128, 256, 0.0625, fa.ATTN_F16) == -2


def test_header_is_plain_c(tmp_path):
    # include/attn.h compiles as strict C99 and a C program links against libattn.so and
    # runs the GPU-free entry points (tests/c/abi_from_c.c)
    import subprocess
    exe = str(tmp_path / "abi_from_c")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_from_c.c")
    libdir = os.path.dirname(fa.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I" + os.path.join(ROOT, "include"), src, "-o", exe, "-L" + libdir,
                    "-lattn", "-Wl,-rpath," + libdir], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_from_c: ok" in r.stdout


def test_binding_output_check():
    # the check fa.fwd applies to caller-provided outputs (pure Python, CPU tensors here)
    import torch
    dev = torch.device("cpu")
    ok = torch.empty(1, 2, 3, 8, dtype=torch.float16)
    fa._check_out("out", ok, (1, 2, 3, 8), torch.float16, dev)
    with pytest.raises(ValueError):
        fa._check_out("out", ok, (1, 2, 4, 8), torch.float16, dev)
    with pytest.raises(TypeError):
        fa._check_out("out", ok, (1, 2, 3, 8), torch.bfloat16, dev)
    with pytest.raises(ValueError):
        fa._check_out("out", ok.transpose(2, 3).contiguous().transpose(2, 3), (1, 2, 3, 8),
                      torch.float16, dev)
    with pytest.raises(ValueError):
        fa._check_out("out", ok, (1, 2, 3, 8), torch.float16, torch.device("cuda:0"))


def test_lse_may_follow_o_directly():
    qbytes = 1 * 32 * 4096 * 256 * 2
    assert validate(lse=O + qbytes) == 0
    assert validate(lse=O + qbytes - 4) == -9


@pytest.mark.parametrize("D,dtype", [(128, fa.ATTN_F16), (128, fa.ATTN_BF16),
                                     (256, fa.ATTN_F16), (256, fa.ATTN_BF16)])
def test_plan(D, dtype):
    p = fa.attn_plan(2, 8, 2, 1000, 777, D, dtype)
    assert p.waves >= 1 and p.block_m % 32 == 0 and p.block_n % 32 == 0
    # the 4 query heads of each key/value head form one block of 4000 rows
    assert p.grid == math.ceil(4 * 1000 / p.block_m) * 2 * 2
    assert 0 < p.lds_bytes <= 160 * 1024
    assert p.kernel.decode().startswith("attn_fwd_d%d" % D)


def test_plan_rejects_like_validate():
    with pytest.raises(fa.AttnError) as e:
        fa.attn_plan(1, 4, 3, 64, 64, 128, fa.ATTN_F16)
    assert e.value.code == -4


def test_version():
    assert re.match(r"^\d+\.\d+\.\d+$", fa.attn_version())


# ---- options: causal flag, key splits, partial results, merge ----

def validate_ex(flags=0, nsplit=1, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.attn_validate_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                               a["Hkv"], a["Lq"], a["Lk"], a["D"], a["scale"], a["in_dtype"],
                               flags, nsplit)


def test_validate_ex():
    assert validate_ex() == 0
    assert validate_ex(flags=fa.ATTN_CAUSAL) == 0
    assert validate_ex(nsplit=0) == 0 and validate_ex(nsplit=fa.ATTN_MAX_SPLITS) == 0
    assert validate_ex(flags=2) == -10 and validate_ex(flags=0x80000000) == -10
    assert validate_ex(nsplit=-1) == -11 and validate_ex(nsplit=fa.ATTN_MAX_SPLITS + 1) == -11
    # the plain checks still run
    assert validate_ex(flags=fa.ATTN_CAUSAL, D=64) == -3 and validate_ex(o=Q) == -9
    # Lq > Lk is allowed under the causal mask (early rows are empty)
    assert validate_ex(flags=fa.ATTN_CAUSAL, Lq=5000, Lk=100) == 0


P_O, P_L = 11 * GB, 13 * GB


def validate_partial(nsplit=4, flags=0, **over):
    a = dict(GOOD, o_part=P_O, lse_part=P_L)
    a.update(over)
    return fa.attn_validate_partial(a["q"], a["k"], a["v"], a["o_part"], a["lse_part"], a["B"],
                                    a["Hq"], a["Hkv"], a["Lq"], a["Lk"], a["D"], a["scale"],
                                    a["in_dtype"], flags, nsplit)


def test_validate_partial():
    assert validate_partial() == 0 and validate_partial(nsplit=1, flags=fa.ATTN_CAUSAL) == 0
    assert validate_partial(lse_part=None) == -1 and validate_partial(o_part=None) == -1
    assert validate_partial(nsplit=0) == -11 and validate_partial(nsplit=257) == -11
    assert validate_partial(flags=4) == -10
    assert validate_partial(o_part=P_O + 4) == -7 and validate_partial(lse_part=P_L + 2) == -7
    assert validate_partial(o_part=Q) == -9 and validate_partial(lse_part=K) == -9
    # o_part of 4 splits: 4 * 32 * 4096 * 256 * 4 bytes = 0.5 GiB; lse_part just after is fine
    pbytes = 4 * 32 * 4096 * 256 * 4
    assert validate_partial(lse_part=P_O + pbytes) == 0
    assert validate_partial(lse_part=P_O + pbytes - 4) == -9
    assert validate_partial(D=100) == -3 and validate_partial(Hkv=5) == -4


def validate_merge(nsplit=3, rows=1000, D=256, out_dtype=fa.ATTN_F16, **over):
    a = dict(o_part=P_O, lse_part=P_L, o=O, lse=L)
    a.update(over)
    return fa.attn_validate_merge(a["o_part"], a["lse_part"], nsplit, rows, D, a["o"], a["lse"],
                                  out_dtype)


def test_validate_merge():
    assert validate_merge() == 0 and validate_merge(lse=None) == 0
    assert validate_merge(D=8, out_dtype=fa.ATTN_F32) == 0 and validate_merge(D=4096) == 0
    assert validate_merge(o=None) == -1 and validate_merge(o_part=None) == -1
    assert validate_merge(lse_part=None) == -1
    assert validate_merge(nsplit=0) == -11 and validate_merge(nsplit=257) == -11
    assert validate_merge(rows=-1) == -2 and validate_merge(D=0) == -2
    # no rows: nothing to merge, the pointers may be NULL
    assert validate_merge(rows=0, o_part=None, lse_part=None, o=None, lse=None) == 0
    assert validate_merge(D=12) == -3 and validate_merge(D=4104) == -3
    assert validate_merge(out_dtype=3) == -5 and validate_merge(out_dtype=-1) == -5
    assert validate_merge(o=O + 8) == -7 and validate_merge(lse=L + 1) == -7
    assert validate_merge(o_part=P_O + 4) == -7
    assert validate_merge(o=P_O) == -9 and validate_merge(lse=P_L) == -9
    assert validate_merge(lse=O + 4) == -9


@pytest.mark.parametrize("Lk,nsplit", [(1, 1), (1, 5), (63, 2), (64, 2), (1000, 3),
                                       (16384, 8), (16384, 7), (100, 4), (4096, 256)])
def test_split_ranges_partition_the_keys(Lk, nsplit):
    ranges = [fa.attn_split_range(Lk, nsplit, s) for s in range(nsplit)]
    assert ranges[0][0] == 0 and ranges[-1][1] == Lk
    for (b0, e0), (b1, e1) in zip(ranges[:-1], ranges[1:]):
        assert e0 == b1 and b0 <= e0 <= b1 <= e1
    if nsplit > 1:
        # ranges of ceil(ceil(Lk / nsplit) / 64) * 64 keys from key 0, cut at Lk
        n = -(-(-(-Lk // nsplit)) // 64) * 64
        assert ranges == [(min(s * n, Lk), min(s * n + n, Lk)) for s in range(nsplit)]


def test_split_range_errors():
    for args, code in [((-1, 1, 0), -2), ((10, 0, 0), -11), ((10, 2, 2), -11), ((10, 2, -1), -11),
                       ((10, 257, 0), -11)]:
        with pytest.raises(fa.AttnError) as e:
            fa.attn_split_range(*args)
        assert e.value.code == code


def test_workspace_bytes():
    assert fa.attn_workspace_bytes(1, 32, 1024, 256, 1) == 0
    rows = 2 * 32 * 1000
    o_bytes = -(-(4 * rows * 128 * 4) // 256) * 256
    l_bytes = -(-(4 * rows * 4) // 256) * 256
    assert fa.attn_workspace_bytes(2, 32, 1000, 128, 4) == o_bytes + l_bytes
    assert fa.attn_workspace_bytes(1, 32, 1024, 256, 0) == -11
    assert fa.attn_workspace_bytes(-1, 32, 1024, 256, 2) == -2
    assert fa.attn_workspace_bytes(0, 32, 1024, 256, 2) == 0  # no rows, no partials


@pytest.mark.parametrize("shape,expect", [
    ((1, 32, 2, 16384, 16384, 256), (1, 1)),    # 2048 workgroups: no split
    ((4, 32, 2, 1024, 16384, 256), (1, 1)),     # 512 workgroups, two full rounds
    ((1, 32, 2, 1024, 16384, 256), (2, 2)),     # 128 workgroups: half the CUs idle unsplit
    # decode: 2 wide workgroups unsplit (16 heads x 16 rows each); split, the narrow shape
    # (two 128-row workgroups per group) needs half as many splits
    ((1, 32, 2, 16, 16384, 256), (16, 64)),
    ((1, 2, 1, 256, 256, 128), (1, 1)),         # too few keys to split
])
def test_plan_ex_split_choice(shape, expect):
    p = fa.attn_plan_ex(*shape, fa.ATTN_F16, 0)
    assert expect[0] <= p.nsplit <= expect[1], p.nsplit
    base = fa.attn_plan(*shape, fa.ATTN_F16)
    B, Hq, Hkv, Lq, Lk, D = shape
    # the grid counts the planner's own tiles (its rows per workgroup) and every split
    assert p.grid == math.ceil(Hq // Hkv * Lq / p.block_m) * Hkv * B * p.nsplit
    if Hq // Hkv * Lq > 128 and p.block_m == 128:
        assert p.nsplit > 1 and p.kernel.decode().endswith("_m128")
    assert p.workspace_bytes == fa.attn_workspace_bytes(B, Hq, Lq, D, p.nsplit)
    assert p.split_len == fa.attn_split_range(Lk, p.nsplit, 0)[1]
    assert base.nsplit == 1 and base.workspace_bytes == 0


def test_planner_weighs_the_narrow_shape_for_split_groups():
    # groups that need splits: narrow (with 64 batch entries the narrow shape fills the GPU
    # with no split at all, rather than the wide one with partials); the same groups with
    # enough work unsplit: wide; explicit plans (attn_plan) keep the default shape
    assert fa.attn_plan_ex(4, 32, 2, 16, 16384, 256, fa.ATTN_F16, 1).block_m == 128
    p = fa.attn_plan_ex(64, 32, 2, 16, 4096, 256, fa.ATTN_F16, 0)
    assert (p.block_m, p.nsplit) == (128, 1)
    assert fa.attn_plan_ex(256, 32, 2, 16, 4096, 256, fa.ATTN_F16, 0).block_m == 256
    assert fa.attn_plan(4, 32, 2, 16, 16384, 256, fa.ATTN_F16).block_m == 256
    # past 256 rows too: 272 rows (a ragged second wide tile) and 512 rows with few groups
    assert fa.attn_plan_ex(1, 32, 2, 17, 16384, 256, fa.ATTN_F16, 0).block_m == 128
    assert fa.attn_plan_ex(2, 16, 2, 64, 8192, 256, fa.ATTN_F16, 0).block_m == 128


# Planner picks on the shapes of a measured sweep (one MI355X; every split count of both tile
# shapes timed, attention and merge launches together): the plan the planner picks, and the
# fastest measured plans it has to be among (those within 1 % of the fastest, or a split count
# between two of them).  B, Hq, Hkv, Lq, Lk, D, dtype, causal -> (rows per workgroup,
# smallest and largest acceptable split count).
MEASURED_BEST = [
    ((4, 32, 2, 16, 16384, 256, fa.ATTN_F16, 1), (128, 16, 16)),    # 52.9 us at 16 splits
    ((1, 32, 8, 1, 65536, 128, fa.ATTN_BF16, 1), (128, 64, 64)),    # 46.7 us at 64
    ((1, 32, 2, 1024, 16384, 256, fa.ATTN_F16, 0), (256, 2, 2)),    # 473.6 us at 2
    ((1, 32, 8, 4, 32768, 128, fa.ATTN_F16, 1), (128, 64, 64)),     # 28.3 us at 64 (best 28.1)
    ((2, 16, 2, 64, 8192, 256, fa.ATTN_F16, 0), (128, 12, 16)),     # 36.5 / 36.8 us at 12 / 16
    ((8, 32, 8, 1, 8192, 128, fa.ATTN_BF16, 1), (128, 8, 8)),       # 46.0 us at 8
    ((1, 32, 4, 256, 32768, 128, fa.ATTN_F16, 0), (256, 8, 8)),     # 142.5 us at 8
    ((1, 64, 8, 128, 16384, 256, fa.ATTN_F16, 0), (256, 8, 8)),     # 139.6 us at 8
    ((16, 32, 8, 2, 4096, 128, fa.ATTN_F16, 1), (128, 4, 4)),       # 46.0 us at 4
    ((1, 8, 1, 2048, 65536, 128, fa.ATTN_F16, 0), (256, 4, 4)),     # 511.0 us at 4
]


@pytest.mark.parametrize("shape,expect", MEASURED_BEST)
def test_planner_matches_measured_best(shape, expect):
    B, Hq, Hkv, Lq, Lk, D, dt, causal = shape
    p = fa.attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, dt, fa.ATTN_CAUSAL if causal else 0)
    assert p.block_m == expect[0] and expect[1] <= p.nsplit <= expect[2], (p.block_m, p.nsplit)


def test_plan_ex_names_the_causal_kernel():
    p = fa.attn_plan_ex(1, 8, 2, 512, 512, 128, fa.ATTN_BF16, fa.ATTN_CAUSAL)
    assert p.kernel.decode() == "attn_fwd_d128_bf16_causal"
    with pytest.raises(fa.AttnError) as e:
        fa.attn_plan_ex(1, 8, 2, 512, 512, 128, fa.ATTN_BF16, 8)
    assert e.value.code == -10


def fwd_ex(nsplit, ws, ws_bytes, flags=0, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.attn_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Lq"], a["Lk"], a["D"], a["scale"], a["in_dtype"], flags, nsplit, ws,
                          ws_bytes, None)


WS = 15 * GB  # a fake, 256-byte aligned workspace address clear of the other arguments


def test_fwd_ex_rejects_bad_workspace_before_any_launch():
    need = fa.attn_workspace_bytes(GOOD["B"], GOOD["Hq"], GOOD["Lq"], GOOD["D"], 4)
    assert need > 0
    assert fwd_ex(4, None, 0) == -12                 # missing
    assert fwd_ex(4, WS, need - 1) == -12            # too small
    assert fwd_ex(4, WS + 16, need) == -12           # not 256-byte aligned
    assert fwd_ex(4, Q, need) == -12                 # overlaps q
    assert fwd_ex(4, O - need + 256, need) == -12    # overlaps o
    # argument errors come first, whatever the workspace
    assert fwd_ex(4, None, 0, flags=8) == -10
    assert fwd_ex(300, WS, need) == -11
    assert fwd_ex(4, WS, need, D=64) == -3


def test_merge_and_partial_reject_before_any_launch():
    assert fa.attn_merge(P_O, P_L, 0, 10, 128, O, L, fa.ATTN_F16, None) == -11
    assert fa.attn_merge(P_O, P_L, 2, 10, 100, O, L, fa.ATTN_F16, None) == -3
    assert fa.attn_merge(P_O, None, 2, 10, 128, O, L, fa.ATTN_F16, None) == -1
    assert fa.attn_merge(P_O, P_L, 2, 10, 128, P_O, L, fa.ATTN_F16, None) == -9
    a = GOOD
    assert fa.attn_fwd_partial(a["q"], a["k"], a["v"], P_O, None, a["B"], a["Hq"], a["Hkv"],
                               a["Lq"], a["Lk"], a["D"], a["scale"], a["in_dtype"], 0, 2,
                               None) == -1
    assert fa.attn_fwd_partial(a["q"], a["k"], a["v"], P_O, P_L, a["B"], a["Hq"], a["Hkv"],
                               a["Lq"], a["Lk"], a["D"], a["scale"], a["in_dtype"], 0, 0,
                               None) == -11
