"""Static checks of the gfx950 code the kernels compile to (CPU only: hipcc cross-compiles).

The kernels rely on invariants the compiler cannot enforce by itself:
* the output accumulator lives in fixed AGPRs written only by inline asm, so no compiler-
  generated instruction may touch an AGPR;
* M0 carries the LDS destination of the direct global->LDS copies, set inside the same
  inline asm statement, so the compiler must not use M0 for anything else;
* no register spills (scratch traffic would wreck the key loop);
* no packed fp32 VALU instructions.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "flash_attention_amd", "csrc", "attn_fwd.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "attn_fwd.s")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-I" + os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", SRC, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def kernels(text):
    """{kernel symbol: list of instruction lines with an in_asm flag}."""
    res = {}
    for m in re.finditer(r"^(_Z\w*attn_fwd_kernel\w*):[^\n]*\n(.*?)^\s*s_endpgm", text, re.M | re.S):
        lines, inside = [], False
        for ln in m.group(2).splitlines():
            s = ln.strip()
            if s.startswith(";;#ASMSTART"):
                inside = True
            elif s.startswith(";;#ASMEND"):
                inside = False
            elif s and not s.startswith(";") and not s.startswith("."):
                lines.append((s.split(";")[0].strip(), inside))
        res[m.group(1)] = lines
    return res


def test_all_kernels_present(asm):
    ks = kernels(asm)
    assert len(ks) == 8, sorted(ks)  # D in {128,256} x {f16,bf16} x scale sign


def test_no_agpr_outside_inline_asm(asm):
    agpr = re.compile(r"\ba\[\d+(:\d+)?\]|\ba\d+\b")
    for name, lines in kernels(asm).items():
        bad = [ln for ln, inside in lines if not inside and agpr.search(ln)]
        assert not bad, (name, bad[:5])


def test_m0_only_in_inline_asm(asm):
    for name, lines in kernels(asm).items():
        bad = [ln for ln, inside in lines if not inside and re.search(r"\bm0\b", ln)]
        assert not bad, (name, bad[:5])


def test_no_scratch(asm):
    for name, lines in kernels(asm).items():
        assert not [ln for ln, _ in lines if ln.startswith("scratch_")], name
    for m in re.finditer(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", asm):
        assert int(m.group(1)) == 0


def test_no_packed_fp32(asm):
    for name, lines in kernels(asm).items():
        assert not [ln for ln, _ in lines if re.match(r"v_pk_(fma|mul|add)_f32", ln)], name
