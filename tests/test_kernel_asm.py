"""Static checks of the gfx950 code the kernels compile to (CPU only: hipcc cross-compiles).

The kernels rely on invariants the compiler cannot enforce by itself:
* the output accumulator lives in fixed AGPRs written only by inline asm, so no compiler-
  generated instruction may touch those AGPRs;
* M0 carries the LDS destination of the direct global->LDS copies, set inside the same
  inline asm statement, so the compiler must not use M0 for anything else;
* no register spills (scratch traffic would wreck the key loop);
* no packed fp32 VALU instructions;
* no scalar-memory writes (stores, atomics and write-backs go through the vector path).
"""
import os
import re
import subprocess

import pytest

from flash_attention_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flash_attention_amd", "csrc")
SOURCES = [os.path.join(CSRC, "attn_fwd.hip"), os.path.join(CSRC, "attn_merge.hip")]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    text = []
    for src in SOURCES:
        out = str(tmp_path_factory.mktemp("asm") / (os.path.basename(src) + ".s"))
        cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
               "-I" + os.path.join(ROOT, "include"), *lib_build.DEVICE_FLAGS,
               "--cuda-device-only", "-S", src, "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        text.append(open(out).read())
    return "\n".join(text)


def kernels(text, which="attn_(?:fwd|merge)_kernel"):
    """{kernel symbol: list of instruction lines with an in_asm flag}."""
    res = {}
    pat = r"^(_Z\w*%s\w*):[^\n]*\n(.*?)^\.Lfunc_end" % which
    for m in re.finditer(pat, text, re.M | re.S):
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
    ks = kernels(asm, "attn_fwd_kernel")
    assert len(ks) == 16, sorted(ks)  # D in {128,256} x tile shape x {f16,bf16} x scale sign
    assert len(kernels(asm, "attn_merge_kernel")) == 15  # output fp16, bf16, fp32 x part groups 1-16


# AGPRs 0 .. PINNED-1 hold the output accumulator, written only by inline asm: 16 x 32-row
# query blocks per wave x 32-dim blocks (HD=256: 2 x 8 blocks, every AGPR; HD=128: 1 x 4
# blocks, with Q's fragments in compiler-allocated AGPRs above them).
PINNED = {"128": 64, "256": 256}


def agprs_in(ln):
    regs = set()
    for m in re.finditer(r"\ba\[(\d+):(\d+)\]", ln):
        regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\ba(\d+)\b", ln):
        regs.add(int(m.group(1)))
    return regs


def test_pinned_agprs_only_in_inline_asm(asm):
    for name, lines in kernels(asm, "attn_fwd_kernel").items():
        pinned = PINNED[re.search(r"ILi(\d+)E", name).group(1)]
        bad = [ln for ln, inside in lines
               if not inside and any(a < pinned for a in agprs_in(ln))]
        assert not bad, (name, bad[:5])
    for name, lines in kernels(asm, "attn_merge_kernel").items():
        assert not [ln for ln, _ in lines if agprs_in(ln)], name


def test_m0_only_in_inline_asm(asm):
    for name, lines in kernels(asm).items():
        bad = [ln for ln, inside in lines if not inside and re.search(r"\bm0\b", ln)]
        assert not bad, (name, bad[:5])


def test_no_scratch(asm):
    for name, lines in kernels(asm).items():
        assert not [ln for ln, _ in lines if ln.startswith("scratch_")], name
    for m in re.finditer(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", asm):
        assert int(m.group(1)) == 0


def test_no_scalar_memory_writes(asm):
    """Stores go through the vector memory path only: no scalar-cache stores, atomics or
    write-backs (the split-merge counters use global_atomic_* instructions)."""
    pat = re.compile(r"s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb)")
    for name, lines in kernels(asm).items():
        assert not [ln for ln, _ in lines if pat.match(ln)], name
    assert not pat.search("\n".join(ln for ls in kernels(asm).values() for ln, _ in ls))


def test_no_packed_fp32(asm):
    for name, lines in kernels(asm).items():
        assert not [ln for ln, _ in lines if re.match(r"v_pk_(fma|mul|add)_f32", ln)], name


# ---- MFMA hazard check ------------------------------------------------------------------
# The MFMAs are inline asm, so the compiler inserts no wait states around them.  The ISA
# requires (gfx940 family): 2 wait states between a VALU write of a VGPR and an MFMA reading
# it, and between an MFMA writing a register and a VALU access to it the 12 wait states that
# the compiler's own hazard recognizer inserts after the 8-pass 32x32x16 ops on gfx950
# (s_nop 11).  MFMA -> MFMA accumulation into the same registers is interlocked by the
# hardware.  These checks walk the emitted code.
RESULT_WAIT_STATES = 12
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def regs_of(text):
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def split_ops(ln):
    parts = ln.split(None, 1)
    op = parts[0]
    args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
    return op, args


def wait_states(ln):
    op, args = split_ops(ln)
    if op == "s_nop":
        return int(args[0], 0) + 1
    return 1


def is_valu(op):
    return op.startswith("v_") and not op.startswith("v_mfma") and op not in (
        "v_readfirstlane_b32", "v_readlane_b32")


def valu_defs(ln):
    op, args = split_ops(ln)
    if not args:
        return set()
    d = regs_of(args[0])
    if op in ("v_permlane32_swap_b32", "v_permlane16_swap_b32", "v_swap_b32") and len(args) > 1:
        d |= regs_of(args[1])
    return d


def instruction_stream(text):
    """Per kernel: list of (line, in_asm, is_label)."""
    res = {}
    for m in re.finditer(r"^(_Z\w*attn_fwd_kernel\w*):[^\n]*\n(.*?)^\s*s_endpgm", text,
                         re.M | re.S):
        seq, inside = [], False
        for ln in m.group(2).splitlines():
            s = ln.strip()
            if s.startswith(";;#ASMSTART"):
                inside = True
            elif s.startswith(";;#ASMEND"):
                inside = False
            elif re.match(r"^\.?[A-Za-z_][\w.]*:", s):
                seq.append((s, inside, True))
            elif s and not s.startswith(";") and not s.startswith("."):
                seq.append((s.split(";")[0].strip(), inside, False))
        res[m.group(1)] = seq
    return res


def _branch_sources(seq):
    """label -> indices of the branch instructions that jump to it."""
    src = {}
    for i, (ln, _, lab) in enumerate(seq):
        if not lab and (ln.startswith("s_cbranch") or ln.startswith("s_branch")):
            src.setdefault(ln.split()[-1], []).append(i)
    return src


def _preceding_writes(seq, branches, j, budget, srcs, seen):
    """Walk back from instruction j over every control-flow predecessor until `budget` wait
    states are covered; return the VALU lines that write one of `srcs` on the way."""
    hits = []
    while j >= 0 and budget > 0:
        if (j, budget) in seen:
            return hits
        seen.add((j, budget))
        ln, _, lab = seq[j]
        if lab:
            for b in branches.get(ln.rstrip(":").split()[0].rstrip(":"), []):
                hits += _preceding_writes(seq, branches, b - 1, budget, srcs, seen)
            prev = seq[j - 1][0] if j > 0 else ""
            if prev.startswith("s_branch"):
                return hits  # no fall-through into this label
            j -= 1
            continue
        op, _ = split_ops(ln)
        if is_valu(op) and valu_defs(ln) & srcs:
            hits.append(ln)
            return hits
        if not op.startswith("s_cbranch") and not op.startswith("s_branch"):
            budget -= wait_states(ln)
        j -= 1
    return hits


def test_mfma_source_hazards(asm):
    """No VALU instruction writes an MFMA source register less than 2 wait states before, on
    any control-flow path into the MFMA."""
    problems = []
    for name, seq in instruction_stream(asm).items():
        branches = _branch_sources(seq)
        for i, (ln, _, lab) in enumerate(seq):
            if lab or not ln.startswith("v_mfma"):
                continue
            op, args = split_ops(ln)
            srcs = set()
            for a in args[1:]:
                srcs |= regs_of(a)
            hits = _preceding_writes(seq, branches, i - 1, 2, srcs, set())
            if hits:
                problems.append((name, hits[0], ln))
    assert not problems, problems[:6]


def test_mfma_result_hazards(asm):
    """No VALU instruction touches an MFMA destination less than RESULT_WAIT_STATES wait
    states after it."""
    problems = []
    for name, seq in instruction_stream(asm).items():
        for i, (ln, _, lab) in enumerate(seq):
            if lab or not ln.startswith("v_mfma"):
                continue
            op, args = split_ops(ln)
            dst = regs_of(args[0])
            ws, j = 0, i + 1
            while j < len(seq) and ws < RESULT_WAIT_STATES:
                nln, _, nlab = seq[j]
                if nlab or nln.startswith("s_cbranch") or nln.startswith("s_branch"):
                    break
                nop, nargs = split_ops(nln)
                if is_valu(nop):
                    touched = set()
                    for a in nargs:
                        touched |= regs_of(a)
                    if touched & dst:
                        problems.append((name, ln, nln, ws))
                        break
                ws += wait_states(nln)
                j += 1
    assert not problems, problems[:6]


def test_hazard_checker_catches_planted_hazards():
    """The two checkers flag a VALU write right before an MFMA source and a VALU read right
    after an MFMA result (planted in a synthetic stream, not in the kernels)."""
    good = ("_Zattn_fwd_kernel_t:\n\tds_read_b128 v[4:7], v1\n\ts_waitcnt lgkmcnt(0)\n"
            "\ts_nop 1\n\tv_mfma_f32_32x32x16_f16 a[0:15], v[4:7], v[8:11], a[0:15]\n"
            "\ts_nop 11\n\tv_accvgpr_read_b32 v2, a3\n\ts_endpgm\n")
    bad_src = good.replace("\ts_nop 1\n", "\tv_mov_b32_e32 v9, 0\n")
    bad_dst = good.replace("\ts_nop 11\n", "\ts_nop 10\n")
    test_mfma_source_hazards(good)
    test_mfma_result_hazards(good)
    with pytest.raises(AssertionError):
        test_mfma_source_hazards(bad_src)
    with pytest.raises(AssertionError):
        test_mfma_result_hazards(bad_dst)
