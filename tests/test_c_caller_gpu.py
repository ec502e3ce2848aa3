"""A plain C caller on the GPU: tests/c/fwd_from_c.c, built by gcc against include/attn.h
and libattn.so with device memory from the HIP runtime's C API, runs attn_fwd (null
stream) and attn_fwd_ex (causal, the planner's key splits, a hipMalloc'ed workspace); its
outputs are compared here with the fp64 oracle on the same 16-bit inputs.  No torch tensor
and no Python binding sits between that program and the kernels."""
import os
import subprocess

import numpy as np
import pytest
import torch

import attn_inputs
import flash_attention_amd as fa
import oracle
from parity_util import check, metrics

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "fwd_from_c.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("cprog") / "fwd_from_c")
    libdir = os.path.dirname(fa.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
                    SRC, "-o", out, "-L" + libdir, "-lattn", "-L" + os.path.join(ROCM, "lib"),
                    "-lamdhip64", "-Wl,-rpath," + libdir,
                    "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
    return out


CASES = [  # B, Hq, Hkv, Lq, Lk, D, dtype, seed
    (1, 2, 1, 256, 256, 128, "f16", 1000),     # the tiny workload's shape and seeds
    (1, 4, 2, 300, 333, 256, "bf16", 31000),   # ragged tiles, wide HD=256 kernel
    (2, 8, 2, 5, 2000, 256, "f16", 32000),     # decode-sized: narrow shape, key splits
]


@pytest.mark.parametrize("case", CASES, ids=["B%d_H%d_%d_L%dx%d_D%d_%s_s%d" % c for c in CASES])
def test_c_program_runs_attention(exe, tmp_path, case):
    B, Hq, Hkv, Lq, Lk, D, dt, seed = case
    print("\n[case] C caller %s" % (case,), flush=True)
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(fin, "wb") as f:
        for t in (q, k, v):
            f.write(t.contiguous().view(-1).view(torch.int16).numpy().tobytes())
    code = fa.ATTN_F16 if dt == "f16" else fa.ATTN_BF16
    r = subprocess.run([exe, fin, fout, str(B), str(Hq), str(Hkv), str(Lq), str(Lk), str(D),
                        str(code), repr(scale)], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0 and "fwd_from_c: ok" in r.stdout
    raw = open(fout, "rb").read()
    rows = B * Hq * Lq
    n16, n32 = rows * D * 2, rows * 4
    assert len(raw) == 2 * (n16 + n32)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    for i, causal in enumerate((False, True)):
        base = i * (n16 + n32)
        o = torch.frombuffer(bytearray(raw[base:base + n16]), dtype=torch.int16).view(tdt)
        lse = torch.frombuffer(bytearray(raw[base + n16:base + n16 + n32]), dtype=torch.float32)
        o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
        m = metrics(o.reshape(rows, D), lse, o_ref, lse_ref)
        print("[parity] C caller causal=%s %s" % (causal, m), flush=True)
        check(m, dt, "C caller causal=%s" % causal)
