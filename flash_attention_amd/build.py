"""Build flash_attention_amd/libattn.so (gfx950 code objects + host C ABI) with hipcc.

Run ``python -m flash_attention_amd.build`` (or ``__graft_entry__.build()``) after any
change to csrc/ or include/.  Cross-compiles on a machine without a GPU.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "attn_fwd.hip"), os.path.join(CSRC, "attn_merge.hip"),
           os.path.join(CSRC, "attn_device.hip"), os.path.join(CSRC, "attn_host.cpp")]

# Packed fp32 VALU instructions are kept out of the device code: the compiler would
# otherwise form them from ordinary float code.  The key loop's `#pragma unroll` loops must
# unroll completely (their arrays are indexed by the loop counters, and a loop left rolled
# would move those arrays to scratch memory); the default size limit for forced unrolling is
# below the attention kernel's loop bodies, so it is raised.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-pragma-unroll-threshold=1000000"]


def build(out=LIB, extra=(), quiet=False, save_temps_dir=None):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I" + os.path.join(ROOT, "include"), *DEVICE_FLAGS, *extra]
    if save_temps_dir:
        os.makedirs(save_temps_dir, exist_ok=True)
        cmd += ["-save-temps=obj", "-o", os.path.join(save_temps_dir, "libattn.so")]
    else:
        cmd += ["-o", tmp]
    cmd += SOURCES
    if not quiet:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, err))
    if err.strip() and not quiet:
        print(err, file=sys.stderr)
    if not save_temps_dir:
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
