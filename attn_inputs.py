"""Seeded synthetic inputs for the attention forward pass.

This module holds the workload shapes and the random-number recipe only; it
does none of the attention arithmetic, so both the oracle and the HIP path
may draw their inputs from it.

Recipe: each tensor is drawn on the CPU with its own ``torch.Generator``
seed as float32 ``randn`` (or ``rand`` - 0.5 for the uniform mix), scaled if
the workload says so, then rounded once to fp16/bf16.  Both sides then read
the same 16-bit values (the CPU reference consumes type-quantised inputs, as
"Xe2 Sdp Bf16", section "Correctness Testing", prescribes).
"""
import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    dtype: str  # "f16" | "bf16"
    k_mult: float = 1.0
    seed_base: int = 0
    causal: bool = False  # row i sees key j only if j <= i + Lk - Lq
    nsplit: int = 1       # key splits of the launch (0: the planner's choice)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self):
        """4*B*Hq*Lq*Lk*D: the two matrix products over every (row, key) pair.  Under the
        causal mask only the visible pairs count; bench.py computes that figure."""
        return 4 * self.B * self.Hq * self.Lq * self.Lk * self.D

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    def describe(self):
        return ("B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d %s%s%s%s" %
                (self.B, self.Hq, self.Hkv, self.Lq, self.Lk, self.D, self.dtype,
                 " K*%g" % self.k_mult if self.k_mult != 1.0 else "",
                 " causal" if self.causal else "",
                 " nsplit=%d" % self.nsplit if self.nsplit != 1 else ""))


# The five workloads of the benchmark plan: the tiny case, the 4K and 8K
# squares, the rectangular short-query/long-key case with sharpened softmax,
# and the 16K x 16K, 32 Q / 2 KV head, HD=256 case (the shape of the
# "Xe2 ... Flash Attention -- HD=256" page's headline figure).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1, 256, 256, 128, "f16", seed_base=1000),
    "gqa4k_d256": Workload("gqa4k_d256", 1, 32, 2, 4096, 4096, 256, "f16", seed_base=2000),
    "gqa8k_d128_bf16": Workload("gqa8k_d128_bf16", 1, 32, 8, 8192, 8192, 128, "bf16",
                                seed_base=3000),
    "rect1kx16k_d256": Workload("rect1kx16k_d256", 4, 32, 2, 1024, 16384, 256, "f16",
                                k_mult=2.0, seed_base=4000),
    "gqa16k_d256": Workload("gqa16k_d256", 1, 32, 2, 16384, 16384, 256, "f16",
                            seed_base=5000),
    # Next to the plan: the headline shape under the causal mask, and a single sequence of
    # 1K queries against 16K keys, which leaves half the compute units idle unless the keys
    # are split (the planner's choice).
    "gqa16k_d256_causal": Workload("gqa16k_d256_causal", 1, 32, 2, 16384, 16384, 256, "f16",
                                   seed_base=6000, causal=True),
    "q1kx16k_d256_split": Workload("q1kx16k_d256_split", 1, 32, 2, 1024, 16384, 256, "f16",
                                   seed_base=7000, nsplit=0),
    # decode-like: 16 new queries per sequence (the last 16 positions, causal) against 16K
    # keys, 4 sequences: the 16 query heads of a key/value head share its workgroups' rows
    # and the planner splits the keys
    "decode16x16k_d256": Workload("decode16x16k_d256", 4, 32, 2, 16, 16384, 256, "f16",
                                  seed_base=8000, causal=True, nsplit=0),
    "decode1x64k_d128_bf16": Workload("decode1x64k_d128_bf16", 1, 32, 8, 1, 65536, 128,
                                      "bf16", seed_base=9000, causal=True, nsplit=0),
    # The headline shape over sharper score ranges ("multiple data ranges" of the HD=256
    # page's section "Performance Testing"): K scaled by 4 and by 8 before the rounding to
    # fp16, so that later key tiles outgrow a row's first-tile maximum and the kernel's lazy
    # rescale runs (scores ~ N(0, 16) and N(0, 64) in natural-log units).
    "gqa16k_d256_k4": Workload("gqa16k_d256_k4", 1, 32, 2, 16384, 16384, 256, "f16",
                               k_mult=4.0, seed_base=10000),
    "gqa16k_d256_k8": Workload("gqa16k_d256_k8", 1, 32, 2, 16384, 16384, 256, "f16",
                               k_mult=8.0, seed_base=11000),
    # Each head dimension's square case with the other 16-bit input type, so that all four
    # kernels (HD 128/256 x fp16/bf16) have a timed workload.
    "gqa16k_d256_bf16": Workload("gqa16k_d256_bf16", 1, 32, 2, 16384, 16384, 256, "bf16",
                                 seed_base=12000),
    "gqa8k_d128_f16": Workload("gqa8k_d128_f16", 1, 32, 8, 8192, 8192, 128, "f16",
                               seed_base=13000),
}
HEADLINE = "gqa16k_d256"


def _draw(shape, seed, dist):
    g = torch.Generator().manual_seed(int(seed))
    if dist == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32)
    if dist == "uniform":
        return torch.rand(shape, generator=g, dtype=torch.float32) - 0.5
    raise ValueError("unknown distribution %r" % dist)


def make_qkv(B, Hq, Hkv, Lq, Lk, D, dtype="f16", seed=0, dist="normal", k_mult=1.0,
             q_mult=1.0, v_mult=1.0):
    """Q [B,Hq,Lq,D], K/V [B,Hkv,Lk,D] as CPU fp16/bf16 tensors.

    Seeds: Q seed+1, K seed+2, V seed+3.
    """
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    q = _draw((B, Hq, Lq, D), seed + 1, dist)
    k = _draw((B, Hkv, Lk, D), seed + 2, dist)
    v = _draw((B, Hkv, Lk, D), seed + 3, dist)
    if q_mult != 1.0:
        q = q * q_mult
    if k_mult != 1.0:
        k = k * k_mult
    if v_mult != 1.0:
        v = v * v_mult
    return q.to(tdt), k.to(tdt), v.to(tdt)


def make_qkv_on(device, B, Hq, Hkv, Lq, Lk, D, dtype="f16", seed=0):
    """make_qkv's recipe (N(0,1) per element, seeds seed+1..seed+3, one rounding to 16 bits)
    drawn by torch's generator of ``device`` (counter-based Philox on a GPU), so that inputs
    of several GiB take seconds instead of minutes.  The values differ from make_qkv's for
    the same seed; both are fixed by the seed.  The tensors stay on ``device``."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    out = []
    for i, shape in enumerate(((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D))):
        g = torch.Generator(device=device).manual_seed(int(seed) + 1 + i)
        t = torch.empty(shape, dtype=tdt, device=device)
        flat = t.view(-1)
        step = 1 << 28  # fp32 draws in slices of 1 GiB
        for s in range(0, flat.numel(), step):
            n = min(step, flat.numel() - s)
            flat[s:s + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        out.append(t)
    return tuple(out)


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, w.dtype, seed=w.seed_base,
                    k_mult=w.k_mult)


def sample_rows(w: Workload, n_random=1024, tile=128):
    """Seeded subset of flat query rows (b*Hq + h)*Lq + i for large workloads.

    n_random rows drawn without replacement (seed seed_base+4), plus every row
    of the first and last ``tile``-row query tile of the first and last head,
    plus rows 0 and Lq-1 of every head.  Sorted, unique.
    """
    total = w.B * w.Hq * w.Lq
    rng = np.random.default_rng(w.seed_base + 4)
    pick = [rng.choice(total, size=min(n_random, total), replace=False)]
    first, last = 0, (w.B * w.Hq - 1) * w.Lq
    t = min(tile, w.Lq)
    pick.append(first + np.arange(t))
    pick.append(first + w.Lq - t + np.arange(t))
    pick.append(last + np.arange(t))
    pick.append(last + w.Lq - t + np.arange(t))
    heads = np.arange(w.B * w.Hq) * w.Lq
    pick.append(heads)
    pick.append(heads + w.Lq - 1)
    return np.unique(np.concatenate(pick).astype(np.int64))
