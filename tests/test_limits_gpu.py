"""GPU parity at the largest shapes the library accepts.

Offsets inside one head are 32-bit: a head's keys (Lk * D elements) and the query rows of
one key/value group (Hq/Hkv * Lq * D elements) must each stay below 2^31, and the
validation refuses anything larger.  These cases sit right at those limits, with ragged
lengths, so that every byte offset up to ~2^32 is taken by the copies, the fragment reads
and the stores; sampled rows (the first and last of every head among them) are compared
with the fp64 oracle, and every row is checked to be written.  Inputs are drawn on the GPU
(attn_inputs.make_qkv_on) and copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

import attn_inputs
import flash_attention_amd as fa
from parity_util import parity, scale_of

pytestmark = pytest.mark.gpu

LIM = (1 << 31) - 1


def _host(*ts):
    return tuple(t.cpu() for t in ts)


@pytest.mark.parametrize("D,dt", [(256, "f16"), (128, "bf16")])
def test_longest_key_sequence(D, dt):
    B, Hq, Hkv, Lq = 1, 2, 1, 40
    Lk = LIM // D  # the largest accepted: 8388607 keys at D=256, a ragged last tile
    assert Lk % 32 == 31
    assert fa.attn_validate(1 << 40, 1 << 41, 3 << 40, 1 << 42, None, B, Hq, Hkv, Lq, Lk, D,
                            0.1, fa.ATTN_F16) == fa.ATTN_OK
    seed = 9500 + D
    print("\n[case] longest keys B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d %s seed=%d"
          % (B, Hq, Hkv, Lq, Lk, D, dt, seed), flush=True)
    q, k, v = _host(*attn_inputs.make_qkv_on("cuda", B, Hq, Hkv, Lq, Lk, D, dt, seed=seed))
    torch.cuda.empty_cache()
    rows = [0, Lq - 1, Lq, 2 * Lq - 1]
    for causal, nsplit in ((False, 1), (True, 0)):
        parity(q, k, v, scale_of(D), dt, rows=rows, causal=causal, nsplit=nsplit,
               what="longest keys D=%d causal=%d nsplit=%d" % (D, causal, nsplit))


@pytest.mark.parametrize("D,dt", [(256, "f16"), (128, "bf16")])
def test_largest_query_block(D, dt):
    G, Lk = 16, 33
    B, Hq, Hkv = 1, G, 1
    Lq = LIM // (G * D)  # 524287 rows per head at D=256: G * Lq * D just below 2^31
    assert G * Lq * D <= LIM < G * (Lq + 1) * D
    seed = 9600 + D
    print("\n[case] largest query block B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d %s seed=%d"
          % (B, Hq, Hkv, Lq, Lk, D, dt, seed), flush=True)
    q, k, v = _host(*attn_inputs.make_qkv_on("cuda", B, Hq, Hkv, Lq, Lk, D, dt, seed=seed))
    torch.cuda.empty_cache()
    rng = np.random.default_rng(seed)
    rows = [rng.choice(B * Hq * Lq, size=64, replace=False)]
    for h in (0, 1, Hq - 1):  # head ends, the causal boundary, the last query tile
        base = h * Lq
        rows.append(base + np.array([0, Lq - Lk - 1, Lq - Lk, Lq - 1]))
        rows.append(base + Lq - 300 + np.arange(0, 300, 7))
    rows = np.unique(np.concatenate(rows)).astype(np.int64)
    for causal in (False, True):
        o, lse, _ = parity(q, k, v, scale_of(D), dt, rows=rows, causal=causal,
                           what="largest query block D=%d causal=%d" % (D, causal))
        if causal:
            # rows before Lq - Lk see no key: exactly O = 0 and LSE = -inf, all of them
            assert bool((o[:, :, :Lq - Lk] == 0).all())
            assert bool(torch.isneginf(lse[:, :, :Lq - Lk]).all())
            assert bool(torch.isfinite(lse[:, :, Lq - Lk:]).all())
        else:
            assert bool(torch.isfinite(lse).all())
