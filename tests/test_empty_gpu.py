"""Empty sizes on the GPU, through the C ABI.

No keys (Lk = 0): every row's softmax is over an empty set, so O = 0 and LSE = -inf
exactly, as the oracle gives (the same values as a causal row that sees no key); checked
for both head dims and dtypes, with and without the mask, in one pass, with key splits and
for the partial results.  No query rows (B, Hq or Lq = 0): a valid call that launches and
writes nothing.
"""
import pytest
import torch

import attn_inputs
import flash_attention_amd as fa
from parity_util import parity, scale_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,dt", [(128, "f16"), (256, "bf16"), (256, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal,nsplit", [(False, 1), (True, 1), (False, 3), (True, 0)])
def test_no_keys(D, dt, causal, nsplit):
    B, Hq, Hkv, Lq = 2, 8, 2, 77
    seed = 9700 + D
    print("\n[case] no keys B=%d Hq=%d Hkv=%d Lq=%d Lk=0 D=%d %s causal=%d nsplit=%d seed=%d"
          % (B, Hq, Hkv, Lq, D, dt, causal, nsplit, seed), flush=True)
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, 1, D, dt, seed=seed)
    k, v = k[:, :, :0].contiguous(), v[:, :, :0].contiguous()
    o, lse, m = parity(q, k, v, scale_of(D), dt, causal=causal, nsplit=nsplit,
                       what="no keys D=%d %s causal=%d nsplit=%d" % (D, dt, causal, nsplit))
    assert m["empty_rows"] == B * Hq * Lq
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("D", [128, 256])
def test_no_keys_partials(D):
    B, Hq, Hkv, Lq, ns = 1, 4, 1, 40, 3
    print("\n[case] no keys, partials B=%d Hq=%d Lq=%d D=%d nsplit=%d" % (B, Hq, Lq, D, ns),
          flush=True)
    dev = torch.device("cuda:0")
    q, _, _ = attn_inputs.make_qkv(B, Hq, Hkv, Lq, 1, D, "f16", seed=9800 + D)
    q = q.to(dev)
    k = torch.empty((B, Hkv, 0, D), dtype=q.dtype, device=dev)
    o_part, lse_part = fa.fwd_partial(q, k, k, ns, causal=True)
    torch.cuda.synchronize()
    assert bool((o_part == 0).all()) and bool(torch.isneginf(lse_part).all())
    o, lse = fa.merge(o_part, lse_part, out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("shape", [(0, 8, 2, 16, 64), (2, 0, 2, 16, 64), (2, 8, 2, 0, 64),
                                   (2, 8, 2, 0, 0)])
def test_no_query_rows(shape):
    B, Hq, Hkv, Lq, Lk = shape
    D = 256
    print("\n[case] no query rows B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d" % (*shape, D),
          flush=True)
    dev = torch.device("cuda:0")
    q = torch.empty((B, Hq, Lq, D), dtype=torch.float16, device=dev)
    k = torch.randn((B, Hkv, Lk, D), device=dev).to(torch.float16)
    v = torch.randn((B, Hkv, Lk, D), device=dev).to(torch.float16)
    for causal, nsplit in ((False, 1), (True, 1), (False, 4), (True, 0)):
        o, lse = fa.fwd(q, k, v, causal=causal, nsplit=nsplit)
        assert tuple(o.shape) == (B, Hq, Lq, D) and tuple(lse.shape) == (B, Hq, Lq)
    o_part, lse_part = fa.fwd_partial(q, k, v, 3)
    o, lse = fa.merge(o_part, lse_part, out_dtype=torch.bfloat16)
    assert o.numel() == 0 and lse.numel() == 0
    torch.cuda.synchronize()  # nothing was launched, nothing can have failed
