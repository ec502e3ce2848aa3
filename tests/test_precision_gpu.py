"""Mixed P.V precision, measured on the GPU: bf16 inputs computed with fp16 weights.

bf16 values with magnitudes inside fp16's normal range are exactly representable in fp16
(8 significant bits into 11), so running the fp16 kernel on bf16 data converted to fp16 is
exactly the mixed path: the same scores, weights rounded to fp16 instead of bf16 before the
P.V product.  Both results are compared with the oracle on the bf16 inputs, the fp16 one
also after rounding its output to bf16 (the type a bf16 caller gets back).  The
"Xe2 Sdp Bf16" page's bf16io kernel keeps bf16 in memory and its own precision inside
(section "Kernel Architecture: bf16io"); on gfx950 the fp16 and bf16 matrix rates are
equal, so the only question is accuracy, which this test records.
"""
import numpy as np
import pytest
import torch

import attn_inputs
import oracle
from parity_util import gpu_fwd, scale_of

pytestmark = pytest.mark.gpu


def _rel_rms(o, ref):
    err = o.double().reshape(ref.shape).numpy() - ref
    return float(np.sqrt((err ** 2).sum() / (ref ** 2).sum()))


@pytest.mark.parametrize("D,km", [(128, 1.0), (128, 2.0), (256, 1.0)])
def test_fp16_weights_for_bf16_inputs(D, km):
    print("\n[case] mixed precision D=%d k*%g" % (D, km), flush=True)
    q, k, v = attn_inputs.make_qkv(1, 4, 2, 512, 2048, D, "bf16", seed=41, k_mult=km)
    # values below fp16's normal range (2^-14) set to 0, so that every value converts exactly
    q, k, v = (torch.where(t.abs() < 2.0 ** -14, torch.zeros_like(t), t) for t in (q, k, v))
    for t in (q, k, v):
        assert torch.equal(t.to(torch.float16).to(torch.bfloat16), t)
    scale = float(np.float32(scale_of(D)))
    ref, _ = oracle.attention(q, k, v, scale)
    o_bf, _ = gpu_fwd(q, k, v, scale)
    o_h, _ = gpu_fwd(q.to(torch.float16), k.to(torch.float16), v.to(torch.float16), scale)
    r_bf = _rel_rms(o_bf, ref)
    r_h = _rel_rms(o_h, ref)
    r_h_bf = _rel_rms(o_h.to(torch.bfloat16), ref)
    print("[precision] D=%d k*%g  bf16 weights: %.3e   fp16 weights, fp16 out: %.3e   "
          "fp16 weights, bf16 out: %.3e" % (D, km, r_bf, r_h, r_h_bf), flush=True)
    # fp16 weights are more accurate; rounded back to bf16 the output rounding dominates
    assert r_h < r_bf and r_h_bf < r_bf
    assert r_h < 0.5 * r_bf
