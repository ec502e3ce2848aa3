"""A second, independent fp64 evaluation of attention with NumPy -- TEST
INFRASTRUCTURE ONLY, used on tiny shapes to cross-check attn_oracle.c.

Same definition as the C oracle, written with whole-array operations instead
of loops: scores = scale * Q K^T per head, row softmax, weights times V, and
LSE = log of the sum of exp(scores).  Grouped-query attention is realised
literally as the repetition of each key/value head for Hq/Hkv consecutive
query heads (SyclKittens summary, section E.1: the GQA baseline repeats KV
heads).
"""
import numpy as np


def attention(q, k, v, scale, causal=False):
    """q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] float64 arrays -> (O [B,Hq,Lq,D], LSE [B,Hq,Lq]).

    causal: query i keeps key j only where j - i <= Lk - Lq (a triangular mask
    aligned to the bottom-right corner of the Lq x Lk score matrix); a row with
    nothing kept gets O = 0 and LSE = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    group = q.shape[1] // k.shape[1]
    k_rep = np.repeat(k, group, axis=1)
    v_rep = np.repeat(v, group, axis=1)
    scores = scale * np.matmul(q, np.swapaxes(k_rep, -1, -2))  # [B,Hq,Lq,Lk]
    Lq, Lk = scores.shape[-2:]
    keep = np.ones((Lq, Lk), dtype=bool)
    if causal:
        keep = np.tril(keep, k=Lk - Lq)
    scores = np.where(keep, scores, -np.inf)
    has = keep.any(axis=-1)[:, None]  # [Lq, 1]
    top = np.where(has, scores.max(axis=-1, keepdims=True), 0.0)
    w = np.exp(scores - top)
    total = w.sum(axis=-1, keepdims=True)
    out = np.matmul(w / np.where(has, total, 1.0), v_rep)
    with np.errstate(divide="ignore"):
        lse = (top + np.log(total))[..., 0]
    return out, lse
