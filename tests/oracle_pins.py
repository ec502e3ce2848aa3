"""Pins of the fp64 oracle to facts fixed by the mathematics of attention.

Each pin takes an ``oracle.Oracle`` and raises AssertionError if the oracle
disagrees with a closed form, an invariant, a library routine or a value
derived by hand.  The same list is run against the real oracle
(test_oracle_pins.py) and against deliberately broken copies of it
(test_oracle_mutants.py), so that every plausible slip in the oracle -- a
dropped scale, a wrong head map, a transposed operand, a missing max
subtraction, the wrong log base, a bad fp16/bf16 decode, an off-by-one --
is shown to fail at least one pin.
"""
import json
import math
import os

import numpy as np
import scipy.special
import torch

import oracle as oracle_pkg
from oracle import numpy_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _f64(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _run(orc, q, k, v, scale, rows=None, **kw):
    o, lse = orc.attention(q, k, v, scale, rows=rows, **kw)
    B, Hq, Lq, D = np.asarray(q).shape if not isinstance(q, torch.Tensor) else q.shape
    if rows is None:
        return o.reshape(B, Hq, Lq, D), lse.reshape(B, Hq, Lq)
    return o, lse


def pin_worked_example(orc):
    """Hand-derived two-key case: O = -tanh(1/2), LSE = ln(1+e) (tests/golden)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    assert abs(g["expected_o"] - (-math.tanh(0.5))) < 1e-16
    assert abs(g["expected_lse"] - math.log1p(math.e)) < 1e-15
    D = g["shape"]["D"]
    for dt in (torch.float16, torch.bfloat16, torch.float64):
        q = torch.zeros(1, 1, 1, D, dtype=dt)
        k = torch.zeros(1, 1, 2, D, dtype=dt)
        v = torch.empty(1, 1, 2, D, dtype=dt)
        q[0, 0, 0, 0] = g["q_e0"]
        k[0, 0, 1, 0] = g["k1_e0"]
        v[0, 0, 0, :] = g["v0"]
        v[0, 0, 1, :] = g["v1"]
        o, lse = _run(orc, q, k, v, g["scale"])
        assert np.all(np.abs(o - g["expected_o"]) <= 4e-16), (dt, o.ravel()[:4])
        assert abs(lse.item() - g["expected_lse"]) <= 4e-16, (dt, lse)


def pin_single_key(orc):
    """Lk = 1: the only weight is 1, so O = V_0 exactly and LSE = s_0.

    Integer-valued q and k make s_0 = scale * q.k exact in fp64."""
    rng = _rng(11)
    D = 16
    q = rng.integers(-3, 4, size=(1, 3, 5, D)).astype(np.float64)
    k = rng.integers(-3, 4, size=(1, 3, 1, D)).astype(np.float64)
    v = _f64((1, 3, 1, D), rng)
    o, lse = _run(orc, q, k, v, 0.5)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    expect = 0.5 * np.einsum("bhid,bhjd->bhi", q, k)
    assert np.array_equal(lse, expect), (lse, expect)


def pin_two_keys_closed_form(orc):
    """Lk = 2: O = sigmoid(s0-s1) V0 + sigmoid(s1-s0) V1, LSE = logaddexp(s0, s1).

    Includes scores near 1e3, which overflow exp() unless the row maximum is
    subtracted first, and a zero score gap."""
    D = 8
    for s0, s1 in [(0.0, 1.0), (2.5, -3.25), (1000.0, 999.5), (-700.0, -705.0), (7.0, 7.0),
                   (0.0, 40.0)]:
        q = np.zeros((1, 1, 1, D))
        q[..., 0] = 1.0
        k = np.zeros((1, 1, 2, D))
        k[0, 0, 0, 0] = s0
        k[0, 0, 1, 0] = s1
        v = _f64((1, 1, 2, D), _rng(int(abs(s0) + abs(s1)) + 3))
        o, lse = _run(orc, q, k, v, 1.0)
        w0 = scipy.special.expit(s0 - s1)
        w1 = scipy.special.expit(s1 - s0)
        expect = w0 * v[0, 0, 0] + w1 * v[0, 0, 1]
        assert np.all(np.isfinite(o)) and np.isfinite(lse).all(), (s0, s1)
        assert np.allclose(o[0, 0, 0], expect, rtol=1e-14, atol=1e-15), (s0, s1)
        assert abs(lse.item() - np.logaddexp(s0, s1)) <= 1e-13 * max(1.0, abs(s0)), (s0, s1)


def pin_constant_values(orc):
    """If every value row is the same vector c, O = c; LSE does not depend on V."""
    rng = _rng(12)
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 7, 33, 16
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    c = _f64((D,), rng)
    v = np.broadcast_to(c, (B, Hkv, Lk, D)).copy()
    o, lse = _run(orc, q, k, v, 0.3)
    assert np.allclose(o, np.broadcast_to(c, o.shape), rtol=1e-14, atol=1e-15)
    _, lse2 = _run(orc, q, k, _f64((B, Hkv, Lk, D), rng), 0.3)
    assert np.array_equal(lse, lse2)


def pin_identical_keys(orc):
    """All keys equal k: uniform weights, O = mean_j V_j, LSE = scale q.k + ln Lk."""
    rng = _rng(13)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 5, 24, 8
    q = rng.integers(-4, 5, size=(B, Hq, Lq, D)).astype(np.float64)
    kk = rng.integers(-4, 5, size=(D,)).astype(np.float64)
    k = np.broadcast_to(kk, (B, Hkv, Lk, D)).copy()
    v = _f64((B, Hkv, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 0.25)
    mean_v = v.mean(axis=2)  # [B,Hkv,D]
    assert np.allclose(o, mean_v[:, :, None, :], rtol=1e-13, atol=1e-14)
    expect = 0.25 * (q @ kk) + math.log(Lk)
    assert np.allclose(lse, expect, rtol=0, atol=1e-13)


def pin_zero_scale(orc):
    """scale = 0: all scores vanish, O = mean of V, LSE = ln Lk."""
    rng = _rng(14)
    B, Hq, Hkv, Lq, Lk, D = 1, 3, 3, 4, 19, 8
    q = _f64((B, Hq, Lq, D), rng, 5.0)
    k = _f64((B, Hkv, Lk, D), rng, 5.0)
    v = _f64((B, Hkv, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 0.0)
    assert np.allclose(o, v.mean(axis=2)[:, :, None, :], rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, math.log(Lk), rtol=0, atol=1e-14)


def pin_dominant_key(orc):
    """One score at least 40 above every other: O = V_j* to within Lk e^-40, LSE = s_j*."""
    rng = _rng(15)
    D, Lk = 8, 50
    q = np.zeros((1, 1, 1, D))
    q[..., 0] = 1.0
    k = _f64((1, 1, Lk, D), rng)
    k[..., 0] = rng.uniform(-5, 5, size=Lk)
    star = 17
    k[0, 0, star, 0] = 50.0
    v = _f64((1, 1, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 1.0)
    assert np.allclose(o[0, 0, 0], v[0, 0, star], rtol=0, atol=Lk * math.exp(-40) * 4)
    assert abs(lse.item() - 50.0) <= Lk * math.exp(-40) + 1e-13


def pin_gqa_is_repeated_kv(orc):
    """GQA equals MHA with each KV head repeated for Hq/Hkv consecutive query heads (bitwise)."""
    rng = _rng(16)
    B, Hq, Hkv, Lq, Lk, D = 2, 8, 2, 6, 13, 16
    q = torch.from_numpy(_f64((B, Hq, Lq, D), rng)).to(torch.float16)
    k = torch.from_numpy(_f64((B, Hkv, Lk, D), rng)).to(torch.float16)
    v = torch.from_numpy(_f64((B, Hkv, Lk, D), rng)).to(torch.float16)
    o, lse = _run(orc, q, k, v, 0.25)
    kr = k.repeat_interleave(Hq // Hkv, dim=1)
    vr = v.repeat_interleave(Hq // Hkv, dim=1)
    o2, lse2 = _run(orc, q, kr, vr, 0.25)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # and it is not the other plausible map (head h -> KV head h % Hkv)
    kt = k.repeat(1, Hq // Hkv, 1, 1)
    vt = v.repeat(1, Hq // Hkv, 1, 1)
    o3, _ = _run(orc, q, kt, vt, 0.25)
    assert not np.allclose(o, o3)


def pin_permutations(orc):
    """Permuting keys with their values leaves O and LSE unchanged (up to summation
    rounding); permuting query rows permutes the output rows exactly."""
    rng = _rng(17)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 9, 40, 16
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    v = _f64((B, Hkv, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 0.4)
    perm = rng.permutation(Lk)
    o2, lse2 = _run(orc, q, k[:, :, perm], v[:, :, perm], 0.4)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)
    qp = rng.permutation(Lq)
    o3, lse3 = _run(orc, q[:, :, qp], k, v, 0.4)
    assert np.array_equal(o3, o[:, :, qp]) and np.array_equal(lse3, lse[:, :, qp])


def pin_key_shift(orc):
    """Adding u to every key adds scale q.u to every score of a row: O is unchanged,
    LSE moves by exactly that amount."""
    rng = _rng(18)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 2, 4, 21, 8
    q = rng.integers(-3, 4, size=(B, Hq, Lq, D)).astype(np.float64)
    k = rng.integers(-3, 4, size=(B, Hkv, Lk, D)).astype(np.float64)
    u = rng.integers(-3, 4, size=(D,)).astype(np.float64)
    v = _f64((B, Hkv, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 0.125)
    o2, lse2 = _run(orc, q, k + u, v, 0.125)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse2 - lse, 0.125 * (q @ u), rtol=0, atol=1e-12)


def pin_linear_in_values(orc):
    """O is linear in V for fixed Q, K: O(aV1 + bV2) = a O(V1) + b O(V2)."""
    rng = _rng(19)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 5, 17, 8
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    v1 = _f64((B, Hkv, Lk, D), rng)
    v2 = _f64((B, Hkv, Lk, D), rng)
    o1, _ = _run(orc, q, k, v1, 0.3)
    o2, _ = _run(orc, q, k, v2, 0.3)
    o3, _ = _run(orc, q, k, 2.0 * v1 - 3.0 * v2, 0.3)
    assert np.allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-12, atol=1e-13)


def pin_identity_values_give_softmax(orc):
    """With V = identity (Lk = D), row i of O is the softmax row itself: it must equal
    scipy.special.softmax of the scores, and LSE scipy.special.logsumexp."""
    rng = _rng(20)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 6, 16, 16
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    v = np.eye(Lk)[None, None]
    o, lse = _run(orc, q, k, v, 0.7)
    scores = 0.7 * np.matmul(q, np.swapaxes(k, -1, -2))
    assert np.allclose(o, scipy.special.softmax(scores, axis=-1), rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, scipy.special.logsumexp(scores, axis=-1), rtol=0, atol=1e-13)
    assert np.allclose(o.sum(axis=-1), 1.0, rtol=0, atol=1e-14)


def pin_numpy_crosscheck(orc):
    """The C oracle and the independent NumPy evaluation agree to 1e-13 on tiny
    random shapes (MHA and GQA, Lk != D so transposed operands would show)."""
    rng = _rng(21)
    for (B, Hq, Hkv, Lq, Lk, D) in [(1, 1, 1, 1, 1, 1), (1, 2, 1, 3, 5, 4), (2, 6, 3, 5, 7, 8),
                                    (1, 4, 4, 8, 3, 6), (2, 8, 2, 4, 9, 5)]:
        q = _f64((B, Hq, Lq, D), rng)
        k = _f64((B, Hkv, Lk, D), rng)
        v = _f64((B, Hkv, Lk, D), rng)
        o, lse = _run(orc, q, k, v, 0.37)
        o2, lse2 = numpy_ref.attention(q, k, v, 0.37)
        assert np.allclose(o, o2, rtol=1e-13, atol=1e-13), (B, Hq, Hkv, Lq, Lk, D)
        assert np.allclose(lse, lse2, rtol=1e-13, atol=1e-13), (B, Hq, Hkv, Lq, Lk, D)


def pin_fp16_widening(orc):
    """Every finite fp16 bit pattern widens to the value numpy's float16 holds."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.widen(int(b), oracle_pkg.F16) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref)) and np.array_equal(np.isnan(got),
                                                                           np.isnan(ref))


def pin_bf16_widening(orc):
    """Every finite bf16 bit pattern widens to the value torch's bfloat16 holds."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.widen(int(b) & 0xFFFF, oracle_pkg.BF16) for b in bits.tolist()])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def pin_sixteen_bit_inputs_match_f64(orc):
    """The fp16/bf16 entry equals the fp64 entry fed the widened values (bitwise), with
    subnormal fp16 values present."""
    rng = _rng(22)
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 5, 11, 16
    for dt in (torch.float16, torch.bfloat16):
        q = torch.from_numpy(_f64((B, Hq, Lq, D), rng)).to(dt)
        k = torch.from_numpy(_f64((B, Hkv, Lk, D), rng)).to(dt)
        v = torch.from_numpy(_f64((B, Hkv, Lk, D), rng, 1e-5)).to(dt)  # fp16 subnormals
        o, lse = _run(orc, q, k, v, 0.25)
        o2, lse2 = _run(orc, q.double(), k.double(), v.double(), 0.25)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2), dt


def pin_row_subset(orc):
    """Selected rows equal the corresponding rows of the full evaluation, in the order
    asked; an out-of-range row index is an error."""
    rng = _rng(23)
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 6, 9, 8
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    v = _f64((B, Hkv, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 0.5)
    rows = np.array([47, 0, 5, 13, 47, B * Hq * Lq - 1], dtype=np.int64)
    o2, lse2 = orc.attention(q, k, v, 0.5, rows=rows)
    assert np.array_equal(o2, o.reshape(-1, D)[rows])
    assert np.array_equal(lse2, lse.reshape(-1)[rows])
    try:
        orc.attention(q, k, v, 0.5, rows=np.array([B * Hq * Lq], dtype=np.int64))
    except ValueError:
        pass
    else:
        raise AssertionError("out-of-range row accepted")


# ---- causal masking: query i sees key j only if j <= i + (Lk - Lq) ----

def pin_causal_identical_keys(orc):
    """All keys equal: row i averages exactly its visible values V_0..V_{i+Lk-Lq}, with
    LSE = scale q.k + ln(count); rows that see no key (Lq > Lk) give O = 0, LSE = -inf.
    Covers Lq < Lk, Lq = Lk and Lq > Lk, so a shifted or top-left diagonal shows."""
    rng = _rng(31)
    D = 8
    for Lq, Lk in [(5, 24), (9, 9), (30, 24), (1, 6)]:
        q = rng.integers(-4, 5, size=(1, 2, Lq, D)).astype(np.float64)
        kk = rng.integers(-4, 5, size=(D,)).astype(np.float64)
        k = np.broadcast_to(kk, (1, 1, Lk, D)).copy()
        v = _f64((1, 1, Lk, D), rng)
        o, lse = _run(orc, q, k, v, 0.25, causal=True)
        for h in range(2):
            for i in range(Lq):
                n = min(max(i + Lk - Lq + 1, 0), Lk)
                if n == 0:
                    assert np.array_equal(o[0, h, i], np.zeros(D)), (Lq, Lk, i)
                    assert lse[0, h, i] == -np.inf, (Lq, Lk, i)
                    continue
                assert np.allclose(o[0, h, i], v[0, 0, :n].mean(axis=0), rtol=1e-13,
                                   atol=1e-14), (Lq, Lk, i)
                expect = 0.25 * float(q[0, h, i] @ kk) + math.log(n)
                assert abs(lse[0, h, i] - expect) <= 1e-13, (Lq, Lk, i)


def pin_causal_is_prefix_attention(orc):
    """A causal row equals the unmasked attention of that row over its visible prefix
    of keys (bitwise: the same sums in the same order)."""
    rng = _rng(32)
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 6, 10, 8
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    v = _f64((B, Hkv, Lk, D), rng)
    o, lse = _run(orc, q, k, v, 0.3, causal=True)
    for i in range(Lq):
        n = i + Lk - Lq + 1
        o2, lse2 = _run(orc, q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], 0.3)
        assert np.array_equal(o[:, :, i], o2[:, :, 0]) and np.array_equal(lse[:, :, i],
                                                                           lse2[:, :, 0]), i
    # and the unmasked result differs wherever a key is hidden
    o3, _ = _run(orc, q, k, v, 0.3)
    assert not np.allclose(o3[:, :, 0], o[:, :, 0])
    assert np.array_equal(o3[:, :, -1], o[:, :, -1])  # the last row sees every key


def pin_causal_numpy_crosscheck(orc):
    """C oracle and NumPy evaluation agree on causal tiny shapes (square, wide, tall)."""
    rng = _rng(33)
    for (B, Hq, Hkv, Lq, Lk, D) in [(1, 2, 1, 4, 4, 4), (2, 4, 2, 3, 8, 5), (1, 2, 2, 9, 5, 6),
                                    (1, 3, 1, 1, 7, 3)]:
        q = _f64((B, Hq, Lq, D), rng)
        k = _f64((B, Hkv, Lk, D), rng)
        v = _f64((B, Hkv, Lk, D), rng)
        o, lse = _run(orc, q, k, v, 0.45, causal=True)
        with np.errstate(divide="ignore", invalid="ignore"):
            o2, lse2 = numpy_ref.attention(q, k, v, 0.45, causal=True)
        assert np.allclose(o, o2, rtol=1e-13, atol=1e-13), (B, Hq, Hkv, Lq, Lk, D)
        fin = np.isfinite(lse2)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.allclose(lse[fin], lse2[fin], rtol=1e-13, atol=1e-13)


# ---- partial results over key ranges and their merge ----

def pin_key_slice_is_sliced_input(orc):
    """Without masking, the partial result over keys [a, b) is the attention over the
    sliced K and V; with causal masking the slice keeps the global key positions."""
    rng = _rng(34)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 5, 12, 4
    q = _f64((B, Hq, Lq, D), rng)
    k = _f64((B, Hkv, Lk, D), rng)
    v = _f64((B, Hkv, Lk, D), rng)
    a, b = 3, 9
    o, lse = _run(orc, q, k[:, :, a:b], v[:, :, a:b], 0.6, key_begin=a, lk_total=Lk)
    o2, lse2 = _run(orc, q, k[:, :, a:b], v[:, :, a:b], 0.6)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    oc, lc = _run(orc, q, k[:, :, a:b], v[:, :, a:b], 0.6, causal=True, key_begin=a,
                  lk_total=Lk)
    for i in range(Lq):
        n = min(max(i + Lk - Lq + 1 - a, 0), b - a)  # visible keys of the slice
        if n == 0:
            assert lc[0, 0, i] == -np.inf and not oc[0, 0, i].any()
            continue
        oi, li = _run(orc, q[:, :, i:i + 1], k[:, :, a:a + n], v[:, :, a:a + n], 0.6)
        assert np.array_equal(oc[:, :, i], oi[:, :, 0]) and np.array_equal(lc[:, :, i],
                                                                           li[:, :, 0])


def pin_merge_of_key_splits(orc):
    """Merging the partial results over a split of the keys gives the full result, with
    and without causal masking (some causal parts are empty for early rows)."""
    rng = _rng(35)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 7, 20, 6
    q = _f64((B, Hq, Lq, D), rng, 1.5)
    k = _f64((B, Hkv, Lk, D), rng, 1.5)
    v = _f64((B, Hkv, Lk, D), rng)
    cuts = [0, 4, 13, 17, 20]
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, 0.5, causal=causal)
        parts = [orc.attention(q, k[:, :, a:b], v[:, :, a:b], 0.5, causal=causal, key_begin=a,
                               lk_total=Lk) for a, b in zip(cuts[:-1], cuts[1:])]
        om, lm = orc.merge([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(om, o, rtol=1e-13, atol=1e-13), causal
        assert np.allclose(lm, lse, rtol=1e-13, atol=1e-13), causal


def pin_merge_identities(orc):
    """Merge of one part is that part; empty parts (LSE = -inf) carry no weight; two
    equal parts give the same output with LSE + ln 2; the order of parts does not
    matter; two parts with LSE 0 and ln 3 weigh 1/4 and 3/4."""
    rng = _rng(36)
    n, D = 5, 4
    o1 = _f64((n, D), rng)
    o2 = _f64((n, D), rng)
    l1 = rng.uniform(-3, 3, n)
    l2 = rng.uniform(-3, 3, n)
    om, lm = orc.merge([o1], [l1])
    assert np.array_equal(om, o1) and np.array_equal(lm, l1)
    empty = np.full(n, -np.inf)
    om, lm = orc.merge([o1, np.zeros((n, D))], [l1, empty])
    assert np.allclose(om, o1, rtol=1e-15, atol=0) and np.allclose(lm, l1, rtol=1e-15, atol=0)
    om, lm = orc.merge([np.zeros((n, D))] * 2, [empty, empty])
    assert not om.any() and np.all(lm == -np.inf)
    om, lm = orc.merge([o1, o1], [l1, l1])
    assert np.allclose(om, o1, rtol=1e-14, atol=1e-15)
    assert np.allclose(lm, l1 + math.log(2), rtol=0, atol=1e-14)
    oa, la = orc.merge([o1, o2], [l1, l2])
    ob, lb = orc.merge([o2, o1], [l2, l1])
    assert np.allclose(oa, ob, rtol=1e-14, atol=1e-15) and np.allclose(la, lb, atol=1e-14)
    om, lm = orc.merge([o1, o2], [np.zeros(n), np.full(n, math.log(3))])
    assert np.allclose(om, 0.25 * o1 + 0.75 * o2, rtol=1e-14, atol=1e-15)
    assert np.allclose(lm, math.log(4), rtol=0, atol=1e-14)
    # large LSE values must not overflow
    om, lm = orc.merge([o1, o2], [np.full(n, 800.0), np.full(n, 800.0)])
    assert np.all(np.isfinite(om)) and np.allclose(lm, 800 + math.log(2), atol=1e-12)


def pin_empty_sizes(orc):
    """No keys (Lk = 0): every row's weighted sum and exponential sum are empty, so O = 0
    and LSE = ln 0 = -inf, with or without the mask and for 16-bit inputs; an empty key
    slice merged with the rest leaves the rest unchanged.  No query rows (B, Hq or Lq = 0):
    results of shape (0, D) and (0,)."""
    rng = _rng(37)
    D = 8
    q = _f64((2, 4, 3, D), rng)
    k0 = np.zeros((2, 2, 0, D))
    for causal in (False, True):
        o, lse = _run(orc, q, k0, k0, 0.5, causal=causal)
        assert o.shape == (2, 4, 3, D) and not o.any(), causal
        assert np.all(lse == -np.inf), causal
    q16 = torch.from_numpy(q).to(torch.float16)
    k16 = torch.zeros((2, 2, 0, D), dtype=torch.float16)
    o, lse = _run(orc, q16, k16, k16, 0.5)
    assert not o.any() and np.all(lse == -np.inf)
    qf, kf, vf = _f64((1, 2, 4, D), rng), _f64((1, 1, 6, D), rng), _f64((1, 1, 6, D), rng)
    o_full, l_full = orc.attention(qf, kf, vf, 0.3)
    o_e, l_e = orc.attention(qf, kf[:, :, 6:], vf[:, :, 6:], 0.3, key_begin=6, lk_total=6)
    assert not o_e.any() and np.all(l_e == -np.inf)
    om, lm = orc.merge([o_full, o_e], [l_full, l_e])
    assert np.array_equal(om, o_full) and np.array_equal(lm, l_full)
    for qs, ks in [((0, 4, 3, D), (0, 2, 5, D)), ((2, 0, 3, D), (2, 2, 5, D)),
                   ((2, 4, 0, D), (2, 2, 5, D)), ((2, 4, 0, D), (2, 2, 0, D))]:
        o, lse = orc.attention(np.zeros(qs), _f64(ks, rng), _f64(ks, rng), 0.5)
        assert o.shape == (0, D) and lse.shape == (0,), (qs, ks)


PINS = [
    pin_worked_example,
    pin_single_key,
    pin_two_keys_closed_form,
    pin_constant_values,
    pin_identical_keys,
    pin_zero_scale,
    pin_dominant_key,
    pin_gqa_is_repeated_kv,
    pin_permutations,
    pin_key_shift,
    pin_linear_in_values,
    pin_identity_values_give_softmax,
    pin_numpy_crosscheck,
    pin_fp16_widening,
    pin_bf16_widening,
    pin_sixteen_bit_inputs_match_f64,
    pin_row_subset,
    pin_causal_identical_keys,
    pin_causal_is_prefix_attention,
    pin_causal_numpy_crosscheck,
    pin_key_slice_is_sliced_input,
    pin_merge_of_key_splits,
    pin_merge_identities,
    pin_empty_sizes,
]
