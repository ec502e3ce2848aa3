"""GPU parity of the causal mask, the key-split path, the partial results and the merge
kernel, through the C ABI, against the fp64 oracle.

Causal: row i sees key j only if j <= i + Lk - Lq; rows that see no key (Lq > Lk) must
come out as O = 0 and LSE = -inf exactly.  Splits: the merged result must meet the same
tolerances as one pass; every partial must match the oracle's attention over its key
range alone.  Every case prints its name, shape and seed before it touches the GPU.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs
import flash_attention_amd as fa
import oracle
from parity_util import check, gpu_fwd, metrics, parity, scale_of

pytestmark = pytest.mark.gpu


def _announce(what):
    print("\n[case] %s" % what, flush=True)


def _causal_cases():
    shapes = [  # B, Hq, Hkv, Lq, Lk
        (1, 2, 1, 256, 256), (1, 4, 2, 300, 300), (1, 2, 1, 1024, 1024), (2, 4, 1, 97, 1000),
        (1, 8, 2, 8, 4096), (1, 2, 2, 700, 300), (1, 2, 1, 513, 64), (1, 1, 1, 1, 1),
        (1, 16, 1, 33, 33), (1, 4, 4, 1000, 1100),
    ]
    cases = []
    i = 0
    for D in (128, 256):
        for dt in ("f16", "bf16"):
            for sh in shapes:
                cases.append((*sh, D, dt, 9000 + 10 * i))
                i += 1
    return cases


CAUSAL = _causal_cases()


@pytest.mark.parametrize("case", CAUSAL, ids=["B%d_H%d_%d_L%dx%d_D%d_%s_s%d" % c for c in CAUSAL])
def test_causal_parity(case):
    B, Hq, Hkv, Lq, Lk, D, dt, seed = case
    _announce("causal " + str(case))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed)
    parity(q, k, v, scale_of(D), dt, what="causal " + str(case), causal=True)


# Shapes whose heads fill whole 256-row query tiles and whose grid gives each XCD several
# heads: the causal launch then deals each XCD's tiles position-major over chunks of
# heads (chunk sizes 4, 4 with a partial last chunk of 2, 4 with two key splits, 3).
ORDER = [  # B, Hq, Hkv, Lq, Lk, D, dtype, nsplit, seed
    (1, 32, 2, 1024, 1024, 256, "f16", 1, 9501), (5, 6, 1, 256, 300, 128, "bf16", 1, 9502),
    (2, 16, 2, 512, 512, 128, "f16", 2, 9503), (1, 24, 2, 768, 800, 256, "bf16", 1, 9504),
]


@pytest.mark.parametrize("case", ORDER, ids=["B%d_H%d_%d_L%dx%d_D%d_%s_n%d_s%d" % c
                                             for c in ORDER])
def test_causal_dispatch_order(case):
    """Every query tile is computed once whatever order the workgroups take them in."""
    B, Hq, Hkv, Lq, Lk, D, dt, nsplit, seed = case
    _announce("causal dispatch order " + str(case))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed)
    parity(q, k, v, scale_of(D), dt, what="causal order " + str(case), causal=True,
           nsplit=nsplit)


@pytest.mark.parametrize("D,dt", [(128, "f16"), (256, "bf16")])
def test_causal_first_row_is_exact(D, dt):
    """Lq = Lk: row 0 sees key 0 alone, so its weight is exactly 1 and O equals V_0 bit
    for bit; the last row sees every key and equals the unmasked result bit for bit."""
    _announce("causal first/last row D=%d %s" % (D, dt))
    q, k, v = attn_inputs.make_qkv(1, 4, 2, 300, 300, D, dt, seed=21)
    o, lse = gpu_fwd(q, k, v, scale_of(D), causal=True)
    v_rep = v.repeat_interleave(2, dim=1)
    assert torch.equal(o[:, :, 0], v_rep[:, :, 0])
    s0 = (q[:, :, 0].double() * k.repeat_interleave(2, dim=1)[:, :, 0].double()).sum(-1)
    assert torch.allclose(lse[:, :, 0].double(), s0 * float(np.float32(scale_of(D))), atol=1e-4)
    o_full, lse_full = gpu_fwd(q, k, v, scale_of(D))
    assert torch.equal(o[:, :, -1], o_full[:, :, -1])
    assert torch.equal(lse[:, :, -1], lse_full[:, :, -1])


def test_causal_empty_rows_exact():
    """Lq > Lk: the first Lq - Lk rows see no key: O = 0 and LSE = -inf, bit for bit."""
    _announce("causal empty rows")
    q, k, v = attn_inputs.make_qkv(1, 4, 2, 600, 100, 256, "f16", seed=22)
    o, lse = gpu_fwd(q, k, v, scale_of(256), causal=True)
    assert torch.equal(o[:, :, :500], torch.zeros_like(o[:, :, :500]))
    assert bool(torch.all(lse[:, :, :500] == -math.inf))
    assert bool(torch.isfinite(lse[:, :, 500:]).all())


@pytest.mark.parametrize("causal", [False, True])
def test_causal_and_split_deterministic(causal):
    _announce("determinism causal=%s nsplit=3" % causal)
    q, k, v = attn_inputs.make_qkv(1, 8, 2, 700, 2000, 256, "f16", seed=23)
    o1, l1 = gpu_fwd(q, k, v, scale_of(256), causal=causal, nsplit=3)
    o2, l2 = gpu_fwd(q, k, v, scale_of(256), causal=causal, nsplit=3)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _split_cases():
    cases = []
    i = 0
    for (B, Hq, Hkv, Lq, Lk) in [(1, 4, 2, 200, 1000), (2, 2, 1, 64, 3000), (1, 8, 8, 300, 700),
                                 (1, 2, 1, 1000, 129), (1, 4, 1, 16, 4096)]:
        for D, dt in ((128, "bf16"), (256, "f16")):
            for nsplit in (2, 5, 0):
                for causal in (False, True):
                    cases.append((B, Hq, Hkv, Lq, Lk, D, dt, nsplit, causal, 9500 + i))
                    i += 1
    return cases


SPLIT = _split_cases()


@pytest.mark.parametrize("case", SPLIT,
                         ids=["B%d_H%d_%d_L%dx%d_D%d_%s_ns%d_c%d_s%d" % c for c in SPLIT])
def test_split_parity(case):
    B, Hq, Hkv, Lq, Lk, D, dt, nsplit, causal, seed = case
    _announce("split " + str(case))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed)
    parity(q, k, v, scale_of(D), dt, what="split " + str(case), causal=causal, nsplit=nsplit)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nsplit", [1, 3, 40])
def test_partials_match_oracle_ranges(nsplit, causal):
    """Each split's partial result is the oracle's attention over that key range alone
    (key positions global, so the causal diagonal stays put); splits past the end, or past
    a row's diagonal, are empty (O = 0, LSE = -inf)."""
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 300, 1000, 128
    _announce("partials nsplit=%d causal=%s" % (nsplit, causal))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "f16", seed=24)
    scale = float(np.float32(scale_of(D)))
    dev = torch.device("cuda:0")
    o_part, lse_part = fa.fwd_partial(q.to(dev), k.to(dev), v.to(dev), nsplit, scale=scale,
                                      causal=causal)
    torch.cuda.synchronize()
    o_part, lse_part = o_part.cpu(), lse_part.cpu()
    for s in range(nsplit):
        b, e = fa.attn_split_range(Lk, nsplit, s)
        if b == e:
            assert not o_part[s].any() and bool(torch.all(lse_part[s] == -math.inf)), s
            continue
        o_ref, lse_ref = oracle.attention(q, k[:, :, b:e].contiguous(), v[:, :, b:e].contiguous(),
                                          scale, causal=causal, key_begin=b, lk_total=Lk)
        m = metrics(o_part[s].reshape(-1, D), lse_part[s].reshape(-1), o_ref, lse_ref)
        print("[partial] split %d [%d,%d) %s" % (s, b, e, m), flush=True)
        check(m, "f16", "partial %d" % s)


@pytest.mark.parametrize("D,out", [(128, torch.float16), (256, torch.bfloat16),
                                   (8, torch.float32), (136, torch.float32)])
def test_merge_kernel_matches_oracle(D, out):
    """Random partials (LSE spread over +-30, some parts empty, one row empty in every
    part) merged on the GPU against the oracle's fp64 merge."""
    _announce("merge D=%d out=%s" % (D, out))
    P, rows = 5, 3001
    g = torch.Generator().manual_seed(25)
    o_part = torch.randn(P, rows, D, generator=g)
    lse_part = torch.rand(P, rows, generator=g) * 60 - 30
    lse_part[1, ::3] = -math.inf  # empty parts carry no weight
    lse_part[:, 7] = -math.inf    # a row empty in every part
    o_part[:, 7] = 0
    dev = torch.device("cuda:0")
    o, lse = fa.merge(o_part.to(dev), lse_part.to(dev), out_dtype=out)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge(o_part.double().numpy(), lse_part.double().numpy())
    og = o.cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    assert not og[7].any() and lg[7] == -math.inf
    fin = np.isfinite(lse_ref)
    assert np.isfinite(lg[fin]).all() and np.isfinite(og).all()
    # fp32 arithmetic, then rounding to the output type
    tol = {torch.float32: 2e-6, torch.float16: 2e-3, torch.bfloat16: 1.6e-2}[out]
    err = np.abs(og - o_ref).max()
    assert err <= tol * max(1.0, np.abs(o_ref).max()), err
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-5 * 30, np.abs(lg[fin] - lse_ref[fin]).max()


@pytest.mark.parametrize("P,rows,D", [(8, 3, 128), (16, 1, 256), (33, 7, 136), (64, 40, 128),
                                      (130, 5, 256), (256, 1, 128), (256, 300, 8)])
def test_merge_many_parts_few_rows(P, rows, D):
    """Decode-sized merges (many key ranges, few rows), where the parts are dealt over
    several wavefronts of a workgroup and summed in LDS: against the oracle's merge, with
    empty parts and a row empty in every part."""
    _announce("merge P=%d rows=%d D=%d" % (P, rows, D))
    g = torch.Generator().manual_seed(27 + P + rows)
    o_part = torch.randn(P, rows, D, generator=g)
    lse_part = torch.rand(P, rows, generator=g) * 40 - 20
    lse_part[::3, :] = -math.inf     # every third part empty
    if rows > 1:
        lse_part[:, rows - 1] = -math.inf  # the last row empty in every part
    o_part[::3] = float("nan")       # an empty part's output is never read
    dev = torch.device("cuda:0")
    o, lse = fa.merge(o_part.to(dev), lse_part.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge(torch.nan_to_num(o_part).double().numpy(),
                                  lse_part.double().numpy())
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    if rows > 1:
        assert not og[rows - 1].any() and lg[rows - 1] == -math.inf
    fin = np.isfinite(lse_ref)
    assert fin.any()
    assert np.isfinite(og).all() and np.isfinite(lg[fin]).all()
    assert np.abs(og - o_ref).max() <= 2e-6 * max(1.0, np.abs(o_ref).max())
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-5 * 20


@pytest.mark.parametrize("P,rows,order", [(16, 2048, "rising"), (16, 2048, "falling"),
                                          (64, 32, "rising"), (7, 513, "last_dominates")])
def test_merge_rescales_across_batches(P, rows, order):
    """The merge takes the parts in batches and rescales its running sums whenever a batch
    brings a larger LSE: LSE rising part by part (every batch rescales), falling (none
    does), and the last part of every row 120 above all others (once it arrives, the
    others' weights exp(-120) underflow to 0 in fp32): against the oracle's merge."""
    _announce("merge rescale P=%d rows=%d %s" % (P, rows, order))
    g = torch.Generator().manual_seed(29 + P)
    o_part = torch.randn(P, rows, 256, generator=g)
    base = torch.rand(P, rows, generator=g) * 2
    steps = torch.arange(P, dtype=torch.float32)[:, None] * 3.0
    if order == "rising":
        lse_part = base + steps
    elif order == "falling":
        lse_part = base - steps
    else:
        lse_part = base.clone()
        lse_part[P - 1] += 120.0
    dev = torch.device("cuda:0")
    o, lse = fa.merge(o_part.to(dev), lse_part.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge(o_part.double().numpy(), lse_part.double().numpy())
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert np.abs(og - o_ref).max() <= 2e-6 * max(1.0, np.abs(o_ref).max())
    assert np.abs(lg - lse_ref).max() <= 1e-5 * max(1.0, np.abs(lse_ref).max())


def test_merge_without_lse_and_single_part():
    """lse = NULL leaves no LSE; one part merges to itself (weight exactly 1)."""
    _announce("merge single part")
    g = torch.Generator().manual_seed(26)
    o_part = torch.randn(1, 100, 64, generator=g)
    lse_part = torch.randn(1, 100, generator=g)
    dev = torch.device("cuda:0")
    o, lse = fa.merge(o_part.to(dev), lse_part.to(dev), lse=False)
    torch.cuda.synchronize()
    assert lse is None and torch.equal(o.cpu(), o_part[0])


BOUNDARY = [(G, Lq, D, causal, nsplit)
            for (G, Lq) in [(1, 127), (8, 16), (1, 129), (16, 8), (4, 33)]
            for D in (128, 256) for causal, nsplit in ((False, 1), (True, 0))]


@pytest.mark.parametrize("G,Lq,D,causal,nsplit", BOUNDARY)
def test_narrow_wide_boundary(G, Lq, D, causal, nsplit):
    """Key/value groups of 127, 128 (narrow 128-row workgroups) and 129, 132 rows (wide
    256-row workgroups): the planner's shape choice and parity on both sides of it."""
    B, Hkv, Lk = 2, 2, 700
    Hq = G * Hkv
    narrow = G * Lq <= 128
    plan = fa.attn_plan(B, Hq, Hkv, Lq, Lk, D, fa.ATTN_F16)
    assert plan.block_m == (128 if narrow else 256)
    assert plan.kernel.decode().endswith("_m128") == narrow
    seed = 14000 + G * 1000 + Lq + D
    _announce("boundary G=%d Lq=%d rows=%d D=%d causal=%d nsplit=%d seed=%d"
              % (G, Lq, G * Lq, D, causal, nsplit, seed))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "f16", seed=seed)
    parity(q, k, v, scale_of(D), "f16", causal=causal, nsplit=nsplit,
           what="boundary G=%d Lq=%d D=%d" % (G, Lq, D))


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,D,causal,nsplit", [
    (3000, 4, 2, 3, 37, 128, False, 1),    # many batch entries, tiny heads (narrow shape)
    (1200, 2, 1, 70, 33, 256, True, 1),    # many batch entries, 140 rows per group (wide)
    (2, 256, 1, 1, 3000, 128, True, 0),    # 256 query heads on one key/value head, decode
    (1, 64, 1, 5, 5000, 256, False, 0),    # 320 rows per group over long keys, split
])
def test_large_batch_and_wide_groups(B, Hq, Hkv, Lq, Lk, D, causal, nsplit):
    """Batch and head indices far from the small cases (grid ids past 10^4, block
    renumbering over many XCD rounds) and very wide query groups, on sampled rows."""
    seed = 15000 + B + Hq + Lq
    _announce("large B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d causal=%d nsplit=%d seed=%d"
              % (B, Hq, Hkv, Lq, Lk, D, causal, nsplit, seed))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "bf16", seed=seed)
    total = B * Hq * Lq
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(total, size=min(3000, total), replace=False),
                                     [0, total - 1]])).astype(np.int64)
    parity(q, k, v, scale_of(D), "bf16", rows=rows, causal=causal, nsplit=nsplit,
           what="large B=%d Hq=%d" % (B, Hq))


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,D,causal,nsplit", [
    (1, 2, 1, 1, 1, 128, False, 1), (2, 4, 2, 37, 77, 128, True, 1), (1, 8, 2, 300, 500, 256,
                                                                        False, 3),
    (1, 16, 1, 8, 999, 256, True, 0), (3, 2, 2, 129, 31, 128, True, 2), (1, 4, 1, 1000, 64,
                                                                          256, False, 1)])
def test_nothing_written_outside_the_outputs(B, Hq, Hkv, Lq, Lk, D, causal, nsplit):
    """O, LSE and the partial results sit inside larger buffers filled with a sentinel:
    after the launches every byte before and after them still holds it (ragged tails, the
    16-byte output stores, both tile shapes, splits and the merge), and Q, K, V are
    unchanged."""
    _announce("guard bands B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d causal=%d nsplit=%d"
              % (B, Hq, Hkv, Lq, Lk, D, causal, nsplit))
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "f16",
                                                     seed=16000 + Lq))
    q0, k0, v0 = q.clone(), k.clone(), v.clone()
    G = 4096  # guard elements on each side (16-byte aligned for both element sizes)
    n_o, n_l = B * Hq * Lq * D, B * Hq * Lq
    obuf = torch.full((n_o + 2 * G,), 7.0, dtype=torch.float16, device=dev)
    lbuf = torch.full((n_l + 2 * G,), 7.0, dtype=torch.float32, device=dev)
    o = obuf[G:G + n_o].view(B, Hq, Lq, D)
    lse = lbuf[G:G + n_l].view(B, Hq, Lq)
    fa.fwd(q, k, v, out=o, lse=lse, causal=causal, nsplit=nsplit)
    ns = max(nsplit, 2)
    n_p, n_pl = ns * n_o, ns * n_l
    pbuf = torch.full((n_p + 2 * G,), 7.0, dtype=torch.float32, device=dev)
    plbuf = torch.full((n_pl + 2 * G,), 7.0, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    rc = fa.attn_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             pbuf[G:].data_ptr(), plbuf[G:].data_ptr(), B, Hq, Hkv, Lq, Lk, D,
                             D ** -0.5, fa.ATTN_F16, fa.ATTN_CAUSAL if causal else 0, ns, s)
    assert rc == 0
    torch.cuda.synchronize()
    for buf, n in ((obuf, n_o), (lbuf, n_l), (pbuf, n_p), (plbuf, n_pl)):
        assert bool((buf[:G] == 7).all()) and bool((buf[G + n:] == 7).all())
    assert not bool(torch.isnan(o.float()).any())
    assert torch.equal(q, q0) and torch.equal(k, k0) and torch.equal(v, v0)  # inputs untouched


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,D,causal", [
    (4, 32, 2, 16, 4096, 256, True), (1, 32, 8, 1, 8192, 128, False),
    (1, 16, 1, 8, 999, 256, True), (1, 8, 2, 200, 3000, 128, False)])
def test_c_entry_with_planner_splits(B, Hq, Hkv, Lq, Lk, D, causal):
    """attn_fwd_ex called through the C ABI with nsplit = 0, so that the library plans the
    key splits itself: parity with the oracle, and O, LSE and the workspace inside sentinel
    guard bands that no launch may touch."""
    flags = fa.ATTN_CAUSAL if causal else 0
    plan = fa.attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, fa.ATTN_F16, flags)
    seed = 17000 + Lq + Lk
    _announce("C entry nsplit=0 (planner %d) B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d causal=%d "
              "seed=%d" % (plan.nsplit, B, Hq, Hkv, Lq, Lk, D, causal, seed))
    dev = torch.device("cuda:0")
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "f16", seed=seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    G = 65536  # guard bytes on each side
    n_o, n_l, n_w = B * Hq * Lq * D * 2, B * Hq * Lq * 4, max(plan.workspace_bytes, 256)
    bufs = [torch.full((n + 2 * G,), 0x5A, dtype=torch.uint8, device=dev) for n in (n_o, n_l, n_w)]
    o_ptr, l_ptr, w_ptr = (b.data_ptr() + G for b in bufs)
    rc = fa.attn_fwd_ex(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_ptr, l_ptr, B, Hq, Hkv,
                        Lq, Lk, D, D ** -0.5, fa.ATTN_F16, flags, 0, w_ptr, n_w,
                        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fa.attn_strerror(rc)
    torch.cuda.synchronize()
    for b, n in zip(bufs, (n_o, n_l, n_w)):
        assert bool((b[:G] == 0x5A).all()) and bool((b[G + n:] == 0x5A).all())
    o = bufs[0][G:G + n_o].view(torch.float16).view(B, Hq, Lq, D).cpu()
    lse = bufs[1][G:G + n_l].view(torch.float32).view(B, Hq, Lq).cpu()
    o_ref, lse_ref = oracle.attention(q, k, v, float(np.float32(D ** -0.5)), causal=causal)
    m = metrics(o.reshape(-1, D), lse.reshape(-1), o_ref, lse_ref)
    check(m, "f16", "C entry nsplit=0")


def _random_cases(n=48, seed=20261202):
    """Seeded random mixes of every option: shapes with ragged tails, GQA ratios, both
    head dims and dtypes, causal or not, split counts (0 = the planner's), scale sign."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        lq = int(rng.integers(1, 700))
        lk = int(rng.integers(1, 2500))
        d = int(rng.choice([128, 256]))
        dt = str(rng.choice(["f16", "bf16"]))
        causal = bool(rng.integers(0, 2))
        nsplit = int(rng.choice([1, 1, 2, 3, 7, 0]))
        sgn = -1.0 if rng.random() < 0.15 else 1.0
        cases.append((int(rng.integers(1, 3)), hkv * g, hkv, lq, lk, d, dt, causal, nsplit, sgn,
                      13000 + i))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=["r%d_B%d_H%d_%d_L%dx%d_D%d_%s_c%d_ns%d_%+d" % (
    i, *c[:8], c[8], int(c[9])) for i, c in enumerate(RANDOM)])
def test_random_options(case):
    B, Hq, Hkv, Lq, Lk, D, dt, causal, nsplit, sgn, seed = case
    _announce("random " + str(case))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed)
    parity(q, k, v, sgn * scale_of(D), dt, what="random " + str(case), causal=causal,
           nsplit=nsplit)
