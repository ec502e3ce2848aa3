"""GPU parity: the HIP kernels through the C ABI against the fp64 oracle, element by
element, plus the invariants that hold exactly (or bitwise) on the GPU.

Every case prints its name, shape and seed before it touches the GPU.
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


def _sweep():
    shapes = [  # B, Hq, Hkv, Lq, Lk
        (1, 2, 1, 128, 128), (1, 4, 1, 256, 256), (1, 2, 2, 512, 512), (1, 2, 1, 1024, 1024),
        (1, 4, 2, 128, 1024), (1, 2, 1, 1024, 128), (1, 1, 1, 1, 1), (2, 4, 2, 17, 33),
        (1, 2, 1, 129, 257), (1, 16, 1, 64, 200), (1, 8, 1, 100, 64), (2, 8, 4, 300, 190),
    ]
    dists = [("normal", 1.0), ("uniform", 1.0), ("normal", 4.0)]
    cases = []
    i = 0
    for D in (128, 256):
        for dt in ("f16", "bf16"):
            for sh in shapes:
                dist, km = dists[i % 3]
                cases.append((*sh, D, dt, dist, km, 7000 + 10 * i))
                i += 1
    return cases


SWEEP = _sweep()


@pytest.mark.parametrize("case", SWEEP, ids=["B%d_H%d_%d_L%dx%d_D%d_%s_%s_k%g_s%d" % c
                                             for c in SWEEP])
def test_parity_sweep(case):
    B, Hq, Hkv, Lq, Lk, D, dt, dist, km, seed = case
    _announce(str(case))
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed, dist=dist, k_mult=km)
    parity(q, k, v, scale_of(D), dt, what=str(case))


@pytest.mark.parametrize("name", list(attn_inputs.WORKLOADS))
def test_parity_workload_full_size(name):
    """The benchmark workloads at full size, in the launch the benchmark times; the
    oracle checks a seeded subset of rows (all rows for the tiny case)."""
    w = attn_inputs.WORKLOADS[name]
    _announce("%s %s" % (name, w.describe()))
    q, k, v = attn_inputs.workload_qkv(w)
    rows = None if name == "tiny" else attn_inputs.sample_rows(w)
    parity(q, k, v, w.scale, w.dtype, rows=rows, what=name, causal=w.causal, nsplit=w.nsplit)


OTHER_DTYPE = ["gqa4k_d256", "gqa8k_d128_bf16", "rect1kx16k_d256", "gqa16k_d256",
               "gqa16k_d256_causal"]


@pytest.mark.parametrize("name", OTHER_DTYPE)
def test_parity_workload_other_dtype(name):
    """The same full-size workloads with the other 16-bit input type (fp16 <-> bf16), so
    that both kernels of each head dimension run at the benchmark's sizes."""
    import dataclasses
    w = attn_inputs.WORKLOADS[name]
    w = dataclasses.replace(w, dtype="bf16" if w.dtype == "f16" else "f16",
                            seed_base=w.seed_base + 500)
    _announce("%s other dtype %s" % (name, w.describe()))
    q, k, v = attn_inputs.workload_qkv(w)
    rows = attn_inputs.sample_rows(w, n_random=512)
    parity(q, k, v, w.scale, w.dtype, rows=rows, what=name + " " + w.dtype, causal=w.causal,
           nsplit=w.nsplit)


def test_worked_example_on_gpu():
    """Two keys, D=256, scale 1/16: O = -tanh(1/2) in every coordinate, LSE = ln(1+e)."""
    _announce("worked example")
    D = 256
    q = torch.zeros(1, 1, 1, D, dtype=torch.float16)
    k = torch.zeros(1, 1, 2, D, dtype=torch.float16)
    v = torch.empty(1, 1, 2, D, dtype=torch.float16)
    q[..., 0] = 4.0
    k[0, 0, 1, 0] = 4.0
    v[0, 0, 0] = 1.0
    v[0, 0, 1] = -1.0
    o, lse = gpu_fwd(q, k, v, 1.0 / 16)
    assert torch.allclose(o.double(), torch.full_like(o.double(), -math.tanh(0.5)), atol=1e-3)
    # the fp16 row sum adds the rounded weights 1 and e^-1: half an ulp of e^-1 (2^-13)
    # over the sum 1 + e^-1 bounds the LSE error by 9e-5
    assert abs(lse.item() - math.log1p(math.e)) <= 1e-4


@pytest.mark.parametrize("D,dt", [(128, "f16"), (256, "bf16")])
def test_single_key_is_exact(D, dt):
    """Lk = 1: the weight is exactly 1, so O equals V_0 bit for bit."""
    _announce("single key D=%d %s" % (D, dt))
    q, k, v = attn_inputs.make_qkv(1, 4, 2, 77, 1, D, dt, seed=11)
    o, lse = gpu_fwd(q, k, v, scale_of(D))
    assert torch.equal(o, v.repeat_interleave(2, dim=1).expand(1, 4, 77, D))
    s = (q.double() @ k.double().repeat_interleave(2, dim=1).transpose(-1, -2))[..., 0]
    assert torch.allclose(lse.double(), s * float(np.float32(scale_of(D))), atol=1e-4)


@pytest.mark.parametrize("D,dt", [(128, "bf16"), (256, "f16")])
def test_gqa_equals_repeated_kv_bitwise(D, dt):
    _announce("gqa vs repeated kv D=%d %s" % (D, dt))
    q, k, v = attn_inputs.make_qkv(2, 8, 2, 200, 300, D, dt, seed=12)
    o1, l1 = gpu_fwd(q, k, v, scale_of(D))
    o2, l2 = gpu_fwd(q, k.repeat_interleave(4, dim=1).contiguous(),
                     v.repeat_interleave(4, dim=1).contiguous(), scale_of(D))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D,dt", [(128, "f16"), (256, "f16"), (256, "bf16")])
def test_deterministic(D, dt):
    """Two launches give bitwise equal results (an LDS race would show here)."""
    _announce("determinism D=%d %s" % (D, dt))
    q, k, v = attn_inputs.make_qkv(1, 8, 2, 1000, 1500, D, dt, seed=13)
    o1, l1 = gpu_fwd(q, k, v, scale_of(D))
    o2, l2 = gpu_fwd(q, k, v, scale_of(D))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_query_permutation_permutes_output_bitwise():
    _announce("query permutation")
    D = 256
    q, k, v = attn_inputs.make_qkv(1, 2, 1, 384, 500, D, "f16", seed=14)
    perm = torch.from_numpy(np.random.default_rng(14).permutation(384))
    o1, l1 = gpu_fwd(q, k, v, scale_of(D))
    o2, l2 = gpu_fwd(q[:, :, perm].contiguous(), k, v, scale_of(D))
    assert torch.equal(o2, o1[:, :, perm]) and torch.equal(l2, l1[:, :, perm])


def test_constant_values():
    """Every value row equal to c: O = c up to the rounding of P to fp16."""
    _announce("constant values")
    D = 128
    q, k, _ = attn_inputs.make_qkv(1, 4, 1, 300, 700, D, "f16", seed=15)
    c = torch.linspace(-2, 2, D).to(torch.float16)
    v = c.expand(1, 1, 700, D).contiguous()
    o, _ = gpu_fwd(q, k, v, scale_of(D))
    err = (o.double() - c.double()).abs().max().item()
    assert err <= 4e-3, err


def test_dominant_key():
    """A key whose score exceeds all others by far selects its value row."""
    _announce("dominant key")
    D = 256
    q, k, v = attn_inputs.make_qkv(1, 2, 1, 64, 300, D, "f16", seed=16)
    k[0, 0, 123] = q[0, 0, 0] * 8  # row 0 of head 0: score ~ 8*|q|^2/16 >> others
    o, _ = gpu_fwd(q, k, v, scale_of(D))
    o_ref, lse_ref = oracle.attention(q, k, v, float(np.float32(scale_of(D))), rows=[0])
    assert torch.allclose(o[0, 0, 0].double(), torch.from_numpy(o_ref[0]), atol=2e-3)
    assert torch.allclose(o[0, 0, 0].double(), v[0, 0, 123].double(), atol=2e-3)


@pytest.mark.parametrize("D,dt", [(128, "f16"), (256, "f16"), (256, "bf16")])
def test_subnormal_weights_counted(D, dt):
    """Key 0 (first tile) dominates by 15.5 in log2 units, so every other weight rounds to
    an fp16 subnormal (about 2^-15.5); together they are ~9 % of each row sum, so both the
    P.V product and the row sum must keep them."""
    _announce("subnormal weights D=%d %s" % (D, dt))
    Lq, Lk = 96, 4096
    q, _, v = attn_inputs.make_qkv(1, 2, 1, Lq, Lk, D, dt, seed=19)
    tdt = q.dtype
    q = torch.zeros_like(q)
    q[..., 0] = 8.0
    k = torch.zeros(1, 1, Lk, D, dtype=tdt)
    scale = scale_of(D)
    # s_0 - s_j = 15.5 ln 2 for j > 0 (scores of the other keys are 0)
    k[0, 0, 0, 0] = 15.5 * math.log(2.0) / (scale * 8.0)
    _, _, m = parity(q, k, v, scale, dt, what="subnormal weights")
    assert m["rel_rms"] < (2e-3 if dt == "f16" else 1e-2)


def test_lse_optional_and_output_unchanged():
    _announce("lse NULL")
    D = 128
    q, k, v = attn_inputs.make_qkv(1, 4, 2, 200, 200, D, "bf16", seed=17)
    o1, _ = gpu_fwd(q, k, v, scale_of(D), with_lse=True)
    o2, _ = gpu_fwd(q, k, v, scale_of(D), with_lse=False)
    assert torch.equal(o1, o2)


def test_null_stream_entry_point():
    """attn_fwd (null stream) and attn_fwd_stream give the same bits."""
    _announce("attn_fwd null stream")
    D = 256
    q, k, v = attn_inputs.make_qkv(1, 2, 1, 130, 70, D, "f16", seed=18)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=dev)
    torch.cuda.synchronize()
    rc = fa.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     1, 2, 1, 130, 70, D, 1 / 16, fa.ATTN_F16)
    assert rc == 0
    torch.cuda.synchronize()
    o2, l2 = gpu_fwd(q, k, v, 1 / 16)
    assert torch.equal(o.cpu(), o2) and torch.equal(lse.cpu(), l2)


def test_rejected_call_writes_nothing():
    _announce("rejected call")
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 64, 64, device=dev).half()
    o = torch.full_like(q, float("nan"))
    torch.cuda.synchronize()
    rc = fa.attn_fwd_stream(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), None,
                            1, 2, 2, 64, 64, 64, 0.125, fa.ATTN_F16,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == -3
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()


def test_binding_rejects_mismatched_outputs():
    # caller-provided outputs must match what the kernel writes; a mismatch is refused
    # before anything is launched
    _announce("binding output checks")
    dev = torch.device("cuda:0")
    q = torch.randn(1, 4, 64, 128, device=dev).half()
    k = torch.randn(1, 2, 80, 128, device=dev).half()
    big = torch.full((2, 4, 64, 128), float("nan"), dtype=torch.float16, device=dev)
    bad = [dict(out=big),                                       # wrong shape
           dict(out=big[:1].float()),                           # wrong dtype
           dict(out=torch.empty(1, 4, 128, 64, dtype=torch.float16,
                                device=dev).transpose(2, 3)),    # not contiguous
           dict(lse=torch.empty(1, 4, 65, device=dev)),
           dict(lse=torch.empty(1, 4, 64, device=dev, dtype=torch.float16)),
           dict(workspace=torch.empty(1 << 20, device=dev), nsplit=2)]  # not bytes
    for kw in bad:
        with pytest.raises((ValueError, TypeError)):
            fa.fwd(q, k, k, **kw)
    with pytest.raises(ValueError):
        fa.fwd(q, k.cpu(), k)
    torch.cuda.synchronize()
    assert torch.isnan(big.float()).all()
    o = torch.empty_like(q)
    lse = torch.empty(1, 4, 64, device=dev)
    fa.fwd(q, k, k, out=o, lse=lse)  # matching outputs are accepted
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_scale_sign_and_zero():
    """Negative and zero scales follow the definition (zero: O = mean of V)."""
    _announce("scale sign/zero")
    D = 128
    q, k, v = attn_inputs.make_qkv(1, 2, 1, 96, 160, D, "f16", seed=19)
    parity(q, k, v, -0.2, "f16", what="scale=-0.2")
    o, lse = gpu_fwd(q, k, v, 0.0)
    mean = v.double().mean(dim=2, keepdim=True)
    assert (o.double() - mean).abs().max().item() <= 2e-3
    assert (lse.double() - math.log(160)).abs().max().item() <= 1e-5


def _growing_scores(D, dt, Lk, spikes, seed):
    """Inputs whose per-row maximum score jumps far above the first key tile's maximum at
    the given key positions, so the kernel's softmax reference must be raised mid-sweep.
    Every query gets a shared component 2*u (u a random unit vector); key `pos` is mult*u,
    so its score is about scale*mult*(2 +- 1) for every row."""
    q, k, v = attn_inputs.make_qkv(1, 4, 2, 200, Lk, D, dt, seed=seed)
    g = torch.Generator().manual_seed(seed + 99)
    u = torch.randn(D, generator=g, dtype=torch.float64)
    u = u / u.norm()
    q = (q.double() + 2.0 * u).to(q.dtype)
    for pos, mult in spikes:
        k[0, :, pos] = (u * mult).to(k.dtype)
    return q, k, v


@pytest.mark.parametrize("D,dt", [(256, "f16"), (128, "bf16"), (256, "bf16")])
def test_reference_growth_mid_sweep(D, dt):
    """A score far above the first tile's maximum in a later tile (the wave holding the row
    rescales its accumulator and sums to a higher reference)."""
    _announce("growth mid sweep D=%d %s" % (D, dt))
    q, k, v = _growing_scores(D, dt, 700, [(333, 300.0)], seed=21)
    parity(q, k, v, scale_of(D), dt, what="growth mid")


def test_reference_growth_last_tile_and_repeated():
    """Growth in the very last (ragged) key tile, and several successive jumps."""
    _announce("growth last tile / repeated")
    D = 256
    q, k, v = _growing_scores(D, "f16", 641, [(640, 400.0)], seed=22)
    parity(q, k, v, scale_of(D), "f16", what="growth last key")
    q, k, v = _growing_scores(D, "f16", 900, [(100, 150.0), (300, 300.0), (500, 450.0),
                                              (899, 600.0)], seed=23)
    parity(q, k, v, scale_of(D), "f16", what="growth repeated")


@pytest.mark.parametrize("D,dt,k,growth", [(128, "bf16", 60, False), (256, "bf16", 80, True),
                                          (256, "f16", 8, True)])
def test_values_scaled_by_power_of_two(D, dt, k, growth):
    """V times 2^k gives O times 2^k bit for bit (where O is a normal number of its type) and
    the same LSE: the weights and the accumulation are linear in V, and scaling by a power
    of two rounds nothing while the fp32 accumulator stays in range (bf16 values up to
    ~2^83 here, far above fp16's range, with rescales mid-sweep in the growth cases)."""
    _announce("V scaled by 2^%d D=%d %s growth=%s" % (k, D, dt, growth))
    if growth:
        q, k_, v = _growing_scores(D, dt, 900, [(130, 200.0), (480, 350.0)], seed=31)
    else:
        q, k_, v = attn_inputs.make_qkv(1, 4, 2, 300, 700, D, dt, seed=31)
    if dt == "f16":
        v = (v.double().clamp(-4, 4)).to(v.dtype)  # 4 * 2^8 stays inside fp16
    big = (v.double() * 2.0 ** k).to(v.dtype)
    assert torch.equal(big.double(), v.double() * 2.0 ** k)  # the scaling itself is exact
    o1, l1 = gpu_fwd(q, k_, v, scale_of(D))
    o2, l2 = gpu_fwd(q, k_, big, scale_of(D))
    # an unscaled output below the output type's smallest normal (fp16: 2^-14) is rounded to
    # the subnormal spacing (2^-24), its scaled twin to full precision
    a, b = o1.double(), o2.double() / 2.0 ** k
    normal = a.abs() >= (2.0 ** -14 if dt == "f16" else 2.0 ** -126)
    assert torch.equal(b[normal], a[normal])
    assert bool(((b - a)[~normal].abs() <= 2.0 ** -25).all())
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("D,dt", [(256, "f16"), (128, "bf16")])
def test_reference_growth_in_one_block_only(D, dt):
    """Growth confined to one 32-row query block: every query row is made orthogonal to a
    unit vector u, then rows 32..63 of head 0 get 2u added, and key 333 is 250u.  Only those
    rows see the large score (block 1 of the first wavefront at D=256, the second wavefront
    at D=128), so only that block rescales; every other row keeps its first-tile reference."""
    _announce("growth in one block D=%d %s" % (D, dt))
    q, k, v = attn_inputs.make_qkv(1, 2, 1, 256, 700, D, dt, seed=25)
    g = torch.Generator().manual_seed(125)
    u = torch.randn(D, generator=g, dtype=torch.float64)
    u = u / u.norm()
    qd = q.double()
    qd = qd - (qd @ u)[..., None] * u
    qd[0, 0, 32:64] += 2.0 * u
    q = qd.to(q.dtype)
    k[0, 0, 333] = (u * 250.0).to(k.dtype)
    parity(q, k, v, scale_of(D), dt, what="growth in one block")


@pytest.mark.parametrize("D,dt", [(128, "f16"), (128, "bf16"), (256, "f16")])
@pytest.mark.parametrize("causal,nsplit", [(False, 3), (True, 1), (True, 2)])
def test_reference_growth_with_mask_and_splits(D, dt, causal, nsplit):
    """Scores outgrowing the first tile's maximum, in several tiles (a rescale each time),
    under the causal mask and inside key splits (each split has its own first tile and its
    own reference)."""
    _announce("growth D=%d %s causal=%s nsplit=%d" % (D, dt, causal, nsplit))
    q, k, v = _growing_scores(D, dt, 900, [(130, 200.0), (480, 350.0), (899, 500.0)],
                              seed=24 + nsplit)
    parity(q, k, v, scale_of(D), dt, what="growth causal=%s nsplit=%d" % (causal, nsplit),
           causal=causal, nsplit=nsplit)
