"""attn_fwd_ex_noalloc, the entry point without a caller workspace, against attn_fwd_ex with
a workspace from torch: the same bits, and both within the attention tolerances of the fp64
oracle.  Two calls in a row on the library's one array per GPU, the second with a smaller
input (so stale partials of the first call lie beyond what the second one writes), then the
host-side refusal of a split count whose partials exceed the array, and the planner's
fallback to fewer splits when its own count would not fit."""
import numpy as np
import pytest
import torch

import attn_inputs
import flash_attention_amd as fa
import oracle
from parity_util import check, metrics

pytestmark = pytest.mark.gpu


def _run(entry, q, k, v, causal, nsplit):
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    dev = q.device
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    flags = fa.ATTN_CAUSAL if causal else 0
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = fa.dtype_code(q)
    if entry == "noalloc":
        rc = fa.attn_fwd_ex_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, Hq, Hkv, Lq, Lk, D, scale, code, flags,
                                    nsplit, stream)
    else:
        need = (fa.attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, code, flags).workspace_bytes
                if nsplit == 0 else fa.attn_workspace_bytes(B, Hq, Lq, D, nsplit))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        rc = fa.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), B, Hq, Hkv, Lq, Lk, D, scale, code, flags, nsplit,
                            ws.data_ptr(), need, stream)
    torch.cuda.synchronize()
    return rc, o.cpu(), lse.cpu()


CALLS = [  # B, Hq, Hkv, Lq, Lk, D, dtype, causal, nsplit, seed: the second one smaller
    (4, 32, 2, 16, 16384, 256, "f16", True, 0, 41000),   # decode-like: the planner's splits
    (1, 8, 2, 100, 3000, 128, "bf16", False, 3, 42000),  # three explicit splits
]


def test_noalloc_matches_workspace_entry_twice():
    dev = torch.device("cuda:0")
    for B, Hq, Hkv, Lq, Lk, D, dt, causal, nsplit, seed in CALLS:
        print("\n[case] noalloc B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d %s causal=%s nsplit=%d" %
              (B, Hq, Hkv, Lq, Lk, D, dt, causal, nsplit), flush=True)
        code = fa.ATTN_F16 if dt == "f16" else fa.ATTN_BF16
        if nsplit == 0:
            plan = fa.attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, code, fa.ATTN_CAUSAL if causal else 0)
            assert plan.nsplit > 1 and plan.workspace_bytes <= fa.ATTN_NOALLOC_WORKSPACE_BYTES
        q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, dt, seed=seed)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        rc1, o1, l1 = _run("noalloc", qd, kd, vd, causal, nsplit)
        rc2, o2, l2 = _run("workspace", qd, kd, vd, causal, nsplit)
        assert rc1 == 0 and rc2 == 0, (rc1, rc2)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        rows = attn_inputs.sample_rows(attn_inputs.Workload("x", B, Hq, Hkv, Lq, Lk, D, dt,
                                                            seed_base=seed), n_random=512)
        scale = float(np.float32(1.0 / np.sqrt(D)))
        o_ref, lse_ref = oracle.attention(q, k, v, scale, rows=rows, causal=causal)
        idx = torch.from_numpy(rows)
        m = metrics(o1.reshape(-1, D)[idx], l1.reshape(-1)[idx], o_ref, lse_ref)
        print("[parity] noalloc %s" % m, flush=True)
        check(m, dt, "noalloc")


def test_noalloc_refuses_and_falls_back():
    dev = torch.device("cuda:0")
    # 1K queries x 32 heads x 256 dims: four splits need 128 MiB of fp32 partials
    B, Hq, Hkv, Lq, Lk, D = 1, 32, 2, 1024, 4096, 256
    print("\n[case] noalloc refusal / fallback %s" % ((B, Hq, Hkv, Lq, Lk, D),), flush=True)
    assert fa.attn_workspace_bytes(B, Hq, Lq, D, 4) > fa.ATTN_NOALLOC_WORKSPACE_BYTES
    q, k, v = attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "f16", seed=43000)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    rc, o, _ = _run("noalloc", qd, kd, vd, False, 4)
    assert rc == -12 and torch.isnan(o.float()).all()  # ATTN_E_WORKSPACE, nothing written
    # the planner's own count for this shape may not fit: the entry point takes the most
    # splits that do, and the result is the one-pass result up to rounding
    rc, o, lse = _run("noalloc", qd, kd, vd, False, 0)
    assert rc == 0
    scale = float(np.float32(1.0 / np.sqrt(D)))
    rows = attn_inputs.sample_rows(attn_inputs.Workload("x", B, Hq, Hkv, Lq, Lk, D, "f16",
                                                        seed_base=43000), n_random=512)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, rows=rows)
    idx = torch.from_numpy(rows)
    m = metrics(o.reshape(-1, D)[idx], lse.reshape(-1)[idx], o_ref, lse_ref)
    print("[parity] noalloc fallback %s" % m, flush=True)
    check(m, "f16", "noalloc fallback")
