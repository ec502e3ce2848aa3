"""The C ABI under HIP graph capture (torch.cuda.CUDAGraph on ROCm): the one-pass launch
and the split launch (attention into a caller-owned workspace, then the merge) are
captured once and replayed several times, with the program's own eager work and
synchronisations between the replays; every replay must equal the eager result bit for
bit.  The library allocates nothing and records no memset, so capture needs nothing
beyond what the caller preallocates.
"""
import pytest
import torch

import attn_inputs
import flash_attention_amd as fa
from parity_util import scale_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal,nsplit", [(False, 1), (True, 1), (False, 4), (True, 3)])
def test_capture_and_replay(causal, nsplit):
    print("\n[case] graph causal=%s nsplit=%d" % (causal, nsplit), flush=True)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, Lq, Lk, D = 2, 8, 2, 100, 1500, 128
    q, k, v = (t.to(dev) for t in attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "f16", seed=31))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev)
    ws_bytes = fa.attn_workspace_bytes(B, Hq, Lq, D, nsplit)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    kw = dict(scale=scale_of(D), out=o, lse=lse, causal=causal, nsplit=nsplit,
              workspace=ws if nsplit > 1 else None)
    fa.fwd(q, k, v, **kw)  # eager (also sets the kernels' LDS attribute before capture)
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fa.fwd(q, k, v, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)  # stale partials must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        # eager work of the program between replays
        x = (q.float() * 2).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(x)
