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


WIDE = (2, 8, 2, 100, 1500, 128)   # 400 rows per key/value group: the wide tile shape
NARROW = (1, 32, 8, 1, 8192, 128)  # decode, 4 rows per group: the narrow shape; the merge
#                                    of 32 parts over 32 rows deals them over 8 wavefronts


@pytest.mark.parametrize("shape,causal,nsplit", [(WIDE, False, 1), (WIDE, True, 1),
                                                 (WIDE, False, 4), (WIDE, True, 3),
                                                 (NARROW, True, 1), (NARROW, True, 32)])
def test_capture_and_replay(shape, causal, nsplit):
    print("\n[case] graph shape=%s causal=%s nsplit=%d" % (shape, causal, nsplit), flush=True)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, Lq, Lk, D = shape
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


def test_concurrent_calls_from_threads():
    """Reentrancy: four host threads, each on its own stream with its own outputs, call the
    library 10 times (one pass, causal with splits, and the merge inside); every result
    equals the single-threaded one bit for bit."""
    import threading
    print("\n[case] four threads, four streams", flush=True)
    dev = torch.device("cuda:0")
    shapes = [(1, 8, 2, 300, 700, 128, False, 1), (2, 4, 1, 64, 2000, 256, True, 0),
              (1, 32, 8, 1, 4096, 128, True, 0), (1, 2, 1, 513, 129, 256, True, 3)]
    inputs, refs = [], []
    for i, (B, Hq, Hkv, Lq, Lk, D, causal, nsplit) in enumerate(shapes):
        q, k, v = (t.to(dev) for t in attn_inputs.make_qkv(B, Hq, Hkv, Lq, Lk, D, "bf16",
                                                         seed=40 + i))
        o, lse = fa.fwd(q, k, v, causal=causal, nsplit=nsplit)
        torch.cuda.synchronize()
        inputs.append((q, k, v, causal, nsplit))
        refs.append((o.clone(), lse.clone()))
    errors = []

    def worker(i):
        try:
            q, k, v, causal, nsplit = inputs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [fa.fwd(q, k, v, causal=causal, nsplit=nsplit, stream=s)
                        for _ in range(10)]
            s.synchronize()
            for o, lse in outs:
                if not (torch.equal(o, refs[i][0]) and torch.equal(lse, refs[i][1])):
                    errors.append(i)
        except Exception as e:  # reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
