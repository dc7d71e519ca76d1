"""Attention under HIP graph capture: the library allocates nothing and never
synchronizes in pkv_decode_attn / pkv_decode_attn_batch, so a model can
capture the attention of all its layers once and replay it.  Every replay,
with eager work and synchronizations between replays and a new query written
into the captured buffer, must give the eager result bit for bit."""
import pytest

import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import make_cache, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _layers(n_layers, T, store=None, P=64):
    d = synth.decode_inputs(2, T=T, B=2, kv_heads=2)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    caches = []
    for _ in range(n_layers):
        c = make_cache(d, store=store, P=P)
        c.prefill(Kd, Vd)
        caches.append(c)
    return caches, d


@pytest.mark.parametrize("store,P", [(None, 64), ("int4", 64), (None, 32)])
def test_captured_attention_replays_exactly(store, P):
    import torch
    require_gpu()
    caches, d = _layers(4, 64 * 30 + 11, store, P)
    q = to_dev(d["q"], "bf16").clone()
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda:0") for _ in caches]
    wss = [c.workspace(0) for c in caches]
    # eager references for two queries
    q2 = to_dev(synth.step_queries(2, 5, d["B"], d["Hq"], 128, "bf16"), "bf16")
    ref1 = [c.decode(q, n_split=0, workspace=w).clone() for c, w in zip(caches, wss)]
    ref2 = [c.decode(q2, n_split=0, workspace=w).clone() for c, w in zip(caches, wss)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        for c, o, w in zip(caches, outs, wss):
            c.decode(q, out=o, workspace=w)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c, o, w in zip(caches, outs, wss):
            c.decode(q, out=o, workspace=w)
    for rep in range(4):
        q.copy_(q2 if rep % 2 else to_dev(d["q"], "bf16"))
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, r1, r2 in zip(outs, ref1, ref2):
            assert torch.equal(o, r2 if rep % 2 else r1), rep
        # eager work between replays
        caches[0].decode(q2, workspace=wss[0])
        torch.cuda.synchronize()


def test_captured_batched_attention_replays_exactly():
    import torch
    require_gpu()
    lengths = [64 * 20 + 3, 64 * 5, 90]
    caches = []
    for i, T in enumerate(lengths):
        d = synth.decode_inputs(2, T=T, B=1, kv_heads=2)
        c = make_cache(d)
        c.prefill(to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16"))
        caches.append(c)
    Hq = d["Hq"]
    q = to_dev(synth.step_queries(2, 0, len(lengths), Hq, 128, "bf16"), "bf16")
    ws = pkv.batch_workspace(caches)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
    ref = pkv.decode_batch(caches, q, workspace=ws).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pkv.decode_batch(caches, q, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pkv.decode_batch(caches, q, out=out, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        pkv.decode_batch(caches, q, workspace=ws)  # eager work between replays
        torch.cuda.synchronize()
