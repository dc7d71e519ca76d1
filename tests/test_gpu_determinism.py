"""Run-to-run determinism of the device kernels, a canary for races: every
reduction has a fixed order and every iteration a fixed count, so the same
inputs must give the same bits -- page decompositions (both eigen-solvers,
bf16 / fp32 / INT4 outputs), prefill, attention (plain, INT4, pre-RoPE) and
decode steps."""
import numpy as np
import pytest

import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import make_cache, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("r,out", [(16, "bf16"), (24, "f32"), (40, "bf16")])
def test_compress_pages_is_deterministic(r, out):
    import torch
    require_gpu()
    pages = synth.to_storage(synth.compression_pages(np.arange(2048)), "bf16")  # spectrum + noise pages
    X = to_dev(pages, "bf16")
    out_dtype = torch.bfloat16 if out == "bf16" else torch.float32
    runs = [pkv.compress_pages(X, r, out_dtype=out_dtype) for _ in range(3)]
    torch.cuda.synchronize()
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b)
    for a, b in zip(runs[0], runs[2]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("store,rope,P", [(None, False, 64), ("int4", False, 64), (None, True, 64),
                                          (None, False, 32)])
def test_prefill_and_attention_are_deterministic(store, rope, P):
    import torch
    require_gpu()
    d = synth.decode_inputs(3, T=64 * 300 + 17, B=1, kv_heads=2)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    q = to_dev(d["q"], "bf16")
    outs, parts = [], []
    for _ in range(2):
        c = make_cache(d, store=store, P=P)
        c.buffer.zero_()  # bytes no kernel writes compare equal too
        if rope:
            c.set_key_rope(synth.rope_inv_freq(1e6))
        c.prefill(Kd, Vd)
        outs.append([c.decode(q, n_split=ns) for ns in (0, 7)])
        parts.append(c.buffer.clone())
        torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    assert torch.equal(parts[0], parts[1])  # the whole cache buffer


def test_decode_steps_are_deterministic():
    import torch
    require_gpu()
    T0, steps = 64 * 10 + 50, 40
    d = synth.decode_inputs(2, T=T0 + steps, B=2, kv_heads=2)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    runs = []
    for _ in range(2):
        c = make_cache(d, max_tokens=T0 + steps)
        c.buffer.zero_()
        c.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
        o = []
        for t in range(steps):
            q = to_dev(synth.step_queries(2, t, d["B"], d["Hq"], 128, "bf16"), "bf16")
            o.append(c.step(Kd[:, :, T0 + t].contiguous(), Vd[:, :, T0 + t].contiguous(), q))
        torch.cuda.synchronize()
        runs.append((o, c.buffer.clone()))
    for a, b in zip(runs[0][0], runs[1][0]):
        assert torch.equal(a, b)
    assert torch.equal(runs[0][1], runs[1][1])
