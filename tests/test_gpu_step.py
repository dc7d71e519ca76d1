"""GPU tests of pkv_decode_step, the one-call decode step (append, promote when
due, attend), whose append is folded into the cross-split merge.

- Against the separate calls (pkv_append, pkv_promote_page, pkv_decode_attn)
  on a twin cache fed the same tokens: page tables and the whole cache buffer
  bit-identical after every step; outputs equal to float32 rounding (the new
  token's state joins at the cross-split merge instead of inside its page),
  max |o_step - o_sep| <= 1e-5 max |o_sep|.
- Against the oracle's incremental decoder at every step (tolerance of the
  storage dtype), including page completions and promotions.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _twin_caches(d, T0, steps, **kw):
    import torch
    cfg = d["cfg"]
    dt = cfg["dtype"]
    a = make_cache(d, max_tokens=T0 + steps, **kw)
    b = make_cache(d, max_tokens=T0 + steps, **kw)
    a.buffer.zero_()
    b.buffer.zero_()
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    a.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    b.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    torch.cuda.synchronize()
    return a, b, Kd, Vd


def _step_vs_separate(cfg_id, T0, steps, B, kv_heads, label, **kw):
    import torch
    require_gpu()
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=B, kv_heads=kv_heads)
    dt = d["cfg"]["dtype"]
    a, b, Kd, Vd = _twin_caches(d, T0, steps, **kw)
    ws_a = a.workspace(512)
    promos = 0
    worst = 0.0
    for t in range(steps):
        T = T0 + t
        k = Kd[:, :, T].contiguous()
        v = Vd[:, :, T].contiguous()
        q = to_dev(synth.step_queries(cfg_id, t, d["B"], d["Hq"], 128, dt), dt)
        oa = a.step(k, v, q, workspace=ws_a)
        if b.append(k, v):
            b.promote()
            promos += 1
        ob = b.decode(q)
        torch.cuda.synchronize()
        assert a.state() == b.state(), (t, a.state(), b.state())
        xa, xb = oa.cpu().numpy().astype(np.float64), ob.cpu().numpy().astype(np.float64)
        worst = max(worst, rel_err(xa, xb))
        assert rel_err(xa, xb) <= 1e-5, (label, t, rel_err(xa, xb))
        n = -(-(T + 1) // 64)
        for x, y in zip(a.page_table(n), b.page_table(n)):
            np.testing.assert_array_equal(x, y, err_msg=f"{label} step {t}")
    assert torch.equal(a.buffer, b.buffer), label
    print(f"[step vs separate {label}] {steps} steps, {promos} promotions: caches bit-identical, "
          f"worst output difference {worst:.2e}")
    return promos


def test_step_matches_separate_calls():
    # crosses two page completions, one promotion each
    assert _step_vs_separate(2, 64 * 12 + 40, 100, B=2, kv_heads=2, label="llama-shape") == 2


def test_step_from_empty_cache():
    # T = 0: the first step attends to the new token alone
    _step_vs_separate(2, 0, 70, B=1, kv_heads=2, label="from T=0")


def test_step_in_sink_region():
    # the first tokens fill the sink page, then the window, no promotion yet
    _step_vs_separate(2, 5, 150, B=1, kv_heads=2, label="from T=5")


def test_step_without_window():
    # w = 0: each completed page is promoted by the step that completes it
    _step_vs_separate(2, 64 * 4 + 60, 70, B=1, kv_heads=1, label="w=0", w=0)


def test_step_fp32_cache():
    # fp32 storage (generic attention kernel)
    _step_vs_separate(1, 64 * 6 + 10, 60, B=1, kv_heads=1, label="fp32")


@pytest.mark.parametrize("rk,rv", [(None, None), (48, 13), (8, 40)])
def test_step_against_oracle(rk, rv):
    """Incremental decode driven by pkv_decode_step, checked against the
    oracle at every step (workload-4 recipe, reduced batch and heads), at
    the workload's ranks and at unequal ranks with one above 32 (promotions
    on the Jacobi route, exact-rank value part at (48, 13))."""
    import torch
    require_gpu()
    cfg_id, T0, steps = 4, 64 * 10 + 3, 140
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=2, kv_heads=2, with_f64=True)
    cfg = d["cfg"]
    dt = cfg["dtype"]
    rk = cfg["r_k"] if rk is None else rk
    rv = cfg["r_v"] if rv is None else rv
    cache = make_cache(d, r_k=rk, r_v=rv, max_tokens=T0 + steps)
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    cache.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    inc = oracle.IncrementalDecoder(d["K64"], d["V64"], 64, cfg["s"], cfg["w"], rk, rv, dt)
    ws = cache.workspace(512)
    worst = 0.0
    for t in range(steps):
        T = T0 + t
        qs = synth.step_queries(cfg_id, t, d["B"], d["Hq"], 128, dt)
        o = to_f64(cache.step(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous(), to_dev(qs, dt),
                              workspace=ws))
        torch.cuda.synchronize()
        ref_s, _ = inc.step(synth.storage_to_f64(qs, dt), T + 1)
        err = rel_err(o, ref_s)
        worst = max(worst, err)
        assert err <= TOL[dt], (t, err)
        cls, slot = cache.page_table(-(-(T + 1) // 64))
        ocls, oslot = oracle.classify(T + 1, 64, cfg["s"], cfg["w"])
        np.testing.assert_array_equal(cls, ocls, err_msg=f"step {t}")
        np.testing.assert_array_equal(slot, oslot, err_msg=f"step {t}")
    print(f"[step vs oracle r=({rk},{rv})] {steps} steps, worst err {worst:.3e}")


def test_step_errors():
    import torch
    require_gpu()
    d = synth.decode_inputs(2, T=70, B=1, kv_heads=1)
    cache = make_cache(d, max_tokens=66)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    cache.prefill(Kd[:, :, :65].contiguous(), Vd[:, :, :65].contiguous())
    q = to_dev(d["q"], "bf16")
    k, v = Kd[:, :, 65].contiguous(), Vd[:, :, 65].contiguous()
    small = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(pkv.PKVError) as ei:
        cache.step(k, v, q, workspace=small)
    assert ei.value.status == 3
    assert cache.state()[0] == 65  # nothing changed
    cache.step(k, v, q)
    assert cache.state()[0] == 66
    with pytest.raises(pkv.PKVError) as ei:  # full
        cache.step(k, v, q)
    assert ei.value.status == 3


def test_step_with_early_factorization():
    """Pages factorized early on an auxiliary stream: outputs and caches
    bit-identical to the synchronous step, across several promotions."""
    import torch
    require_gpu()
    cfg_id, T0, steps = 2, 64 * 12 + 40, 300
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=2, kv_heads=2)
    dt = d["cfg"]["dtype"]
    a, b, Kd, Vd = _twin_caches(d, T0, steps)
    aux = torch.cuda.Stream()
    a.set_aux_stream(aux)
    ws_a, ws_b = a.workspace(512), b.workspace(512)
    promos = 0
    for t in range(steps):
        T = T0 + t
        k = Kd[:, :, T].contiguous()
        v = Vd[:, :, T].contiguous()
        q = to_dev(synth.step_queries(cfg_id, t, d["B"], d["Hq"], 128, dt), dt)
        nf = b.state()[1]
        oa = a.step(k, v, q, workspace=ws_a)
        ob = b.step(k, v, q, workspace=ws_b)
        promos += b.state()[1] > nf
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), (t, (oa - ob).abs().max().item())
        assert a.state() == b.state()
    aux.synchronize()
    assert torch.equal(a.buffer, b.buffer)
    print(f"[early factorization] {steps} steps, {promos} promotions: bit-identical")
    assert promos >= 4


def test_aux_stream_switching():
    import torch
    require_gpu()
    d = synth.decode_inputs(2, T=64 * 8, B=1, kv_heads=1)
    cache = make_cache(d, max_tokens=64 * 8)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    cache.prefill(Kd[:, :, :64 * 4 + 62].contiguous(), Vd[:, :, :64 * 4 + 62].contiguous())
    aux = torch.cuda.Stream()
    cache.set_aux_stream(aux)
    q = to_dev(d["q"], "bf16")
    for T in (64 * 4 + 62, 64 * 4 + 63):  # the second step completes a window page
        cache.step(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous(), q)
    with pytest.raises(pkv.PKVError) as ei:  # its factorization is outstanding
        cache.set_aux_stream(None)
    assert ei.value.status == 5
    torch.cuda.synchronize()
    # a prefill resets the cache (and orders itself after the early work)
    cache.prefill(Kd[:, :, :100].contiguous(), Vd[:, :, :100].contiguous())
    cache.set_aux_stream(None)
    cache.set_aux_stream(aux)
