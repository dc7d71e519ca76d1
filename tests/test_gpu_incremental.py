"""GPU parity of the incremental decode loop (append -> promote -> attend)
against the oracle at every step, with the page table checked bit-exact
against the oracle's classification after every step."""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu


def run_incremental(T0, steps, B, kv_heads, cfg_id=4, check_every=1, label=""):
    import torch
    require_gpu()
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=B, kv_heads=kv_heads, with_f64=True)
    cfg = d["cfg"]
    dt = cfg["dtype"]
    P, s, w = cfg["P"], cfg["s"], cfg["w"]
    cache = make_cache(d, max_tokens=T0 + steps)
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    cache.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    inc = oracle.IncrementalDecoder(d["K64"], d["V64"], P, s, w, cfg["r_k"], cfg["r_v"], dt)
    promos = []
    worst = 0.0
    for t in range(steps):
        T = T0 + t
        pend = cache.append(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous())
        if pend:
            with pytest.raises(pkv.PKVError) as ei:  # must promote before the next append
                cache.append(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous())
            assert ei.value.status == 5
            cache.promote()
            promos.append(t + 1)
        else:
            with pytest.raises(pkv.PKVError) as ei:
                cache.promote()
            assert ei.value.status == 4
        if (t + 1) % check_every and t + 1 != steps:
            continue
        qs = synth.step_queries(cfg_id, t, d["B"], d["Hq"], 128, dt)
        o = to_f64(cache.decode(to_dev(qs, dt)))
        torch.cuda.synchronize()
        ref_s, ref_e = inc.step(synth.storage_to_f64(qs, dt), T + 1)
        err = rel_err(o, ref_s)
        worst = max(worst, err)
        assert err <= TOL[dt], (t, err)
        cls, slot = cache.page_table(-(-(T + 1) // P))
        ocls, oslot = oracle.classify(T + 1, P, s, w)
        np.testing.assert_array_equal(cls, ocls, err_msg=f"step {t}")
        np.testing.assert_array_equal(slot, oslot, err_msg=f"step {t}")
    print(f"[incremental {label}] steps={steps} promotions at {promos} worst err={worst:.3e}")
    return promos


def test_incremental_reduced():
    promos = run_incremental(64 * 10, 200, B=2, kv_heads=2, label="reduced")
    assert promos == [64, 128, 192]


def test_incremental_from_short_prefill():
    # starts inside the sink and crosses the window fill-up
    promos = run_incremental(30, 300, B=1, kv_heads=2, label="short start")
    assert promos == [64 * k - 30 for k in range(4, 6)]


def test_append_capacity():
    require_gpu()
    d = synth.decode_inputs(2, T=70, B=1, kv_heads=1)
    cache = make_cache(d, max_tokens=65)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    cache.prefill(Kd[:, :, :64].contiguous(), Vd[:, :, :64].contiguous())
    cache.append(Kd[:, :, 64].contiguous(), Vd[:, :, 64].contiguous())
    with pytest.raises(pkv.PKVError) as ei:
        cache.append(Kd[:, :, 65].contiguous(), Vd[:, :, 65].contiguous())
    assert ei.value.status == 3
    assert cache.state() == (65, 0, False)
