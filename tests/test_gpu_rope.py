"""GPU parity of caches holding pre-RoPE keys (PuzzleKV App. D.3 "RoPE Key
Analysis"; pkv_cache_set_key_rope).

The oracle stores and factorizes the keys as given and rotates every key,
dense or reconstructed, at its token index before the scores; the GPU must
match it to the same gates as the post-RoPE caches (bf16 storage 1e-2,
fp32 storage 1e-4, relative to max |o_ref|).  Covered: the matrix-core
kernel (bf16: r_K and r_V <= 32, equal or unequal padded ranks; equal
padded ranks up to 64), the VALU kernel (fp32, or unequal padded ranks with
one above 32), positions up to 131071, decode steps (the new key turns
in the merge), promotions and chunked prefill (the channel-major key part),
and the stored factors themselves.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu

BASE = {1: 1e4, 2: 5e5, 3: 1e6, 4: 5e5}  # rotary bases of the workloads' model families


def _freqs(cfg_id):
    return synth.rope_inv_freq(BASE[cfg_id])


def _rope_case(cfg_id, T, B=1, kv_heads=2, r_k=None, r_v=None, n_splits=(0,), label=""):
    import torch
    require_gpu()
    d = synth.decode_inputs(cfg_id, T=T, B=B, kv_heads=kv_heads, with_f64=True)
    cfg = d["cfg"]
    dt = cfg["dtype"]
    rk = cfg["r_k"] if r_k is None else r_k
    rv = cfg["r_v"] if r_v is None else r_v
    f = _freqs(cfg_id)
    cache = make_cache(d, r_k=rk, r_v=rv)
    cache.set_key_rope(f)
    cache.prefill(to_dev(d["K"], dt), to_dev(d["V"], dt))
    q = to_dev(d["q"], dt)
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, 64, cfg["s"], cfg["w"], rk, rv, dt, key_rope=f)
    for ns in n_splits:
        o = to_f64(cache.decode(q, n_split=ns))
        torch.cuda.synchronize()
        e_s, e_e = rel_err(o, ref["o_stored"]), rel_err(o, ref["o_exact"])
        print(f"[pre-RoPE {label} cfg{cfg_id} T={T} r=({rk},{rv}) split={ns}] "
              f"err_vs_stored={e_s:.3e} err_vs_exact={e_e:.3e}")
        assert e_s <= TOL[dt], (label, ns, e_s)
    return cache, d


@pytest.mark.parametrize("cfg_id,T,B,kv,rk,rv,splits", [
    (3, 64 * 40 + 5, 1, 2, 24, 24, (0, 3)),     # matrix cores, r = 24
    (2, 64 * 30 + 37, 2, 2, 16, 16, (0, 1, 64)),  # matrix cores, r = 16, ragged tail
    (2, 64 * 20 + 63, 1, 2, 8, 8, (0,)),       # r = 8
    (2, 64 * 20, 1, 2, 32, 32, (0,)),          # r = 32, page-aligned T
    (2, 64 * 20 + 9, 1, 2, 16, 14, (0,)),      # (16, 14): same padded rank
    (2, 64 * 12 + 7, 1, 2, 24, 16, (0, 2)),    # unequal padded ranks
    (3, 64 * 16 + 33, 1, 2, 8, 24, (0,)),      # key rank below the value rank
    (2, 64 * 14 + 5, 2, 2, 32, 13, (0, 3)),    # unequal, odd value rank (exact-rank part)
    (4, 64 * 11 + 40, 1, 2, 16, 30, (0,)),     # unequal, value rank 30
    (2, 64 * 10 + 50, 1, 2, 40, 40, (0, 2)),   # r > 32: one wave per SIMD, two reduction steps
    (3, 64 * 12 + 3, 1, 2, 64, 64, (0,)),      # full rank of a 64-token page
    (2, 64 * 9 + 17, 2, 1, 56, 52, (0, 3)),    # (56, 52): same padded rank
])
def test_pre_rope_matrix_core_path(cfg_id, T, B, kv, rk, rv, splits):
    _rope_case(cfg_id, T, B, kv, rk, rv, splits, label="mfma")


@pytest.mark.parametrize("cfg_id,T,rk,rv", [
    (2, 64 * 12 + 7, 40, 24),   # unequal, key rank > 32
    (2, 64 * 10 + 50, 24, 48),  # unequal, value rank > 32
    (1, 64 * 16, 16, 16),       # fp32 storage
    (1, 64 * 9 + 3, 64, 64),    # fp32, full rank
])
def test_pre_rope_valu_path(cfg_id, T, rk, rv):
    _rope_case(cfg_id, T, 1, 1, rk, rv, (0, 2), label="valu")


def test_pre_rope_short_caches():
    # all pages dense: sink only, sink + window + partial
    _rope_case(2, 40, 1, 2, label="sink only")
    _rope_case(2, 64 * 3 + 20, 1, 2, label="all dense")


def test_pre_rope_at_long_positions():
    # positions up to 131071: the angles' reduction must stay accurate where
    # t * theta_0 is of the order of 1e5 radians
    _rope_case(3, 131072, 1, 1, n_splits=(0,), label="128K")


def test_pre_rope_factors_are_the_pages_own():
    """The key parts (channel-major Rf_K) hold a rank-r decomposition of the
    unrotated page: unpacked as PKV_KEYS_PRE_ROPE their product meets the
    bf16 reconstruction bound against the oracle's optimal error."""
    import torch
    cache, d = _rope_case(3, 64 * 12, 1, 1, label="factors")
    r = d["cfg"]["r_k"]
    T, nf, _ = cache.state()
    X = d["K64"][0, 0, 64:64 * (1 + nf)].reshape(nf, 64, 128)
    U, S, Wt = oracle.svd_batch(X)
    opt = oracle.optimal_error(S, r)
    for f in range(nf):
        part = cache.factor_part(0, 0, f, pkv.KEYS).cpu().numpy()
        torch.cuda.synchronize()
        Lf, Rf = pkv.unpack_factors(pkv.KEYS_PRE_ROPE, r, pkv.BF16, part.view(np.uint16))
        err = np.linalg.norm(X[f] - Lf.astype(np.float64) @ Rf.astype(np.float64))
        nrm = np.linalg.norm(X[f])
        bound = np.hypot(1.001 * opt[f] + 1e-5 * nrm, 2.0 ** -8 * nrm)
        assert err <= bound, (f, err, opt[f], bound)


@pytest.mark.parametrize("rk,rv", [(None, None), (48, 48), (40, 13)])
def test_pre_rope_decode_steps_against_oracle(rk, rv):
    """pkv_decode_step on a pre-RoPE cache: the new key is rotated at its
    position in the merge, promotions store channel-major key parts; checked
    against the oracle at every step.  Ranks: the workload's r = 16; r = 48
    (the one-wave matrix-core format, promotions on the Jacobi route);
    (40, 13) (vector-ALU kernel, an exact-rank value part written by the
    Jacobi route)."""
    import torch
    require_gpu()
    cfg_id, T0, steps = 4, 64 * 10 + 3, 140
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=2, kv_heads=2, with_f64=True)
    cfg = d["cfg"]
    dt = cfg["dtype"]
    f = _freqs(cfg_id)
    rk = cfg["r_k"] if rk is None else rk
    rv = cfg["r_v"] if rv is None else rv
    cache = make_cache(d, r_k=rk, r_v=rv, max_tokens=T0 + steps)
    cache.set_key_rope(f)
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    cache.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    inc = oracle.IncrementalDecoder(d["K64"], d["V64"], 64, cfg["s"], cfg["w"], rk, rv, dt, key_rope=f)
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
    print(f"[pre-RoPE step vs oracle r=({rk},{rv})] {steps} steps, worst err {worst:.3e}")


def test_pre_rope_chunked_prefill_matches_one_shot():
    import torch
    require_gpu()
    d = synth.decode_inputs(3, T=3000, B=1, kv_heads=2, with_f64=True)
    cfg = d["cfg"]
    f = _freqs(3)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    one = make_cache(d)
    one.set_key_rope(f)
    one.prefill(Kd, Vd)
    ch = make_cache(d)
    ch.set_key_rope(f)
    ch.prefill(Kd[:, :, :0].contiguous(), Vd[:, :, :0].contiguous())
    T = 0
    for C in (700, 1300, 64, 936):
        ch.prefill_chunk(Kd[:, :, T:T + C].contiguous(), Vd[:, :, T:T + C].contiguous())
        T += C
    torch.cuda.synchronize()
    assert one.state() == ch.state()
    for h in range(2):
        for s in range(one.state()[1]):
            for kind in (pkv.KEYS, pkv.VALUES):
                assert torch.equal(one.factor_part(0, h, s, kind), ch.factor_part(0, h, s, kind))
    q = to_dev(d["q"], "bf16")
    oa, ob = one.decode(q), ch.decode(q)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], 3000, 64, cfg["s"], cfg["w"], cfg["r_k"], cfg["r_v"],
                        "bf16", key_rope=f)
    assert rel_err(to_f64(oa), ref["o_stored"]) <= TOL["bf16"]


def test_pre_rope_errors():
    require_gpu()
    d = synth.decode_inputs(2, T=200, B=1, kv_heads=1)
    cache = make_cache(d)
    cache.prefill(to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16"))
    with pytest.raises(pkv.PKVError) as ei:  # not on a filled cache
        cache.set_key_rope(_freqs(2))
    assert ei.value.status == 1
    cache.prefill(to_dev(d["K"], "bf16")[:, :, :0].contiguous(), to_dev(d["V"], "bf16")[:, :, :0].contiguous())
    cache.set_key_rope(_freqs(2))  # emptied: allowed
    q4 = make_cache(d, store="int4")
    with pytest.raises(pkv.PKVError) as ei:
        q4.set_key_rope(_freqs(2))
    assert ei.value.status == 2
