"""GPU parity at the workloads' full sizes, in the launch configurations that
bench.py times (default split counts, one launch over the whole batch).

Every (sequence, KV head) holds its own recipe tokens (its own seeded
streams), so a kernel that read another head's factor slot, ring slot or
query rows would fail:

- Workloads 2 and 3 (one decode and one decode step; workload 3 also with
  INT4 factor pages, workload 2 also in 32-token pages at (16, 14), bf16 and
  INT4): every (sequence, KV head) is reconstructed by the oracle and every
  query head's output is checked (tolerance of the storage dtype, relative to
  max |o_ref| over the tensor).
- Workload 4 (512 incremental steps): the page table at every step; the
  outputs of three (sequence, KV head) pairs -- the first, a middle one and
  the last -- at every one of the 512 steps against the oracle's incremental
  decoder, and of all 64 pairs at each promotion step and the last step.
- Workload 5 (524288 pages): the whole distinct pool drawn on the device
  (synth.compression_pool_device); every noise page and a seeded 1% sample
  of the spectrum pages are checked against the oracle's SVD by the
  reconstruction bound for bf16 factors.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu

WORKERS = 16


@functools.lru_cache(maxsize=2)
def workload_tokens(cfg_id, T):
    """Stored K, V (B, H_kv, T, d) and q (B, H_q, d) of the workload, every
    (sequence, KV head) from its own streams."""
    return synth.decode_inputs(cfg_id, T=T, workers=WORKERS)


def make_full_cache(cfg, max_tokens, store=None):
    return pkv.Cache(batch=cfg["B"], n_q_heads=cfg["Hq"], n_kv_heads=cfg["Hkv"], rank_k=cfg["r_k"],
                     rank_v=cfg["r_v"], sink=cfg["s"], window=cfg["w"], max_tokens=max_tokens,
                     dtype=store or cfg["dtype"], page_len=cfg["P"])


@functools.lru_cache(maxsize=1)
def oracle_svds(cfg_items, T):
    """The oracle's SVDs of every factorized page of every (sequence, KV head,
    K / V) of a workload's cache of length T (page classes of length T):
    {(b, h, kind): (fact pages, U, S, Wt)}."""
    cfg = dict(cfg_items)
    d = workload_tokens(cfg["cfg_id"], cfg["T_gen"])
    P, dt = cfg["P"], cfg["dtype"]
    cls, _ = oracle.classify(T, P, cfg["s"], cfg["w"])
    fact = np.nonzero(cls == oracle.FACT)[0]
    out = {}
    for b in range(cfg["B"]):
        for h in range(cfg["Hkv"]):
            for kind, src in (("K", d["K"]), ("V", d["V"])):
                X = synth.storage_to_f64(src[b, h, :len(cls) * P], dt)
                pages = np.stack([X[p * P:(p + 1) * P] for p in fact])
                out[(b, h, kind)] = (fact, *oracle.svd_batch(pages))
    return out


def oracle_heads(cfg, d, TT, store, pairs, svds):
    """The oracle's outputs (len(pairs), G, d) for the query heads of the
    given (sequence, KV head) pairs at length TT: the stored tokens with
    every FACT page replaced by its rank-r truncated SVD in the cache's
    storage (Sec. 3.2 Eq. 1 over the reconstructed cache)."""
    dt, G, P = cfg["dtype"], cfg["Hq"] // cfg["Hkv"], cfg["P"]
    out = []
    for b, h in pairs:
        rec = {}
        for kind, src, r in (("K", d["K"], cfg["r_k"]), ("V", d["V"], cfg["r_v"])):
            X = synth.storage_to_f64(src[b, h, :TT], dt)
            fact, U, S, Wt = svds[(b, h, kind)]
            Lf, Rf = oracle.stored_factors(U, S, Wt, r, store, kind)
            Xh = Lf @ Rf
            for i, p in enumerate(fact):
                X[p * P:(p + 1) * P] = Xh[i]
            rec[kind] = X
        q64 = synth.storage_to_f64(d["q"][b, h * G:(h + 1) * G], dt)
        out.append(oracle.attention(q64, rec["K"], rec["V"]))
    return np.stack(out)


def decode_full(cfg_id, store=None, overrides=None):
    """One decode and one decode step of workload cfg_id at full size, every
    (sequence, KV head) checked; `overrides` replaces cache parameters (page
    length, ranks, sink, window) over the same tokens."""
    import torch
    require_gpu()
    cfg = dict(synth.CONFIGS[cfg_id])
    cfg.update(overrides or {})
    T, P, dt, G = cfg["T"], cfg["P"], cfg["dtype"], cfg["Hq"] // cfg["Hkv"]
    st = store or dt
    print(f"[full size workload {cfg_id} {st} P={P}] generating", flush=True)
    d = workload_tokens(cfg_id, T + 1)
    cache = make_full_cache(cfg, T + 1, store)
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    cache.prefill(Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
    qd = to_dev(d["q"], dt)
    o1 = to_f64(cache.decode(qd))  # pkv_decode_attn, default split count
    # the bench's path: one pkv_decode_step appending token T
    o2 = to_f64(cache.step(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous(), qd))
    torch.cuda.synchronize()
    del Kd, Vd
    pairs = [(b, h) for b in range(cfg["B"]) for h in range(cfg["Hkv"])]
    # lengths T and T + 1 (T a multiple of P) have the same factorized pages
    c0, c1 = oracle.classify(T, P, cfg["s"], cfg["w"])[0], oracle.classify(T + 1, P, cfg["s"], cfg["w"])[0]
    assert np.array_equal(np.nonzero(c0 == oracle.FACT)[0], np.nonzero(c1 == oracle.FACT)[0])
    key = dict(cfg, cfg_id=cfg_id, T_gen=T + 1)
    svds = oracle_svds(tuple(sorted((k, v) for k, v in key.items() if not isinstance(v, tuple))), T + 1)
    for TT, o in ((T, o1), (T + 1, o2)):
        ref = oracle_heads(cfg, d, TT, st, pairs, svds)
        got = np.stack([o[b, h * G:(h + 1) * G] for b, h in pairs])
        err = rel_err(got, ref)
        worst = max(pairs, key=lambda bh: np.abs(got[pairs.index(bh)] - ref[pairs.index(bh)]).max())
        print(f"[full size workload {cfg_id} {st} P={P}] T={TT}: max err / max|o_ref| = {err:.3e} "
              f"over {len(pairs)} (sequence, KV head) pairs x {G} query heads, each from its own "
              f"tokens (largest at {worst})", flush=True)
        assert err <= TOL[st], (cfg_id, TT, err, worst)
    cls, slot = cache.page_table(-(-(T + 1) // P))
    ocls, oslot = oracle.classify(T + 1, P, cfg["s"], cfg["w"])
    np.testing.assert_array_equal(cls, ocls)
    np.testing.assert_array_equal(slot, oslot)


def test_qwen3_32b_layer_128k_full():
    decode_full(3)


def test_qwen3_32b_layer_128k_int4_full():
    # INT4 factor pages (Sec. 4.3), the bench's qwen3-32b-layer-128k-int4
    decode_full(3, store="int4")


def test_llama31_8b_layer_32k_full():
    decode_full(2)


def test_llama31_8b_layer_32k_p32_full():
    # the bench's llama3.1-8b-layer-p32: 32-token pages at (16, 14), sink 32,
    # window 32 (Sec. 4.1's operating point) on the matrix-core kernel
    decode_full(2, overrides=dict(P=32, r_k=16, r_v=14, s=32, w=32))


def test_llama31_8b_layer_32k_p32_int4_full():
    # the bench's llama3.1-8b-layer-p32-int4: INT4 factor pages of 32 tokens
    decode_full(2, store="int4", overrides=dict(P=32, r_k=16, r_v=14, s=32, w=32))


def test_incremental_512_steps_full():
    import torch
    require_gpu()
    cfg_id = 4
    cfg = synth.CONFIGS[cfg_id]
    T0, steps, P, dt = cfg["T"], cfg["steps"], cfg["P"], cfg["dtype"]
    B, Hq, Hkv = cfg["B"], cfg["Hq"], cfg["Hkv"]
    G = Hq // Hkv
    print("[full size workload 4] generating", flush=True)
    d = synth.decode_inputs(cfg_id, T=T0 + steps, workers=WORKERS)
    cache = make_full_cache(cfg, T0 + steps)
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    cache.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    ws = cache.workspace(512)
    # three pairs at every step: one decoder over them as the KV heads of one
    # sequence (their query heads gathered to match)
    few = [(0, 0), (3, 5), (B - 1, Hkv - 1)]
    K_few = synth.storage_to_f64(np.stack([d["K"][b, h] for b, h in few])[None], dt)
    V_few = synth.storage_to_f64(np.stack([d["V"][b, h] for b, h in few])[None], dt)
    inc_few = oracle.IncrementalDecoder(K_few, V_few, P, cfg["s"], cfg["w"], cfg["r_k"], cfg["r_v"], dt)
    inc_all = oracle.IncrementalDecoder(synth.storage_to_f64(d["K"], dt), synth.storage_to_f64(d["V"], dt),
                                        P, cfg["s"], cfg["w"], cfg["r_k"], cfg["r_v"], dt)
    promos, worst_few, worst_all, n_all = [], 0.0, 0.0, 0
    for t in range(steps):
        T = T0 + t
        nf_before = cache.state()[1]
        qs = synth.step_queries(cfg_id, t, B, Hq, 128, dt)
        o = cache.step(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous(), to_dev(qs, dt), workspace=ws)
        promoted = cache.state()[1] > nf_before
        if promoted:
            promos.append(t + 1)
        cls, slot = cache.page_table(-(-(T + 1) // P))
        ocls, oslot = oracle.classify(T + 1, P, cfg["s"], cfg["w"])
        np.testing.assert_array_equal(cls, ocls, err_msg=f"step {t}")
        np.testing.assert_array_equal(slot, oslot, err_msg=f"step {t}")
        torch.cuda.synchronize()
        og = to_f64(o)
        q64 = synth.storage_to_f64(qs, dt)
        qf = np.concatenate([q64[b, h * G:(h + 1) * G] for b, h in few])[None]
        ref = inc_few.step(qf, T + 1)[0][0].reshape(len(few), G, 128)
        got = np.stack([og[b, h * G:(h + 1) * G] for b, h in few])
        err = rel_err(got, ref)
        worst_few = max(worst_few, err)
        assert err <= TOL[dt], (t, few, err)
        if promoted or t == steps - 1:
            ref_all = inc_all.step(q64, T + 1)[0]
            err = rel_err(og, ref_all)
            worst_all = max(worst_all, err)
            n_all += 1
            assert err <= TOL[dt], (t, "all pairs", err)
    print(f"[full size workload 4] {steps} steps from T={T0}: promotions at {promos}; pairs {few} "
          f"checked at all {steps} steps (worst {worst_few:.3e}), all {B * Hkv} pairs at {n_all} "
          f"steps (worst {worst_all:.3e}); page table at every step", flush=True)
    assert promos == [64 * k for k in range(1, steps // 64 + 1)]


def test_batched_compression_full():
    import torch
    require_gpu()
    cfg = synth.CONFIGS[5]
    n_total = cfg["layers"] * cfg["Hkv"] * 2 * cfg["pages_per_head"]
    import time
    print(f"[full size workload 5] drawing {n_total} distinct pages on the device", flush=True)
    t0 = time.time()
    bits = synth.compression_pool_device(n_total, device="cuda:0")
    torch.cuda.synchronize()
    print(f"[full size workload 5] drawn in {time.time() - t0:.1f} s", flush=True)
    X = bits.view(torch.bfloat16)
    assert X.shape[0] == n_total
    g = np.random.default_rng(5)
    noise = synth.noise_page_ids(5, n_total, 0.02)
    spec = np.setdiff1d(np.arange(n_total), noise)
    ids = np.sort(np.concatenate([noise, g.choice(spec, n_total // 100, replace=False)]))
    at = torch.from_numpy(ids).to("cuda:0")
    X64 = synth.storage_to_f64(bits[at].cpu().numpy().view(np.uint16), "bf16")
    U, S, Wt = oracle.svd_batch(X64)
    nrm = np.sqrt((X64 ** 2).sum(axis=(1, 2)))
    is_noise = np.isin(ids, noise)
    for r in cfg["ranks"]:
        Lf, Rf, _ = pkv.compress_pages(X, r, out_dtype=torch.bfloat16, with_sigma=False)
        torch.cuda.synchronize()
        L64, R64 = to_f64(Lf[at]), to_f64(Rf[at])
        err = np.sqrt(((X64 - L64 @ R64) ** 2).sum(axis=(1, 2)))
        opt = oracle.optimal_error(S, r)
        bound = np.sqrt((1.001 * opt + 1e-5 * nrm) ** 2 + (2.0 ** -8 * nrm) ** 2)
        ratio = err / bound
        print(f"[full size workload 5] r={r}: {n_total} distinct pages in one launch; all "
              f"{noise.size} noise pages (worst err/bound {ratio[is_noise].max():.4f}) and "
              f"{(~is_noise).sum()} sampled spectrum pages (worst {ratio[~is_noise].max():.4f})",
              flush=True)
        assert np.all(err <= bound), (r, float(ratio.max()))
        del Lf, Rf
