"""GPU parity of the INT4 factor pages (PuzzleKV Sec. 4.3) against the oracle.

- Page decomposition into INT4 parts (prefill, promotion): each part is
  unpacked on the host and compared with the oracle's codes and scales of the
  same page (oracle.int4_codes on its float64 SVD).  The decomposition is
  unique up to the sign of each singular pair (the cfg-3 recipe has distinct
  singular values), so after aligning signs every GPU scale must lie within
  one bfloat16 step (2^-7 relative) of the oracle's, every GPU code c must
  round the oracle's exact factor x at the GPU's scale s to within the
  float32 eigen-solve's error, |c - x / s| <= 0.55 (a rounding error of 0.5
  plus 5% of a quantization step; trailing ranks of the Gram route are
  accurate to ~1e-3 relative), and at least 99% of the codes must equal the
  oracle's.
- Attention on INT4 parts that hold the oracle's own codes (packed on the host
  and written into the factor pool): the kernel's arithmetic alone, against
  the oracle's attention over the same dequantized factors; gate
  max |o - o_ref| <= 1e-3 max |o_ref| (the kernel carries fp32 operands as
  bf16 hi/lo pairs, ~2^-16 relative, and a code as 1.5 + c/16 whose offset
  cancels in fp32).
- End to end (GPU codes, oracle codes): the bf16 gate 1e-2 max |o_ref|.
- pkv_decode_step on an INT4 cache: bit-identical to the separate calls and
  to early factorization, and within the gate of the oracle at every step.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu

KIND = {pkv.KEYS: "K", pkv.VALUES: "V"}


def _prefilled(cfg_id, T, B, kv_heads, r_k=None, r_v=None, s=None, w=None, max_tokens=None, P=64):
    d = synth.decode_inputs(cfg_id, T=T, B=B, kv_heads=kv_heads, with_f64=True)
    cache = make_cache(d, r_k=r_k, r_v=r_v, s=s, w=w, max_tokens=max_tokens, store="int4", P=P)
    cache.prefill(to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16"))
    return d, cache


def _fact_pages(d, cache, b, h, kind):
    """float64 pages (n_fact, P, 128) of the factorized region of (b, h)."""
    T, nf, _ = cache.state()
    P = cache.shape.page_len
    n_s = cache.shape.sink // P
    src = d["K64"] if kind == pkv.KEYS else d["V64"]
    return src[b, h, P * n_s: P * (n_s + nf)].reshape(nf, P, 128)


def _gpu_codes(cache, b, h, slot, kind, r):
    import torch
    part = cache.factor_part(b, h, slot, kind).cpu().numpy()
    torch.cuda.synchronize()
    return pkv.unpack_factors_int4(kind, r, part, P=cache.shape.page_len)


def _compare_codes(gq, gs, oq, os_, x, label):
    """gq, oq codes; gs, os_ their scales (group axis kept, broadcastable);
    x the oracle's unquantized factor.  Returns the number of equal codes."""
    gs = np.broadcast_to(gs, os_.shape).astype(np.float64)
    assert np.all(np.abs(gs - os_) <= 2.0 ** -7 * np.maximum(gs, os_)), f"{label}: scales"
    sb = np.broadcast_to(gs, x.shape)
    dev = np.where(sb > 0, np.abs(gq - x / np.where(sb > 0, sb, 1.0)), np.abs(x) * 1e12)
    assert dev.max() <= 0.55, f"{label}: code off by {dev.max():.3f} steps"
    return int((gq == oq).sum())


@pytest.mark.parametrize("cfg_id,r,P", [(3, 24, 64), (3, 16, 64), (3, 8, 64), (3, 32, 64), (3, 20, 64),
                                        (3, 16, 32), (3, 24, 32)])
def test_int4_decomposition_codes_match_oracle(cfg_id, r, P):
    """Prefill factorizes every FACT page straight into INT4 parts (cfg-3
    key/value recipe: sigma_i = i^-1.2, distinct singular values); also for
    32-token pages."""
    require_gpu()
    d, cache = _prefilled(cfg_id, 64 * 24, B=1, kv_heads=2, r_k=r, r_v=r, P=P)
    equal = total = 0
    for b in range(d["B"]):
        for h in range(d["Hkv"]):
            for kind in (pkv.KEYS, pkv.VALUES):
                X = _fact_pages(d, cache, b, h, kind)
                U, S, Wt = oracle.svd_batch(X)
                Lt, Rt, lq, ls, rq, rs = oracle.int4_codes(U, S, Wt, r, KIND[kind])
                for f in range(X.shape[0]):
                    gl, gls, gr, grs = _gpu_codes(cache, b, h, f, kind, r)
                    # sign of each singular pair from the codes' agreement
                    sgn = np.sign(np.sum(gl.astype(np.float64) * lq[f], axis=0))
                    sgn[sgn == 0] = 1
                    gl = (gl * sgn[None, :]).astype(np.int8)
                    gr = (gr * sgn[:, None]).astype(np.int8)
                    lab = f"{KIND[kind]} b{b} h{h} page {f}"
                    gls = gls[None, :] if kind == pkv.KEYS else gls[:, None]
                    equal += _compare_codes(gl, gls, lq[f], ls[f], Lt[f], lab + " Lt")
                    equal += _compare_codes(gr, grs[None, :], rq[f], rs[f], Rt[f], lab + " Rt")
                    total += gl.size + gr.size
    print(f"[int4 codes r={r} P={P}] {equal}/{total} codes equal to the oracle's, all within the bound")
    assert equal >= 0.99 * total


@pytest.mark.parametrize("r,P", [(24, 64), (8, 64), (20, 64), (32, 64), (16, 32), (20, 32), (24, 32)])
def test_int4_parts_are_canonical(r, P):
    """Every byte of a GPU-written part, padding included, is what the host
    packer writes for the part's own codes and scales: pack(unpack(part))
    reproduces it exactly, so a part depends on the page alone."""
    require_gpu()
    d, cache = _prefilled(3, 64 * 8, B=1, kv_heads=2, r_k=r, r_v=r, P=P)
    for h in range(2):
        for f in range(cache.state()[1]):
            for kind in (pkv.KEYS, pkv.VALUES):
                part = cache.factor_part(0, h, f, kind).cpu().numpy()
                again = pkv.pack_factors_int4(kind, r, *pkv.unpack_factors_int4(kind, r, part, P=P), P=P)
                np.testing.assert_array_equal(part, again, err_msg=f"h{h} page {f} kind {kind}")


def _oracle_parts(d, cache, r_k, r_v):
    """Write the oracle's INT4 codes of every FACT page into the pool."""
    import torch
    for b in range(d["B"]):
        for h in range(d["Hkv"]):
            for kind, r in ((pkv.KEYS, r_k), (pkv.VALUES, r_v)):
                X = _fact_pages(d, cache, b, h, kind)
                U, S, Wt = oracle.svd_batch(X)
                _, _, lq, ls, rq, rs = oracle.int4_codes(U, S, Wt, r, KIND[kind])
                for f in range(X.shape[0]):
                    lsf = ls[f, 0] if kind == pkv.KEYS else ls[f, :, 0]
                    part = pkv.pack_factors_int4(kind, r, lq[f], lsf, rq[f], rs[f, 0], P=cache.shape.page_len)
                    cache.factor_part(b, h, f, kind).copy_(torch.from_numpy(part))
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg_id,T,B,kv,rk,rv,splits,P", [
    (3, 64 * 48 + 5, 1, 2, 24, 24, (0, 3), 64),
    (2, 64 * 40 + 37, 2, 2, 16, 16, (0, 1, 64), 64),
    (2, 64 * 20 + 1, 1, 2, 16, 14, (0,), 64),
    (2, 64 * 20 + 1, 1, 2, 24, 16, (0,), 64),
    (2, 64 * 20 + 63, 1, 2, 8, 8, (0,), 64),
    (2, 64 * 20, 1, 2, 32, 32, (0,), 64),
    (2, 64 * 20 + 9, 1, 2, 20, 12, (0,), 64),
    (3, 32 * 60 + 5, 1, 2, 24, 24, (0, 3), 32),   # 32-token pages: 3-byte rank units
    (2, 32 * 40 + 9, 2, 2, 16, 14, (0, 2), 32),   # 2-byte units
    (2, 32 * 30 + 3, 1, 2, 8, 8, (0, 2), 32),     # 1-byte units
    (2, 32 * 24 + 30, 1, 2, 32, 32, (0, 5), 32),  # 4-byte units (full rank)
    (2, 32 * 30 + 7, 1, 2, 8, 24, (0, 2), 32),    # unequal padded ranks: 1- and 3-byte units
    (3, 32 * 28 + 19, 1, 2, 32, 13, (0, 3), 32),  # 4- and 2-byte units
    (2, 32 * 26 + 5, 2, 2, 24, 8, (0,), 32),
])
def test_int4_attention_on_oracle_codes(cfg_id, T, B, kv, rk, rv, splits, P):
    require_gpu()
    d, cache = _prefilled(cfg_id, T, B, kv, r_k=rk, r_v=rv, P=P)
    _oracle_parts(d, cache, rk, rv)
    cfg = d["cfg"]
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, P, cfg["s"], cfg["w"], rk, rv, "int4")
    q = to_dev(d["q"], "bf16")
    for ns in splits:
        o = to_f64(cache.decode(q, n_split=ns))
        err = rel_err(o, ref["o_stored"])
        print(f"[int4 oracle codes cfg{cfg_id} T={T} P={P} r=({rk},{rv}) split={ns}] err={err:.3e} "
              f"(vs unquantized: {rel_err(o, ref['o_exact']):.3e})")
        assert err <= 1e-3, (ns, err)


@pytest.mark.parametrize("cfg_id,T,B,kv,rk,rv,P", [
    (3, 64 * 48 + 5, 1, 2, 24, 24, 64),
    (2, 64 * 40 + 37, 2, 2, 16, 16, 64),
    (2, 64 * 30 + 17, 1, 2, 16, 14, 64),
    (2, 32 * 60 + 17, 1, 2, 16, 14, 32),  # the pages' operating point (sink 64, window 128)
    (3, 32 * 44 + 11, 1, 2, 8, 24, 32),   # 32-token pages, unequal padded ranks
])
def test_int4_decode_end_to_end(cfg_id, T, B, kv, rk, rv, P):
    require_gpu()
    d, cache = _prefilled(cfg_id, T, B, kv, r_k=rk, r_v=rv, P=P)
    cfg = d["cfg"]
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, P, cfg["s"], cfg["w"], rk, rv, "int4")
    o = to_f64(cache.decode(to_dev(d["q"], "bf16")))
    err = rel_err(o, ref["o_stored"])
    print(f"[int4 end to end cfg{cfg_id} T={T} P={P} r=({rk},{rv})] err={err:.3e} "
          f"(vs unquantized: {rel_err(o, ref['o_exact']):.3e})")
    assert err <= TOL["int4"]
    cls, slot = cache.page_table(-(-T // P))
    ocls, oslot = oracle.classify(T, P, cfg["s"], cfg["w"])
    np.testing.assert_array_equal(cls, ocls)
    np.testing.assert_array_equal(slot, oslot)


def _twins(cfg_id, T0, steps, B, kv, **kw):
    import torch
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=B, kv_heads=kv)
    a = make_cache(d, max_tokens=T0 + steps, store="int4", **kw)
    b = make_cache(d, max_tokens=T0 + steps, store="int4", **kw)
    a.buffer.zero_()
    b.buffer.zero_()
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    for c in (a, b):
        c.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    torch.cuda.synchronize()
    return d, a, b, Kd, Vd


def test_int4_step_matches_separate_calls():
    import torch
    require_gpu()
    T0, steps = 64 * 12 + 40, 100
    d, a, b, Kd, Vd = _twins(2, T0, steps, B=2, kv=2)
    promos = 0
    for t in range(steps):
        T = T0 + t
        k, v = Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous()
        q = to_dev(synth.step_queries(2, t, d["B"], d["Hq"], 128, "bf16"), "bf16")
        oa = a.step(k, v, q)
        if b.append(k, v):
            b.promote()
            promos += 1
        ob = b.decode(q)
        torch.cuda.synchronize()
        assert a.state() == b.state()
        assert rel_err(to_f64(oa), to_f64(ob)) <= 1e-5, t
    assert torch.equal(a.buffer, b.buffer)
    print(f"[int4 step vs separate] {steps} steps, {promos} promotions: caches bit-identical")
    assert promos == 2


@pytest.mark.parametrize("P", [64, 32])
def test_int4_step_against_oracle(P):
    """Incremental decode on INT4 pages against the oracle at every step.
    The cfg-3 recipe (distinct singular values) makes the codes of each
    promoted page unique up to rounding ties; on the cfg-2/4 recipe (rank 8
    plus noise) ranks above 8 span a near-degenerate noise subspace, where
    two correct decompositions quantize to different codes (see
    test_int4_decomposition_valid_on_degenerate_spectra)."""
    import torch
    require_gpu()
    cfg_id, T0, steps = 3, 64 * 10 + 3, 140
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=1, kv_heads=2, with_f64=True)
    cfg = d["cfg"]
    cache = make_cache(d, max_tokens=T0 + steps, store="int4", P=P)
    Kd, Vd = to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16")
    cache.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    inc = oracle.IncrementalDecoder(d["K64"], d["V64"], P, cfg["s"], cfg["w"], cfg["r_k"], cfg["r_v"],
                                    "int4")
    worst, promos = 0.0, 0
    for t in range(steps):
        T = T0 + t
        nf = cache.state()[1]
        qs = synth.step_queries(cfg_id, t, d["B"], d["Hq"], 128, "bf16")
        o = to_f64(cache.step(Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous(), to_dev(qs, "bf16")))
        promos += cache.state()[1] > nf
        torch.cuda.synchronize()
        ref, _ = inc.step(synth.storage_to_f64(qs, "bf16"), T + 1)
        err = rel_err(o, ref)
        worst = max(worst, err)
        assert err <= TOL["int4"], (t, err)
    print(f"[int4 step vs oracle P={P}] {steps} steps, {promos} promotions, worst err {worst:.3e}")
    assert promos == (T0 + steps) // P - T0 // P


def test_int4_decomposition_valid_on_degenerate_spectra():
    """cfg-2 recipe (rank-8 pages plus noise): the kept ranks above 8 are not
    unique, so the codes are checked for validity instead of equality.  With
    the GPU's codes c and scales s, each factor's dequantization error is at
    most s/2 per element, so ||X - Lq Rq||_F <= E_r + dL ||Rq||_2 +
    ||Lq||_2 dR + dL dR, with E_r the oracle's optimal rank-r error (times the
    decomposition tolerance 1.001, + 1e-5 ||X||_F) and dL, dR the Frobenius
    bounds sqrt(sum over groups of n_g s_g^2 / 4)."""
    require_gpu()
    r = 16
    d, cache = _prefilled(2, 64 * 20, B=1, kv_heads=2, r_k=r, r_v=r)
    worst = 0.0
    for h in range(d["Hkv"]):
        for kind in (pkv.KEYS, pkv.VALUES):
            X = _fact_pages(d, cache, 0, h, kind)
            _, S, _ = oracle.svd_batch(X)
            for f in range(X.shape[0]):
                gl, gls, gr, grs = _gpu_codes(cache, 0, h, f, kind, r)
                Ls = gls[None, :] if kind == pkv.KEYS else gls[:, None]
                Lq = gl.astype(np.float64) * Ls
                Rq = gr.astype(np.float64) * grs[None, :]
                dL = 0.5 * np.sqrt(np.sum(np.broadcast_to(Ls, Lq.shape).astype(np.float64) ** 2))
                dR = 0.5 * np.sqrt(np.sum(np.broadcast_to(grs[None, :], Rq.shape).astype(np.float64) ** 2))
                opt = 1.001 * oracle.optimal_error(S[f], r) + 1e-5 * np.linalg.norm(X[f])
                bound = opt + dL * np.linalg.norm(Rq, 2) + np.linalg.norm(Lq, 2) * dR + dL * dR
                err = np.linalg.norm(X[f] - Lq @ Rq)
                worst = max(worst, err / bound)
                assert err <= bound, (h, kind, f, err, bound)
    print(f"[int4 degenerate spectra r={r}] worst error / bound {worst:.3f}")


def test_int4_step_with_early_factorization():
    import torch
    require_gpu()
    T0, steps = 64 * 12 + 40, 200
    d, a, b, Kd, Vd = _twins(2, T0, steps, B=1, kv=2)
    aux = torch.cuda.Stream()
    a.set_aux_stream(aux)
    for t in range(steps):
        T = T0 + t
        k, v = Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous()
        q = to_dev(synth.step_queries(2, t, d["B"], d["Hq"], 128, "bf16"), "bf16")
        oa = a.step(k, v, q)
        ob = b.step(k, v, q)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), t
    aux.synchronize()
    assert torch.equal(a.buffer, b.buffer)
