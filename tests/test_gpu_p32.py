"""GPU parity of caches with 32-token pages against the oracle at P = 32
(PuzzleKV Sec. 4.1 "Implementation": pages of 32 tokens, (r_K, r_V) =
(16, 14), one 32-token sink page, the most recent completed page and the
page being filled kept dense).

Such caches keep their factor parts in the 64-token matrix-core operand
order with the operand rows of page rows 32..63 left out.  bf16 caches
(any rank pair up to 32, keys post- or pre-RoPE) and INT4 caches (any rank
pair up to 32) are attended by the matrix-core kernel, which reads a
factorized page in a two-tile compact token order and dense pages in the
64-row frame (absent rows zero, their scores masked); fp32 caches by the
vector-ALU kernel.  A 32-row page is
decomposed on the leading 32 x 32 block of its zero-padded 64-row Gram
matrix.  Gates as for 64-token pages: bf16 storage 1e-2, fp32 storage 1e-4,
relative to max |o_ref|; stored factors meet the reconstruction bound of the
standalone decomposition; chunked prefill and batched steps agree bit for
bit with their token-by-token and per-cache twins.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64
from test_gpu_chunk import _chunk_vs_tokens

pytestmark = pytest.mark.gpu

P = 32
RK, RV = 16, 14  # the pages' operating point
S, W = 32, 32    # one sink page, one window page


def _case(cfg_id, T, B=1, kv_heads=2, rk=RK, rv=RV, s=S, w=W, splits=(0,), rope=None, label=""):
    import torch
    require_gpu()
    d = synth.decode_inputs(cfg_id, T=T, B=B, kv_heads=kv_heads, with_f64=True)
    dt = d["cfg"]["dtype"]
    cache = make_cache(d, r_k=rk, r_v=rv, s=s, w=w, P=P)
    if rope is not None:
        cache.set_key_rope(rope)
    cache.prefill(to_dev(d["K"], dt), to_dev(d["V"], dt))
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, P, s, w, rk, rv, dt, key_rope=rope)
    q = to_dev(d["q"], dt)
    for ns in splits:
        o = to_f64(cache.decode(q, n_split=ns))
        torch.cuda.synchronize()
        e_s, e_e = rel_err(o, ref["o_stored"]), rel_err(o, ref["o_exact"])
        print(f"[P=32 {label} cfg{cfg_id} T={T} r=({rk},{rv}) s={s} w={w} split={ns}] "
              f"err_vs_stored={e_s:.3e} err_vs_exact={e_e:.3e}")
        assert e_s <= TOL[dt], (label, ns, e_s)
    return cache, d


@pytest.mark.parametrize("cfg_id,T,B,kv,rk,rv,splits", [
    (2, 32 * 40 + 5, 2, 2, RK, RV, (0, 1, 5)),  # bf16, ragged tail
    (2, 32 * 64, 1, 2, RK, RV, (0, 7)),         # page-aligned T
    (2, 32 * 20 + 31, 1, 1, 32, 32, (0,)),     # full rank of a 32-token page
    (2, 32 * 20 + 1, 1, 2, 1, 3, (0, 2)),      # tiny ranks
    (2, 32 * 20 + 9, 1, 2, 8, 24, (0, 2)),     # unequal padded ranks (compacted K1 and V1 tiles)
    (2, 32 * 33 + 17, 1, 2, 24, 24, (0, 4)),   # odd n8: compacted last rank tile
    (1, 32 * 30 + 17, 1, 1, RK, RV, (0, 3)),   # fp32 storage
    (1, 32 * 12, 1, 1, 32, 32, (0,)),          # fp32, full rank
])
def test_p32_decode_against_oracle(cfg_id, T, B, kv, rk, rv, splits):
    _case(cfg_id, T, B, kv, rk, rv, splits=splits, label="decode")


@pytest.mark.parametrize("T", [32 * 9 + 3, 32 * 10 + 3, 32 * 41 + 30, 32 * 42 + 30])
def test_p32_factorized_counts_and_splits_against_oracle(T):
    """The pages' operating point at odd and even factorized page counts
    (7, 8, 39, 40) and split counts from one workgroup to more waves than
    factorized pages, so that waves hold none, one, or runs of them."""
    _case(2, T, 1, 2, RK, RV, splits=(0, 1, 2, 3, 16, 64), label="counts")


def test_p32_short_and_windowless_caches():
    _case(2, 20, label="sink only")
    _case(2, 32 * 2 + 3, label="all dense")
    _case(2, 32 * 10 + 7, s=0, w=0, splits=(0, 2), label="no sink, no window")
    _case(2, 32 * 10 + 7, s=64, w=96, splits=(0,), label="s=64 w=96")


def test_p32_pre_rope_keys():
    # matrix-core kernel (equal, then unequal padded ranks), then the
    # vector-ALU kernel (fp32 storage)
    _case(2, 32 * 30 + 9, rope=synth.rope_inv_freq(5e5), splits=(0, 2), label="pre-RoPE")
    _case(3, 32 * 40 + 21, rk=24, rv=24, rope=synth.rope_inv_freq(1e6), splits=(0, 3), label="pre-RoPE r=24")
    _case(2, 32 * 12 + 7, rk=8, rv=24, rope=synth.rope_inv_freq(5e5), label="pre-RoPE r=(8,24)")
    _case(1, 32 * 12 + 7, rk=8, rv=24, rope=synth.rope_inv_freq(1e4), splits=(0, 2), label="pre-RoPE fp32 valu")


@pytest.mark.parametrize("cfg_id,T,rk,rv,splits", [
    (2, 32 * 25 + 3, 8, 8, (0, 3)),     # n8 = 1: compacted rank tile
    (4, 32 * 18 + 30, 5, 7, (0, 1)),    # n8 = 1, unequal ranks
    (3, 32 * 27 + 16, 20, 24, (0, 5)),  # n8 = 3
    (2, 32 * 22 + 1, 32, 32, (0, 2)),   # n8 = 4: full rank of a 32-token page
    (2, 32 * 20 + 9, 8, 24, (0, 2)),    # unequal padded ranks: key n8 = 1, value n8 = 3
    (3, 32 * 23 + 5, 32, 13, (0, 3)),   # key n8 = 4, value n8 = 2 (exact-rank part, r2 = 14)
    (4, 32 * 19 + 17, 24, 30, (0,)),    # key n8 = 3, value n8 = 4
    (2, 32 * 21 + 2, 16, 1, (0,)),      # value rank 1
])
def test_p32_pre_rope_every_rank_tile_count(cfg_id, T, rk, rv, splits):
    """Pre-RoPE 32-token pages on the matrix-core kernel at every padded rank
    it takes (8 to 32, key and value ranks equal or not), against the
    oracle."""
    f = synth.rope_inv_freq(5e5 if cfg_id != 3 else 1e6)
    _case(cfg_id, T, rk=rk, rv=rv, rope=f, splits=splits, label="pre-RoPE n8")


def test_p32_factors_are_the_pages_own():
    """The packed parts (compacted matrix-core order) of a 32-token page hold
    its rank-r decomposition: unpacked at P = 32 their product meets the bf16
    reconstruction bound against the oracle's optimal error."""
    import torch
    cache, d = _case(2, 32 * 12 + 4, label="factors")
    T, nf, _ = cache.state()
    assert nf == 12 - 1 - 1
    for kind, r, src in ((pkv.KEYS, RK, d["K64"]), (pkv.VALUES, RV, d["V64"])):
        for h in range(2):
            X = src[0, h, P:P * (1 + nf)].reshape(nf, P, 128)
            U, S_, Wt = oracle.svd_batch(X)
            opt = oracle.optimal_error(S_, r)
            for f in range(nf):
                part = cache.factor_part(0, h, f, kind).cpu().numpy()
                torch.cuda.synchronize()
                assert part.size == pkv.factor_part_bytes(kind, r, pkv.BF16, P=P)
                Lf, Rf = pkv.unpack_factors(kind, r, pkv.BF16, part.view(np.uint16), P=P)
                err = np.linalg.norm(X[f] - Lf.astype(np.float64) @ Rf.astype(np.float64))
                nrm = np.linalg.norm(X[f])
                bound = np.hypot(1.001 * opt[f] + 1e-5 * nrm, 2.0 ** -8 * nrm)
                assert err <= bound, (kind, h, f, err, opt[f], bound)


@pytest.mark.parametrize("r,out,pages", [
    (16, "f32", "kv"), (14, "bf16", "kv"), (8, "f32", "kv"), (1, "f32", "kv"), (32, "f32", "kv"),
    (32, "f32", "gauss"),
])
def test_p32_standalone_decomposition(r, out, pages):
    """pkv_compress_pages on (n, 32, 128) pages against the oracle's SVD:
    ||X - Lf Rf|| <= 1.001 opt + 1e-5 ||X|| (bf16 output: plus the 2^-8 ||X||
    storage floor), sigma within 2e-3 relative where the spectrum is
    resolved.  Full rank (r = P) on the synthetic key / value pages, whose
    trailing singular values crowd into 1-2% of sigma_1, holds the literal
    bound only because the kept columns are orthonormalized after the
    eigen-solve."""
    import torch
    require_gpu()
    if pages == "kv":
        cfg = synth.CONFIGS[2]
        k, v = synth.kv_head(cfg, 0, 0, 64 * P)
        X0 = np.concatenate([k, v]).reshape(-1, P, 128)
    else:
        X0 = np.random.default_rng(32).standard_normal((16, P, 128))
    dt = "bf16" if pages == "kv" else "f32"
    Xs = synth.to_storage(X0, dt)
    X = to_dev(Xs, dt)
    tdt = torch.bfloat16 if out == "bf16" else torch.float32
    Lf, Rf, sig = pkv.compress_pages(X, r, out_dtype=tdt)
    torch.cuda.synchronize()
    assert tuple(Lf.shape) == (Xs.shape[0], P, r)
    X64 = synth.storage_to_f64(Xs, dt)
    err = np.sqrt(((X64 - to_f64(Lf) @ to_f64(Rf)) ** 2).sum(axis=(1, 2)))
    U, S_, Wt = oracle.svd_batch(X64)
    opt = oracle.optimal_error(S_, r)
    nrm = np.sqrt((X64 ** 2).sum(axis=(1, 2)))
    bound = 1.001 * opt + 1e-5 * nrm
    if out == "bf16":
        bound = np.sqrt(bound ** 2 + (2.0 ** -8 * nrm) ** 2)
    print(f"[P=32 compress {pages} r={r} out={out}] worst err/bound = "
          f"{np.max(err / np.maximum(bound, 1e-300)):.4f}")
    assert np.all(err <= bound)
    dev = np.abs(sig.cpu().numpy().astype(np.float64) - S_[:, :r]) - (2e-3 * S_[:, :r] + 1e-5 * S_[:, :1])
    assert np.all(dev <= 0), float(dev.max())


@pytest.mark.parametrize("rope,w", [(False, W), (True, W), (False, 0)])
def test_p32_decode_steps_against_oracle(rope, w):
    """pkv_decode_step over 100 tokens from a ragged start: a page completes
    every 32 steps and the page leaving the window is factorized in the same
    call; every step's output against the oracle's incremental decoder (with
    pre-RoPE keys the new key turns at its position in the merge)."""
    import torch
    require_gpu()
    cfg_id, T0, steps = 4, 32 * 10 + 3, 100
    d = synth.decode_inputs(cfg_id, T=T0 + steps, B=2, kv_heads=2, with_f64=True)
    dt = d["cfg"]["dtype"]
    f = synth.rope_inv_freq(5e5) if rope else None
    cache = make_cache(d, r_k=RK, r_v=RV, s=S, w=w, P=P, max_tokens=T0 + steps)
    if rope:
        cache.set_key_rope(f)
    Kd, Vd = to_dev(d["K"], dt), to_dev(d["V"], dt)
    cache.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    inc = oracle.IncrementalDecoder(d["K64"], d["V64"], P, S, w, RK, RV, dt, key_rope=f)
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
    assert cache.state()[1] == (T0 + steps) // P - S // P - w // P
    print(f"[P=32 step vs oracle w={w}] {steps} steps, worst err {worst:.3e}")


def test_p32_chunks_match_token_by_token():
    _chunk_vs_tokens(2, 32 * 5 + 17, [40, 7, 32, 300, ("step", 45), 1, 513], P=P, r_k=RK, r_v=RV, s=S, w=W)


def test_p32_chunks_int4_pages():
    # INT4 factor pages (Sec. 4.3) of 32 tokens at (16, 14)
    _chunk_vs_tokens(3, 32 * 3 + 9, [100, 33, ("step", 40), 600, ("tok", 33), 5], store="int4", P=P, r_k=RK,
                     r_v=RV, s=S, w=W)


def test_p32_chunks_on_aux_stream():
    _chunk_vs_tokens(2, 32 * 3 + 5, [40, 600, ("tok", 70), 1, 333], B=2, aux=True, P=P, r_k=RK, r_v=RV,
                     s=S, w=W)


@pytest.mark.parametrize("lengths,rope,store,rk,rv", [
    ([32 * 20 + 5, 7, 32 * 3, 32 * 9 + 31], False, None, RK, RV),    # pages complete at different steps
    ([32 * 20 + 9, 32 * 5 + 9, 32 * 11 + 9], False, None, RK, RV),   # ... at the same steps: one promotion launch
    ([32 * 20 + 5, 7, 32 * 3, 32 * 9 + 31], True, None, RK, RV),     # pre-RoPE keys
    ([32 * 20 + 9, 32 * 5 + 9, 32 * 11 + 9], False, "int4", RK, RV),  # INT4 factor pages
    ([32 * 20 + 5, 32 * 3, 32 * 9 + 31], True, None, 8, 24),         # unequal padded ranks: one launch per cache
    ([32 * 20 + 9, 32 * 5 + 9, 32 * 11 + 9], False, "int4", 24, 8),
])
def test_p32_batches_equal_single_caches(lengths, rope, store, rk, rv):
    """Batched attention and batched steps over 32-token caches of different
    lengths equal the per-cache calls bit for bit."""
    import torch
    require_gpu()
    steps, ns = 40, 3
    A, Bs, seqs = [], [], []
    for i, T in enumerate(lengths):
        d = synth.decode_inputs(2, T=T + steps + 32 * i, B=1, kv_heads=2)
        Kd = to_dev(np.ascontiguousarray(d["K"][:, :, 32 * i:]), "bf16")
        Vd = to_dev(np.ascontiguousarray(d["V"][:, :, 32 * i:]), "bf16")
        for group in (A, Bs):
            c = make_cache(d, r_k=rk, r_v=rv, s=S, w=W, P=P, max_tokens=T + steps, store=store)
            if rope:
                c.set_key_rope(synth.rope_inv_freq(5e5))
            c.prefill(Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
            group.append(c)
        seqs.append((Kd, Vd, T))
    Hq = d["Hq"]
    q0 = to_dev(synth.step_queries(2, 999, len(lengths), Hq, 128, "bf16"), "bf16")
    out = pkv.decode_batch(A, q0, n_split=ns)
    for i, c in enumerate(Bs):
        assert torch.equal(out[i:i + 1], c.decode(q0[i:i + 1].contiguous(), n_split=ns)), i
    ws = pkv.batch_workspace(A, ns)
    for t in range(steps):
        k = torch.stack([Kd[0, :, T + t] for Kd, _, T in seqs]).contiguous()
        v = torch.stack([Vd[0, :, T + t] for _, Vd, T in seqs]).contiguous()
        q = to_dev(synth.step_queries(2, t, len(lengths), Hq, 128, "bf16"), "bf16")
        oa = pkv.step_batch(A, k, v, q, n_split=ns, workspace=ws)
        for i, c in enumerate(Bs):
            ob = c.step(k[i:i + 1].contiguous(), v[i:i + 1].contiguous(), q[i:i + 1].contiguous(), n_split=ns)
            torch.cuda.synchronize()
            assert torch.equal(oa[i:i + 1], ob), (t, i)
    for a, b in zip(A, Bs):
        assert a.state() == b.state()


def test_p32_errors():
    require_gpu()
    d = synth.decode_inputs(2, T=200, B=1, kv_heads=1)
    with pytest.raises(pkv.PKVError) as ei:  # rank above the page length
        make_cache(d, r_k=33, r_v=RV, s=S, w=W, P=P)
    assert ei.value.status == 1


def test_p32_random_shapes_against_oracle():
    """Seeded random 32-token caches: workload recipes with GQA groups 1, 4
    and 8, ranks 1..32 (K and V drawn apart, so both kernels run), sink and
    window of 0..3 pages, ragged lengths, batch and KV heads 1..2, default
    and explicit split counts -- each against the oracle."""
    import torch
    require_gpu()
    g = np.random.default_rng(3232)
    for case in range(14):
        cfg_id = int(g.choice([1, 2, 3, 4]))
        rk = int(g.integers(1, 33))
        rv = rk if g.random() < 0.5 else int(g.integers(1, 33))
        s, w = 32 * int(g.integers(0, 4)), 32 * int(g.integers(0, 4))
        T = int(g.integers(1, 32 * 40))
        B, kv = int(g.integers(1, 3)), int(g.integers(1, 3))
        ns = int(g.choice([0, 1, 3, 8]))
        d = synth.decode_inputs(cfg_id, T=T, B=B, kv_heads=kv, with_f64=True)
        dt = d["cfg"]["dtype"]
        cache = make_cache(d, r_k=rk, r_v=rv, s=s, w=w, P=P)
        cache.prefill(to_dev(d["K"], dt), to_dev(d["V"], dt))
        o = to_f64(cache.decode(to_dev(d["q"], dt), n_split=ns))
        torch.cuda.synchronize()
        ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, P, s, w, rk, rv, dt)
        err = rel_err(o, ref["o_stored"])
        print(f"[P=32 random {case}] cfg{cfg_id} T={T} B={B} kv={kv} r=({rk},{rv}) s={s} w={w} "
              f"split={ns}: err {err:.3e}")
        assert err <= TOL[dt], (case, cfg_id, T, rk, rv, s, w, ns, err)
