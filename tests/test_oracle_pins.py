"""Pins for the CPU oracle: it is checked against what the pages and the
mathematics fix, never against itself.

Each test names what it pins.  Together they are chosen so that a plausible
slip in the oracle -- a dropped scale, a flipped rotation sign, a transposed
factor, the wrong singular vectors kept, an off-by-one in the page classes, the
wrong GQA head, a rounding that is not nearest-even -- fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")


# ---------------------------------------------------------------- rounding

def _bf16_nearest_bruteforce(x):
    """Nearest bfloat16 by enumeration of the neighbours of the truncation,
    ties to the even pattern (independent of both implementations)."""
    f32 = np.float32(x)
    u = int(np.array(f32).view(np.uint32)) >> 16
    best = None
    for c in (u - 1, u, u + 1):
        c &= 0xFFFF
        val = float(np.array(np.uint32(c << 16)).view(np.float32))
        if math.isinf(val) or math.isnan(val):
            continue
        dist = abs(val - x)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_rounding_nearest_even(oracle):
    g = np.random.default_rng(11)
    xs = np.concatenate([
        g.standard_normal(3000) * 10.0 ** g.integers(-6, 6, 3000),
        # exact midpoints between consecutive bf16 values: ties must go to even
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0 + 2.0 ** -7,
                  1.0 + 2.0 ** -8 + 2.0 ** -40]),
    ])
    want = np.array([_bf16_nearest_bruteforce(x) for x in xs], dtype=np.uint16)
    got_o = oracle.bf16_bits(xs)
    got_s = synth.to_bf16_bits(xs)
    np.testing.assert_array_equal(got_o, want)
    np.testing.assert_array_equal(got_s, want)
    # the tie cases explicitly: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oracle.bf16_decode(oracle.bf16_bits([1.0 + 2.0 ** -8]))[0] == 1.0
    assert oracle.bf16_decode(oracle.bf16_bits([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # just above the tie rounds up
    assert oracle.bf16_decode(oracle.bf16_bits([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7


def test_f32_rounding_matches_numpy(oracle):
    g = np.random.default_rng(12)
    x = g.standard_normal(1000) * 1e3
    np.testing.assert_array_equal(oracle.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- SVD

def _pages(g):
    P, d = 64, 128
    yield "gauss", g.standard_normal((P, d))
    yield "rank8", g.standard_normal((P, 8)) @ g.standard_normal((8, d))
    yield "spectrum", synth.spectrum_pages(g, 1, P, d)[0]
    yield "outlier", synth.lowrank_pages(g, 1, P, d)[0] * np.where(np.arange(d) % 37 == 0, 10, 1)


def test_svd_singular_values_match_lapack(oracle):
    g = np.random.default_rng(1)
    for name, X in _pages(g):
        U, S, Wt = oracle.svd(X)
        ref = np.linalg.svd(X, compute_uv=False)
        np.testing.assert_allclose(S, ref, rtol=0, atol=1e-12 * ref[0], err_msg=name)
        assert np.all(np.diff(S) <= 0), name
        np.testing.assert_allclose(U.T @ U, np.eye(64), atol=1e-13, err_msg=name)
        nz = S > 1e-10 * S[0]
        np.testing.assert_allclose((Wt[nz] @ Wt[nz].T), np.eye(nz.sum()), atol=1e-13, err_msg=name)
        np.testing.assert_allclose(U @ np.diag(S) @ Wt, X, atol=1e-13 * np.abs(X).max(), err_msg=name)


def test_svd_2x2_closed_form(oracle):
    # sigma_1^2 + sigma_2^2 = ||X||_F^2 and sigma_1 sigma_2 = |det X|
    for X in ([[3.0, 1.0], [1.0, 3.0]], [[1.0, 2.0], [3.0, 4.0]], [[0.0, 5.0], [0.0, 0.0]]):
        X = np.array(X)
        U, S, Wt = oracle.svd(X)
        fro2 = (X ** 2).sum()
        det = abs(np.linalg.det(X))
        disc = math.sqrt(max(fro2 ** 2 - 4 * det ** 2, 0.0))
        s1 = math.sqrt((fro2 + disc) / 2)
        s2 = math.sqrt(max((fro2 - disc) / 2, 0.0))
        np.testing.assert_allclose(S, [s1, s2], atol=1e-14 * max(s1, 1))
        np.testing.assert_allclose(U @ np.diag(S) @ Wt, X, atol=1e-14 * max(s1, 1))


def test_gram_route_spans_same_subspace(oracle):
    """The Gram matrix's leading eigenvectors are the left singular vectors
    (PuzzleKV Sec. 3.3, after Eq. 3): principal angles between the oracle's
    U_r and the top-r eigenvectors of X X^T are ~0 when sigma_r/sigma_r+1 > 1.1."""
    g = np.random.default_rng(2)
    X = synth.spectrum_pages(g, 1, 64, 128)[0]
    U, S, Wt = oracle.svd(X)
    lam, Q = np.linalg.eigh(X @ X.T)
    Q = Q[:, ::-1]
    for r in (8, 16, 24, 32):
        assert S[r - 1] / S[r] > 1.01
        cosines = np.linalg.svd(U[:, :r].T @ Q[:, :r], compute_uv=False)
        assert np.arccos(np.clip(cosines.min(), -1, 1)) < 1e-6


# ------------------------------------------------ truncation (Eckart-Young)

def test_truncation_error_is_tail_energy(oracle):
    g = np.random.default_rng(3)
    for name, X in _pages(g):
        for r in (1, 8, 16, 24, 32):
            Lf, Rf, S = oracle.factorize(X, r)
            assert Lf.shape == (64, r) and Rf.shape == (r, 128)
            err = np.linalg.norm(X - Lf @ Rf)
            tail = math.sqrt((np.linalg.svd(X, compute_uv=False)[r:] ** 2).sum())
            assert abs(err - tail) <= 1e-12 * np.linalg.norm(X) + 1e-12 * tail, (name, r)
            np.testing.assert_allclose(oracle.optimal_error(S, r), tail, rtol=1e-12,
                                       atol=1e-12 * np.linalg.norm(X))
            # stored placement: Rf rows orthonormal, Lf columns carry sigma
            np.testing.assert_allclose(np.linalg.norm(Lf, axis=0), S[:r], rtol=1e-12)


def test_eckart_young_bruteforce_2x3():
    """P=2, d=3, r=1: the best rank-1 error over a fine scan of left unit vectors
    u(theta) (X_hat = u u^T X is optimal for a given u) approaches the oracle's."""
    import oracle as o
    g = np.random.default_rng(4)
    for _ in range(3):
        X = g.standard_normal((2, 3))
        Lf, Rf, S = o.factorize(X, 1)
        opt = np.linalg.norm(X - Lf @ Rf)
        th = np.linspace(0, np.pi, 1_000_000, endpoint=False)
        u = np.stack([np.cos(th), np.sin(th)])            # (2, n)
        proj = u.T @ X                                    # (n, 3) = u^T X
        err2 = (X ** 2).sum() - (proj ** 2).sum(axis=1)   # ||X - u u^T X||^2
        best = math.sqrt(max(err2.min(), 0.0))
        assert best >= opt * (1 - 1e-12)
        assert best - opt < 1e-9 * max(1.0, np.linalg.norm(X))


def test_eckart_young_bruteforce_3x4():
    import oracle as o
    g = np.random.default_rng(5)
    X = g.standard_normal((3, 4))
    Lf, Rf, S = o.factorize(X, 1)
    opt = np.linalg.norm(X - Lf @ Rf)
    n = 2000
    th = np.linspace(0, np.pi, n)
    ph = np.linspace(0, 2 * np.pi, n, endpoint=False)
    TH, PH = np.meshgrid(th, ph, indexing="ij")
    u = np.stack([np.sin(TH) * np.cos(PH), np.sin(TH) * np.sin(PH), np.cos(TH)], -1).reshape(-1, 3)
    proj = u @ X
    err2 = (X ** 2).sum() - (proj ** 2).sum(axis=1)
    best = math.sqrt(max(err2.min(), 0.0))
    assert best >= opt * (1 - 1e-12)
    assert best - opt < 1e-4 * np.linalg.norm(X)


@pytest.mark.parametrize("P", [64, 32])
def test_full_rank_reconstructs(oracle, P):
    g = np.random.default_rng(6)
    X = g.standard_normal((P, 128))
    Lf, Rf, _ = oracle.factorize(X, P)  # r = min(P, d)
    assert np.linalg.norm(X - Lf @ Rf) <= 1e-13 * np.linalg.norm(X)


@pytest.mark.parametrize("P", [64, 32])
def test_exact_rank_k_reconstructs(oracle, P):
    g = np.random.default_rng(7)
    X = g.standard_normal((P, 8)) @ g.standard_normal((8, 128))
    for r in (8, 9, 16):
        Lf, Rf, _ = oracle.factorize(X, r)
        assert np.linalg.norm(X - Lf @ Rf) <= 1e-12 * np.linalg.norm(X)
    Lf, Rf, _ = oracle.factorize(X, 7)
    assert np.linalg.norm(X - Lf @ Rf) > 1e-3 * np.linalg.norm(X)


def test_zero_page_factors_are_zero(oracle):
    Lf, Rf, S = oracle.factorize(np.zeros((64, 128)), 16)
    assert not np.any(Lf) and not np.any(Rf) and not np.any(S)


# ---------------------------------------------------------------- attention

def test_attention_two_token_closed_form(oracle):
    """Scores q.k/sqrt(d): with q = c sqrt(d) e0 and k_j = beta_j e0 the
    weights are a logistic function of c (beta_1 - beta_0)."""
    d = 128
    c = 0.7
    q = np.zeros((1, d))
    q[0, 0] = c * math.sqrt(d)
    K = np.zeros((2, d))
    K[0, 0], K[1, 0] = 1.0, 3.0
    V = np.zeros((2, d))
    V[0, 5], V[1, 9] = 1.0, 1.0
    o = oracle.attention(q, K, V)
    w1 = 1.0 / (1.0 + math.exp(-c * (3.0 - 1.0)))
    np.testing.assert_allclose(o[0, 9], w1, rtol=1e-14)
    np.testing.assert_allclose(o[0, 5], 1 - w1, rtol=1e-14)


def test_attention_special_cases(oracle):
    g = np.random.default_rng(8)
    d = 128
    q = g.standard_normal((3, d))
    V = g.standard_normal((50, d))
    K = np.tile(g.standard_normal(d), (50, 1))            # equal keys -> mean of V
    np.testing.assert_allclose(oracle.attention(q, K, V), np.tile(V.mean(0), (3, 1)), atol=1e-13)
    np.testing.assert_allclose(oracle.attention(q, K[:1], V[:1]), np.tile(V[0], (3, 1)), atol=1e-15)


def test_attention_matches_torch_sdpa(oracle):
    import torch
    g = np.random.default_rng(9)
    q = g.standard_normal((4, 128))
    K = g.standard_normal((300, 128)) * 3
    V = g.standard_normal((300, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None]
    )[0].numpy()
    np.testing.assert_allclose(oracle.attention(q, K, V), ref, atol=1e-12)


def test_gqa_head_mapping(oracle):
    """Query head j reads KV head floor(j / G): make every value row of KV head
    h equal to h * ones, then o[j] must be floor(j / G) * ones."""
    B, Hkv, G, T, d = 1, 4, 3, 64 * 6, 128
    g = np.random.default_rng(10)
    K = g.standard_normal((B, Hkv, T, d))
    V = np.ones((B, Hkv, T, d)) * np.arange(Hkv)[None, :, None, None]
    q = g.standard_normal((B, Hkv * G, d))
    out = oracle.decode(q, K, V, T, 64, 64, 128, 64, 64, None)["o_stored"]
    want = np.repeat(np.arange(Hkv), G)[None, :, None] * np.ones((B, Hkv * G, d))
    np.testing.assert_allclose(out, want, atol=1e-12)


def test_pagewise_eq4_eq5_equals_global_softmax(oracle):
    """Eq. 4 per page (factorized pages contracted through their factors,
    dense pages directly) merged by Eq. 5 equals softmax attention over the
    reconstructed cache; an empty state contributes nothing."""
    g = np.random.default_rng(11)
    P, d, T, r = 64, 128, 64 * 9 + 17, 16
    K = synth.lowrank_pages(g, 10, P, d).reshape(-1, d)[:T] * 2
    V = synth.lowrank_pages(g, 10, P, d).reshape(-1, d)[:T]
    q = g.standard_normal((4, d))
    cls, _ = oracle.classify(T, P, 64, 128)
    Khat, Vhat = K.copy(), V.copy()
    states = []
    for p in range(len(cls)):
        sl = slice(p * P, min((p + 1) * P, T))
        if cls[p] == oracle.FACT:
            LK, RK, _ = oracle.factorize(K[sl], r)
            LV, RV, _ = oracle.factorize(V[sl], r)
            Khat[sl], Vhat[sl] = LK @ RK, LV @ RV
            states.append(oracle.page_state_factored(q, LK, RK, LV, RV))
        else:
            states.append(oracle.page_state_dense(q, K[sl], V[sl]))
    states.append((np.full(4, -np.inf), np.zeros(4), np.zeros((4, d))))
    merged = oracle.merge_states(states)
    naive = oracle.attention(q, Khat, Vhat)
    np.testing.assert_allclose(merged, naive, rtol=1e-13, atol=1e-13 * np.abs(naive).max())
    assert (cls == oracle.FACT).sum() == 6


@pytest.mark.parametrize("P,s,w", [(64, 64, 128), (32, 32, 32)])
def test_full_rank_decode_equals_dense(oracle, P, s, w):
    # r = min(P, d): every factorized page is reproduced, so the hybrid cache
    # is the dense cache (32-token pages: the pages' default dense region)
    d = synth.decode_inputs(1, with_f64=True)
    assert int((oracle.classify(d["T"], P, s, w)[0] == oracle.FACT).sum()) > 0
    out = oracle.decode(d["q64"], d["K64"], d["V64"], d["T"], P, s, w, P, P, None)["o_stored"]
    dense = oracle.attention(d["q64"][0], d["K64"][0, 0], d["V64"][0, 0])
    np.testing.assert_allclose(out[0], dense, atol=1e-12 * np.abs(dense).max())


def test_dense_only_cache_is_standard_attention(oracle):
    d = synth.decode_inputs(1, T=64 + 128 + 40, with_f64=True)
    cfg = d["cfg"]
    cls, _ = oracle.classify(d["T"], 64, 64, 128)
    assert not np.any(cls == oracle.FACT)
    out = oracle.decode(d["q64"], d["K64"], d["V64"], d["T"], 64, 64, 128, 16, 16, "f32")
    dense = oracle.attention(d["q64"][0], d["K64"][0, 0], d["V64"][0, 0])
    np.testing.assert_array_equal(out["o_stored"][0], dense)


# ---------------------------------------------------------- classification

def _counts(oracle, T, P=64, s=64, w=128, n_fact=None):
    cls, _ = oracle.classify(T, P, s, w, n_fact)
    return {k: int((cls == v).sum()) for k, v in
            (("sink", oracle.SINK), ("fact", oracle.FACT), ("win", oracle.WIN), ("part", oracle.PART))}


def test_classification_workload_counts(oracle):
    assert _counts(oracle, 1024) == dict(sink=1, fact=13, win=2, part=0)
    assert _counts(oracle, 32768)["fact"] == 509
    assert _counts(oracle, 131072)["fact"] == 2045
    assert _counts(oracle, 8192)["fact"] == 125
    assert _counts(oracle, 8192 + 512)["fact"] == 133
    # a promotion happens exactly when a step completes a page (steps 64k)
    prev = 125
    promos = []
    for t in range(1, 513):
        f = _counts(oracle, 8192 + t)["fact"]
        if f != prev:
            assert f == prev + 1
            promos.append(t)
        prev = f
    assert promos == [64 * k for k in range(1, 9)]


def test_classification_default_dense_region(oracle):
    """PuzzleKV, Sec. 4.1 (default dense region): a 32-token sink page, the
    last page to complete and the page being filled are kept uncompressed."""
    gold = json.load(open(GOLDEN))["default_dense_region"]
    P = gold["P"]
    cls, slot = oracle.classify(10 * P + 5, P, gold["sink_tokens"], gold["window_completed_pages"] * P)
    assert list(cls) == [oracle.SINK] + [oracle.FACT] * 8 + [oracle.WIN, oracle.PART]
    assert list(slot[1:9]) == list(range(8))
    # the partial page reuses the ring slot of the page that left the window
    assert slot[10] != slot[9]


def test_classification_slots_and_pending_promotion(oracle):
    P, s, w = 64, 64, 128
    cls, slot = oracle.classify(8192, P, s, w)
    assert cls[0] == oracle.SINK and slot[0] == 0
    assert list(np.nonzero(cls == oracle.WIN)[0]) == [126, 127]
    assert sorted(slot[cls == oracle.WIN]) == sorted([(126 - 1) % 3, (127 - 1) % 3])
    # after the page-completing append but before promotion: 3 window pages
    cls2, slot2 = oracle.classify(8256, P, s, w, n_fact=125)
    assert list(np.nonzero(cls2 == oracle.WIN)[0]) == [126, 127, 128]
    assert len(set(slot2[cls2 == oracle.WIN])) == 3
    cls3, slot3 = oracle.classify(8256, P, s, w)
    assert cls3[126] == oracle.FACT and slot3[126] == 125
    # few tokens: everything in the (partial) sink
    cls4, _ = oracle.classify(40, P, s, w)
    assert list(cls4) == [oracle.SINK]
    with pytest.raises(ValueError):
        oracle.classify(100, 64, 32, 128)


# ---------------------------------------------------------- storage

def test_storage_ratio_printed_values(oracle):
    gold = json.load(open(GOLDEN))
    for e in gold["storage_ratio"]:
        got = oracle.storage_ratio(e["P"], e["r_k"], e["r_v"], e["d"])
        assert abs(got - e["value"]) <= e["abs_tol"], e
    for e in gold["kv_footprint_gib"]:
        nbytes = oracle.kv_cache_elements(e["layers"], e["kv_heads"], e["tokens"], e["head_dim"]) * \
            e["bytes_per_elem"]
        assert abs(nbytes / 2 ** 30 - e["value"]) <= e["abs_tol"], e
