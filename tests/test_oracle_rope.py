"""Pins of the oracle's pre-RoPE key path (PuzzleKV App. D.3 "RoPE Key
Analysis"; the rotary embedding is RoFormer's, the page's ref. [15]).

The rotation is pinned by its definition on basis vectors (pairing and sign),
by the properties that make it a rotary embedding (orthogonal, identity at
position 0, additive in the position, scores depending only on the position
difference), and the pre-RoPE decode by two reductions to plain attention over
rotated keys: a cache whose pages are all dense, and full-rank factors."""
import math

import numpy as np
import pytest

import oracle
import synth

D = 128


def _freqs():
    return synth.rope_inv_freq(1e6, D).astype(np.float64)


@pytest.mark.parametrize("m", [0, 1, 17, 63])
def test_basis_vectors_turn_in_their_pair(m):
    # a single pair with angle pi/2 at position 1: (1, 0) -> (0, 1), (0, 1) -> (-1, 0)
    f = np.zeros(D // 2)
    f[m] = math.pi / 2
    e = np.zeros((2, D))
    e[0, m] = 1.0
    e[1, m + D // 2] = 1.0
    out = oracle.rope_rotate(e, [1, 1], f)
    want = np.zeros((2, D))
    want[0, m + D // 2] = 1.0
    want[1, m] = -1.0
    np.testing.assert_allclose(out, want, atol=1e-15)
    # other pairs (frequency 0 here) are untouched
    g = np.random.default_rng(m).standard_normal((1, D))
    g[0, [m, m + D // 2]] = 0.0
    np.testing.assert_array_equal(oracle.rope_rotate(g, [1], f), g)


def test_rotation_by_a_known_angle():
    f = _freqs()
    x = np.zeros((1, D))
    x[0, 5] = 2.0
    t = 1000
    out = oracle.rope_rotate(x, [t], f)
    a = t * float(np.float32(1e6 ** (-10 / 128)))
    assert abs(out[0, 5] - 2.0 * math.cos(a)) < 1e-13
    assert abs(out[0, 5 + 64] - 2.0 * math.sin(a)) < 1e-13
    assert np.count_nonzero(out) == 2


def test_orthogonal_identity_at_zero_and_additive():
    f = _freqs()
    g = np.random.default_rng(1).standard_normal((50, D))
    pos = np.arange(50) * 997 + 3
    r = oracle.rope_rotate(g, pos, f)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(g, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(oracle.rope_rotate(g, np.zeros(50), f), g)
    twice = oracle.rope_rotate(oracle.rope_rotate(g, pos, f), pos + 11, f)
    np.testing.assert_allclose(twice, oracle.rope_rotate(g, 2 * pos + 11, f), atol=1e-9)


def test_scores_depend_on_the_position_difference():
    f = _freqs()
    g = np.random.default_rng(2).standard_normal((2, D))
    for a, b in [(0, 5), (100, 131071), (7, 7), (40000, 12)]:
        lhs = oracle.rope_rotate(g[:1], [a], f) @ oracle.rope_rotate(g[1:], [b], f).T
        rhs = g[:1] @ oracle.rope_rotate(g[1:], [b - a], f).T
        assert abs(lhs[0, 0] - rhs[0, 0]) < 1e-9 * np.abs(g).sum() ** 2


def _inputs(T, seed=3):
    g = np.random.default_rng(seed)
    q = g.standard_normal((1, 2, D))
    K = g.standard_normal((1, 1, T, D))
    V = g.standard_normal((1, 1, T, D))
    return q, K, V


def test_all_dense_cache_is_attention_over_rotated_keys():
    f = _freqs()
    T = 64 + 128 + 40  # sink, window and a partial page: nothing factorized
    q, K, V = _inputs(T)
    out = oracle.decode(q, K, V, T, 64, 64, 128, 8, 8, None, key_rope=f)
    ref = oracle.attention(q[0], oracle.rope_rotate(K[0, 0], np.arange(T), f), V[0, 0])
    np.testing.assert_allclose(out["o_exact"][0], ref, atol=1e-12)
    np.testing.assert_allclose(out["o_stored"][0], ref, atol=1e-12)


def test_full_rank_factors_are_attention_over_rotated_keys():
    # r = P reconstructs every page exactly: the rotation must act on each
    # reconstructed key at its own token index
    f = _freqs()
    T = 64 * 9 + 13
    q, K, V = _inputs(T, seed=4)
    out = oracle.decode(q, K, V, T, 64, 64, 128, 64, 64, None, key_rope=f)
    ref = oracle.attention(q[0], oracle.rope_rotate(K[0, 0], np.arange(T), f), V[0, 0])
    np.testing.assert_allclose(out["o_exact"][0], ref, atol=1e-12)


def test_truncation_acts_on_the_unrotated_keys():
    # with r < P the pre-RoPE result differs from factorizing rotated keys;
    # and equals attention over rope(truncated pre-RoPE pages)
    f = _freqs()
    T = 64 * 6
    q, K, V = _inputs(T, seed=5)
    out = oracle.decode(q, K, V, T, 64, 64, 128, 8, 64, None, key_rope=f)
    Khat = K[0, 0].copy()
    for p in range(1, 4):  # the factorized pages at T = 384: 1 to 3
        U, S, Wt = np.linalg.svd(Khat[64 * p:64 * (p + 1)], full_matrices=False)
        Khat[64 * p:64 * (p + 1)] = (U[:, :8] * S[:8]) @ Wt[:8]
    ref = oracle.attention(q[0], oracle.rope_rotate(Khat, np.arange(T), f), V[0, 0])
    np.testing.assert_allclose(out["o_exact"][0], ref, atol=1e-10)
    post = oracle.decode(q, oracle.rope_rotate(K[0, 0], np.arange(T), f)[None, None], V, T, 64, 64, 128,
                         8, 64, None)
    assert np.abs(post["o_exact"] - out["o_exact"]).max() > 1e-6


def test_incremental_decoder_rotates_like_decode():
    f = _freqs()
    T = 64 * 7
    q, K, V = _inputs(T, seed=6)
    inc = oracle.IncrementalDecoder(K, V, 64, 64, 128, 16, 16, "bf16", key_rope=f)
    for t in (64 * 5 + 1, T):
        o_s, o_e = inc.step(q, t)
        full = oracle.decode(q, K, V, t, 64, 64, 128, 16, 16, "bf16", key_rope=f)
        np.testing.assert_allclose(o_s, full["o_stored"], atol=1e-13)
        np.testing.assert_allclose(o_e, full["o_exact"], atol=1e-13)
