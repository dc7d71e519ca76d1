"""Pins of the oracle's INT4 factor quantization (PuzzleKV Sec. 4.3
"Quantization Compatibility"): symmetric INT4 codes with one 16-bit scale per
group, the singular values split as Sigma^(1/2) between the two factors,
column-wise groups for Lt_K, Rt_K, Rt_V and row-wise groups for Lt_V."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")


def test_grid_values_round_trip_exactly():
    g = np.random.default_rng(1)
    s0 = O.round_to(np.abs(g.standard_normal(6)) + 0.1, "bf16")  # one scale per column
    k = g.integers(-7, 8, (9, 6)).astype(np.float64)
    k[0] = 7  # the group maximum sits on the grid's end, so the scale is recovered
    x = k * s0[None, :]
    q, s = O.quantize_int4(x, axis=0)
    np.testing.assert_array_equal(q, k)
    np.testing.assert_array_equal(s[0], s0)
    np.testing.assert_array_equal(O.dequantize_int4(q, s), x)


def test_error_within_half_a_step():
    g = np.random.default_rng(2)
    x = g.standard_normal((64, 24)) * np.exp(g.standard_normal(24))[None, :]
    for axis in (0, 1):
        q, s = O.quantize_int4(x, axis=axis)
        assert q.min() >= -7 and q.max() <= 7
        err = np.abs(O.dequantize_int4(q, s) - x)
        assert np.all(err <= 0.5 * s + 1e-15 * np.abs(x))
        # each group's largest entry uses code +-7 (the scale's bf16 rounding
        # moves max|x| / s by less than half a step)
        assert np.all(np.max(np.abs(q), axis=axis) == 7)


def test_zero_group_and_signs():
    x = np.array([[0.0, 1.0], [0.0, -1.0], [0.0, 0.5]])
    q, s = O.quantize_int4(x, axis=0)
    assert s[0, 0] == 0 and np.all(q[:, 0] == 0)
    assert q[0, 1] == 7 and q[1, 1] == -7
    assert q[2, 1] == 4  # 3.5 / 1 -> ties to even


def test_group_orientation():
    """A single large entry only coarsens its own group: row-wise groups keep
    the other rows fine, column-wise groups keep the other columns fine."""
    x = np.full((4, 4), 1.0)
    x[0, 0] = 100.0
    qr, sr = O.quantize_int4(x, axis=1)  # one scale per row
    qc, sc = O.quantize_int4(x, axis=0)  # one scale per column
    dr, dc = O.dequantize_int4(qr, sr), O.dequantize_int4(qc, sc)
    np.testing.assert_allclose(dr[1:], x[1:], rtol=0, atol=0.08)
    np.testing.assert_allclose(dc[:, 1:], x[:, 1:], rtol=0, atol=0.08)
    assert abs(dr[0, 1] - 1.0) > 0.9 and abs(dc[1, 0] - 1.0) > 0.9  # coarse in the big group


def test_sqrt_sigma_split_and_group_axes():
    """int4_factors places Sigma^(1/2) on both factors: before quantization the
    product is the rank-r truncation, and each factor's groups are the ones
    Sec. 4.3 names (checked against quantize_int4 on the split factors)."""
    g = np.random.default_rng(3)
    X = g.standard_normal((64, 128)) @ np.diag(np.arange(1, 129) ** -1.0)
    U, S, Wt = O.svd(X)
    r = 16
    h = np.sqrt(S[:r])
    Lt, Rt = U[:, :r] * h, Wt[:r] * h[:, None]
    np.testing.assert_allclose(Lt @ Rt, (U[:, :r] * S[:r]) @ Wt[:r], rtol=0, atol=1e-12)
    for kind, laxis in (("K", 0), ("V", 1)):
        Lq, Rq = O.int4_factors(U, S, Wt, r, kind)
        np.testing.assert_array_equal(Lq, O.dequantize_int4(*O.quantize_int4(Lt, axis=laxis)))
        np.testing.assert_array_equal(Rq, O.dequantize_int4(*O.quantize_int4(Rt, axis=0)))
        # reconstruction within the first-order quantization error bound
        dL, dR = Lq - Lt, Rq - Rt
        bound = (np.linalg.norm(dL) * np.linalg.norm(Rt) + np.linalg.norm(Lt) * np.linalg.norm(dR)
                 + np.linalg.norm(dL) * np.linalg.norm(dR))
        assert np.linalg.norm(Lq @ Rq - Lt @ Rt) <= bound


def test_group_orientation_of_int4_codes_by_outcome():
    """Sec. 4.3 groups Lt_K, Rt_K and Rt_V by column and Lt_V by row.  The
    page below makes each choice visible in the codes int4_codes returns:
    U (Hadamard / 8) and W (the first 64 rows of Hadamard / sqrt(128)) have
    entries of one magnitude, and sigma_1 exceeds the other kept singular
    values 256-fold, so Lt = U_r Sigma_r^(1/2) has entries +-7 * 2^0 in its
    first column and +-7 * 2^-4 elsewhere.
      - per column of Lt (keys): every column sits on its own grid, so the
        dequantized Lt_K is exact;
      - per row of Lt (values): each row's scale comes from its first-column
        entry, so every other column rounds to code 0;
      - per column of Rt (keys and values): each channel's scale comes from
        row 0, so rows 1.. round to code 0.
    A swapped axis in any of the four factors flips one of these."""
    from scipy.linalg import hadamard
    P, d, r = 64, 128, 8
    U = hadamard(P).astype(np.float64) / 8.0
    Wt = hadamard(d)[:P].astype(np.float64) / np.sqrt(d)
    # Lt[j, i] = U[j, i] sqrt(S_i) = +-7 * 2^e_i  <=>  S_i = (56 * 2^e_i)^2
    e = np.array([0.0] + [-4.0] * (P - 1))
    S = (56.0 * 2.0 ** e) ** 2
    np.testing.assert_allclose(U.T @ U, np.eye(P), atol=1e-15)
    np.testing.assert_allclose(Wt @ Wt.T, np.eye(P), atol=1e-15)
    for kind in ("K", "V"):
        Lt, Rt, lq, ls, rq, rs = O.int4_codes(U, S, Wt, r, kind)
        np.testing.assert_allclose(np.abs(Lt[:, 0]), 7.0, rtol=1e-15)
        np.testing.assert_allclose(np.abs(Lt[:, 1:]), 7.0 / 16, rtol=1e-15)
        Ld, Rd = O.dequantize_int4(lq, ls), O.dequantize_int4(rq, rs)
        if kind == "K":
            np.testing.assert_array_equal(Ld, Lt)  # each column on its own grid
            assert np.all(np.abs(lq) == 7)
        else:
            np.testing.assert_array_equal(Ld[:, 0], Lt[:, 0])
            assert np.all(lq[:, 1:] == 0)  # coarsened by the row's first entry
        # Rt, per column for both kinds: row 0 kept to the scale's rounding,
        # the smaller rows round to zero
        assert np.all(np.abs(rq[0]) == 7) and np.all(rq[1:] == 0)
        np.testing.assert_allclose(Rd[0], Rt[0], rtol=2.0 ** -8)


def test_int4_storage_ratio_printed_value():
    for e in json.load(open(GOLDEN))["int4_storage_ratio"]:
        v = O.int4_storage_ratio(e["T"], e["P"], e["d"], e["r_k"], e["r_v"], e["dense_pages"])
        assert abs(v - e["value"]) <= e["abs_tol"], (v, e)


def test_int4_cache_reconstruction():
    """A cache reconstructed with INT4 factors keeps its dense pages exactly
    and moves its factorized pages by a few percent of their energy (INT4
    codes), never by zero."""
    g = np.random.default_rng(4)
    P, d, T, r = 64, 128, 64 * 5, 8
    X = g.standard_normal((T, d))
    Xs, Xe, _ = O.reconstruct_cache(X, T, P, 64, 128, r, "int4", kind="K")
    cls, _ = O.classify(T, P, 64, 128)
    dense = np.repeat(cls != O.FACT, P)
    np.testing.assert_array_equal(Xs[dense], X[dense])
    f = ~dense
    rel = np.linalg.norm(Xs[f] - Xe[f]) / np.linalg.norm(Xe[f])
    assert 0 < rel < 0.2  # INT4 codes: a few percent of the factored pages' energy
