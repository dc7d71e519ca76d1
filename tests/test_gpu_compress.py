"""GPU parity of the batched page decomposition (pkv_compress_pages) against
the oracle's double-precision SVD of the same stored pages.

Bound (per page): ||X - Lf Rf||_F <= 1.001 * opt + 1e-5 ||X||_F with
opt = sqrt(sum_{i>r} sigma_i^2) from the oracle.  It is applied literally to
float32 factor output.  For bfloat16 factor output, storage rounding alone
adds an error floor, so the bound there is
    e^2 <= (1.001 opt + 1e-5 ||X||)^2 + (2^-8 ||X||)^2.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _check(Xs, dtype, r, out_dtype, label, check_sigma=True):
    """Xs: stored pages (n, 64, 128) numpy; returns worst ratios."""
    import torch
    require_gpu()
    X = to_dev(Xs, dtype)
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    Lf, Rf, sig = pkv.compress_pages(X, r, out_dtype=tdt)
    torch.cuda.synchronize()
    X64 = synth.storage_to_f64(Xs, dtype)
    L64, R64 = to_f64(Lf), to_f64(Rf)
    err = np.sqrt(((X64 - L64 @ R64) ** 2).sum(axis=(1, 2)))
    U, S, Wt = oracle.svd_batch(X64)
    opt = oracle.optimal_error(S, r)
    nrm = np.sqrt((X64 ** 2).sum(axis=(1, 2)))
    bound = 1.001 * opt + 1e-5 * nrm
    if out_dtype == "bf16":
        bound = np.sqrt(bound ** 2 + (2.0 ** -8 * nrm) ** 2)
    worst = np.max(err / np.maximum(bound, 1e-300))
    print(f"[compress {label} r={r} out={out_dtype}] worst err/bound = {worst:.4f} "
          f"max (e-opt)/opt = {np.max((err - opt) / np.maximum(opt, 1e-300)):.3e}")
    assert np.all(err <= bound), (label, r, out_dtype, worst)
    if not check_sigma:
        return worst
    # singular values agree with the oracle's for well-separated ranks
    sg = sig.cpu().numpy().astype(np.float64)
    dev = np.abs(sg - S[:, :r]) - (2e-3 * S[:, :r] + 1e-5 * S[:, :1])
    assert np.all(dev <= 0), float(dev.max())
    return worst


def _kv_pages(cfg_id, n_pages):
    cfg = synth.CONFIGS[cfg_id]
    k, v = synth.kv_head(cfg, 0, 0, n_pages * 64)
    X = np.concatenate([k, v]).reshape(2 * n_pages, 64, 128)
    return synth.to_storage(X, cfg["dtype"]), cfg["dtype"]


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_compress_lowrank_outlier_pages(out):
    Xs, dt = _kv_pages(2, 24)
    _check(Xs, dt, 16, out, "lowrank+outliers")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_compress_spectrum_pages(out):
    Xs, dt = _kv_pages(3, 16)
    _check(Xs, dt, 24, out, "spectrum")


def test_compress_fp32_pages():
    Xs, dt = _kv_pages(1, 13)
    assert dt == "f32"
    _check(Xs, dt, 16, "f32", "fp32 lowrank")


@pytest.mark.parametrize("r", [8, 16, 32])
def test_compress_batched_prefill_pages(r):
    n_total = 524288
    ids = np.concatenate([synth.noise_page_ids(5, n_total, 0.02)[:24], np.arange(40)])
    X = synth.compression_pages(ids, n_total)
    _check(synth.to_storage(X, "bf16"), "bf16", r, "f32", "spectrum+noise")


@pytest.mark.parametrize("r", [1, 5, 14, 40, 56])
def test_compress_odd_ranks(r):
    Xs, dt = _kv_pages(2, 6)
    _check(Xs, dt, r, "f32", "odd rank")


def test_compress_exact_rank_pages():
    """Integer A (64 x 8), B (8 x 128) with small entries: X = A B is exact in
    bf16, so rank >= 8 reconstructs it to float32 precision."""
    g = np.random.default_rng(3)
    A = g.integers(-3, 4, (6, 64, 8)).astype(np.float64)
    B = g.integers(-3, 4, (6, 8, 128)).astype(np.float64)
    X = A @ B
    assert np.abs(X).max() <= 256
    Xs = synth.to_storage(X, "bf16")
    assert np.array_equal(synth.storage_to_f64(Xs, "bf16"), X)
    import torch
    require_gpu()
    for r in (8, 16):
        Lf, Rf, _ = pkv.compress_pages(to_dev(Xs, "bf16"), r, out_dtype=torch.float32)
        err = np.sqrt(((X - to_f64(Lf) @ to_f64(Rf)) ** 2).sum(axis=(1, 2)))
        nrm = np.sqrt((X ** 2).sum(axis=(1, 2)))
        assert np.all(err <= 1e-5 * nrm), err / nrm


def test_compress_full_rank_reconstructs():
    import torch
    require_gpu()
    g = np.random.default_rng(4)
    X = g.standard_normal((4, 64, 128))
    Xs = synth.to_storage(X, "f32")
    Lf, Rf, _ = pkv.compress_pages(to_dev(Xs, "f32"), 64, out_dtype=torch.float32)
    X64 = Xs.astype(np.float64)
    err = np.sqrt(((X64 - to_f64(Lf) @ to_f64(Rf)) ** 2).sum(axis=(1, 2)))
    assert np.all(err <= 1e-5 * np.sqrt((X64 ** 2).sum(axis=(1, 2))))


def _tied_pages(n, seed):
    """Pages with exactly repeated singular values, exact in bf16: X = A diag(s) B
    with A a row-permuted, sign-flipped 64 x 64 Hadamard matrix, B the first
    64 rows of a column-signed 128 x 128 Hadamard matrix and s = (4 x 8,
    2 x 16, 1 x 40).  Entries are integers of magnitude <= 104; the singular
    values are 8 sqrt(128) s, in three tied groups."""
    from scipy.linalg import hadamard
    g = np.random.default_rng(seed)
    s = np.concatenate([np.full(8, 4.0), np.full(16, 2.0), np.full(40, 1.0)])
    H64, H128 = hadamard(64).astype(np.float64), hadamard(128).astype(np.float64)
    out = []
    for _ in range(n):
        A = H64[g.permutation(64)] * g.choice([-1.0, 1.0], 64)[:, None]
        B = H128[g.permutation(128)[:64]] * g.choice([-1.0, 1.0], 128)[None, :]
        out.append((A * s) @ B)
    X = np.stack(out)
    assert np.abs(X).max() <= 104 and np.all(X == np.rint(X))
    return X


@pytest.mark.parametrize("r", [8, 12, 16, 24, 32])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_compress_exactly_tied_singular_values(r, out):
    """Error-only (the truncation inside a tied group is not unique): the
    kept columns must stay orthonormal across each group, so a rank-r
    truncation reaches the optimal error whatever the cut (r = 8 and 24 cut
    between groups, 12, 16 and 32 inside one)."""
    X = _tied_pages(12, 7)
    Xs = synth.to_storage(X, "bf16")
    assert np.array_equal(synth.storage_to_f64(Xs, "bf16"), X)
    _check(Xs, "bf16", r, out, "tied sigma", check_sigma=False)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("r", [8, 16, 32])
def test_compress_crowded_spectrum(dt, r):
    """Kept singular values 1e-4 apart (relative) on Haar factors: the
    eigenvectors of such a cluster come out orthogonal only after the kept
    columns are orthonormalized; the literal bound on float32 output."""
    g = np.random.default_rng(100 + r)
    n = 12
    U = synth.haar_columns(g.standard_normal((n, 64, 64)))
    W = synth.haar_columns(g.standard_normal((n, 128, 64)))
    s = 1.0 - 1e-4 * np.arange(64)
    s[40:] *= 1e-2  # a clear drop after the first 40
    X = (U * s) @ np.swapaxes(W, -1, -2)
    _check(synth.to_storage(X, dt), dt, r, "f32", f"crowded {dt}", check_sigma=False)


def test_compress_zero_page():
    import torch
    require_gpu()
    X = torch.zeros((3, 64, 128), dtype=torch.bfloat16, device="cuda:0")
    Lf, Rf, sig = pkv.compress_pages(X, 16)
    torch.cuda.synchronize()
    assert not Lf.float().abs().sum().item() and not Rf.float().abs().sum().item()
    assert not sig.abs().sum().item()


def test_compress_empty_batch():
    import torch
    require_gpu()
    X = torch.zeros((0, 64, 128), dtype=torch.bfloat16, device="cuda:0")
    Lf, Rf, sig = pkv.compress_pages(X, 16)
    assert Lf.shape == (0, 64, 16)
