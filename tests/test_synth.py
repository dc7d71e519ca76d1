"""CPU tests of the seeded input generators (synth): the device-side pool of
the batched-compression workload follows the same recipe as the host one
(spectrum pages with sigma_i = i^-1.2, exactly the seeded noise pages), and
its float64 -> bfloat16 step rounds once, as the host routine does."""
import numpy as np
import torch

import synth


def test_bf16_bits_torch_rounds_once_like_the_host():
    g = np.random.default_rng(11)
    x = g.standard_normal(400_000) * np.exp(3 * g.standard_normal(400_000))
    # values at and next to bf16 rounding ties, where a double rounding through
    # float32 would go wrong
    b = synth.bf16_bits_to_f64(synth.to_bf16_bits(x[:50_000]))
    tie = b + 0.5 * np.abs(b) * 2.0 ** -7 * np.sign(b)
    x = np.concatenate([x, tie, tie * (1 + 2.0 ** -30), tie * (1 - 2.0 ** -30), -tie, [0.0, -0.0]])
    ref = synth.to_bf16_bits(x).view(np.int16)
    got = synth.bf16_bits_torch(torch.from_numpy(x)).numpy()
    np.testing.assert_array_equal(got, ref)


def test_device_pool_recipe_on_the_host():
    n = 1500
    bits = synth.compression_pool_device(n, device="cpu", chunk=512)
    assert bits.shape == (n, 64, 128) and bits.dtype == torch.int16
    X = synth.bf16_bits_to_f64(bits.numpy().view(np.uint16))
    noise = synth.noise_page_ids(5, n, 0.02)
    assert noise.size == round(0.02 * n)
    spec = np.setdiff1d(np.arange(n), noise)
    s = np.linalg.svd(X[spec[:200]], compute_uv=False)
    want = np.arange(1, 65) ** -1.2
    # one bf16 rounding of a unit-spectrum page moves sigma_i by ~2^-9 of sigma_1
    assert np.abs(s - want).max() < 4e-3
    sn = np.linalg.svd(X[noise], compute_uv=False)
    # N(0,1) pages of 64 x 128: singular values near sqrt(128) (1 +- sqrt(1/2))
    assert sn.max() < np.sqrt(128) * 1.9 and sn.min() > np.sqrt(128) * 0.15
    assert np.abs(X[noise].mean()) < 0.01 and abs(X[noise].std() - 1) < 0.01
    # pages are distinct and the pool does not repeat
    flat = bits.numpy().reshape(n, -1)
    assert len({row.tobytes() for row in flat}) == n
    # deterministic for a seed, pool size and chunk size
    assert torch.equal(synth.compression_pool_device(n, device="cpu", chunk=512), bits)
