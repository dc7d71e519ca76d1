"""CPU tests of the INT4 factor format (PuzzleKV Sec. 4.3) at the C-ABI:
host packing and unpacking, the documented byte layout of a part (re-derived
here from the description in pkv_internal.h, not from the library), cache
layout sizes against the pages' byte count, argument validation, and the
nibble -> bf16 operand identity the attention kernel relies on.  No device
compute is called."""
import ctypes
import os

import numpy as np
import pytest

import oracle
import long_context_decode_pkv_amd as pkv


@pytest.fixture(scope="session", autouse=True)
def _built():
    if not os.path.exists(pkv.LIB_PATH):
        from long_context_decode_pkv_amd import build
        build.build()


RANKS = [1, 6, 8, 14, 16, 20, 24, 31, 32]


def _bf16_values(g, shape):
    """Random positive scales that are exact bfloat16 values."""
    return oracle.round_to(np.exp(g.normal(-3.0, 1.0, shape)), "bf16").astype(np.float32)


def _random_part(g, kind, r, P=64):
    Lq = g.integers(-7, 8, (P, r)).astype(np.int8)
    Rq = g.integers(-7, 8, (r, 128)).astype(np.int8)
    Ls = _bf16_values(g, r if kind == pkv.KEYS else P)
    Rs = _bf16_values(g, 128)
    return Lq, Ls, Rq, Rs


@pytest.mark.parametrize("P", [64, 32])
@pytest.mark.parametrize("r", RANKS)
@pytest.mark.parametrize("kind", [pkv.KEYS, pkv.VALUES])
def test_int4_pack_unpack_round_trip(kind, r, P):
    g = np.random.default_rng(100 * r + kind + P)
    Lq, Ls, Rq, Rs = _random_part(g, kind, r, P)
    packed = pkv.pack_factors_int4(kind, r, Lq, Ls, Rq, Rs, P=P)
    assert packed.size == pkv.factor_part_bytes(kind, r, pkv.BF16_INT4, P=P)
    # every code nibble of the part is used once: a part of codes 0 (nibble
    # 8) and zero scales differs from this one at each code position
    L2, Ls2, R2, Rs2 = pkv.unpack_factors_int4(kind, r, packed, P=P)
    np.testing.assert_array_equal(L2, Lq)
    np.testing.assert_array_equal(R2, Rq)
    np.testing.assert_array_equal(Ls2, Ls)
    np.testing.assert_array_equal(Rs2, Rs)


# -- the documented layout, written out independently ------------------------

def _dims(r):
    n8 = -(-r // 8)
    A = 2 * n8
    full, part = A // 4, int(A % 4 != 0)
    ub = A // 2  # a rank unit: A codes, one nibble each
    return n8, A, full, part, ub


def _tile_row(r, i, qk):
    _, A, _, _, _ = _dims(r)
    b, a = divmod(i, A)
    mt, v = divmod(a, 4)
    partial = 4 * mt + 4 > A
    return mt, (qk * 8 + b * 2 + v) if partial else (16 * qk + 4 * b + v)


def _nib(W, e):
    return 4 * ((e % 2) * (W // 2) + e // 2)


def _code_slots(kind, r):
    """{(factor, row, col): (byte, bit)} for every code of a part, from the
    layout description: factor 'L' (Lt, P x r) or 'R' (Rt, r x d)."""
    _, A, full, part, ub = _dims(r)
    slots = {}
    if kind == pkv.KEYS:
        k2 = full * 1024 + part * 512
        for i in range(r):
            for c in range(128):  # K1: Rt_K rank tiles, dwords [tile][lane][ks]
                ks, qk, e = c // 32, (c % 32) // 8, c % 8
                mt, row = _tile_row(r, i, qk)
                byte = mt * 1024 + (row * 4 + ks) * 4
                slots[("R", i, c)] = (byte + _nib(8, e) // 8, _nib(8, e) % 8)
            for j in range(64):  # K2: Lt_K units [lane][mt]
                lane = 16 * (i // A) + 4 * (j // 16) + j % 4
                mt = (j % 16) // 4
                bit = _nib(2 * ub, i % A)
                slots[("L", j, i)] = (k2 + (lane * 4 + mt) * ub + bit // 8, bit % 8)
    else:
        v2 = full * 512 + part * 256
        for i in range(r):
            for j in range(64):  # V1: Lt_V^T rank tiles, dwords [tile][lane][ks]
                qk, ks, e = j // 16, (j % 16) // 8, j % 8
                mt, row = _tile_row(r, i, qk)
                byte = mt * 512 + (row * 2 + ks) * 4
                slots[("L", j, i)] = (byte + _nib(8, e) // 8, _nib(8, e) % 8)
            for c in range(128):  # V2: Rt_V^T units [lane][mt]
                lane = 16 * (i // A) + c % 16
                mt = c // 16
                bit = _nib(2 * ub, i % A)
                slots[("R", i, c)] = (v2 + (lane * 8 + mt) * ub + bit // 8, bit % 8)
    return slots


def _scale_bytes(kind, r):
    """{(factor, index): byte offset} of every scale."""
    n8, A, full, part, ub = _dims(r)
    out = {}
    if kind == pkv.KEYS:
        srk = full * 1024 + part * 512 + 256 * ub
        for c in range(128):
            out[("R", c)] = srk + 2 * c
        for i in range(8 * n8):
            out[("L", i)] = srk + 256 + 2 * i
    else:
        slv = full * 512 + part * 256 + 512 * ub
        for j in range(64):
            out[("L", j)] = slv + 2 * j
        for c in range(128):
            out[("R", c)] = slv + 128 + 2 * (((c % 16) // 4) * 32 + (c // 16) * 4 + c % 4)
    return out


@pytest.mark.parametrize("r", RANKS)
@pytest.mark.parametrize("kind", [pkv.KEYS, pkv.VALUES])
def test_int4_part_follows_documented_layout(kind, r):
    g = np.random.default_rng(7 * r + kind)
    Lq, Ls, Rq, Rs = _random_part(g, kind, r)
    packed = pkv.pack_factors_int4(kind, r, Lq, Ls, Rq, Rs)
    slots = _code_slots(kind, r)
    assert len(set(slots.values())) == len(slots)  # no two codes share a nibble
    used = np.zeros(packed.size * 2, bool)  # nibble map
    for (f, a, b), (byte, bit) in slots.items():
        code = Lq[a, b] if f == "L" else Rq[a, b]
        assert (packed[byte] >> bit) & 0xF == code + 8, (f, a, b)
        used[2 * byte + bit // 4] = True
    bits = packed.view(np.uint8)
    for (f, idx), byte in _scale_bytes(kind, r).items():
        want = (Ls[idx] if idx < Ls.size else 0.0) if f == "L" else Rs[idx]
        got = (int(bits[byte]) | (int(bits[byte + 1]) << 8)) << 16
        assert np.frombuffer(np.uint32(got).tobytes(), np.float32)[0] == want, (f, idx)
        assert not used[2 * byte: 2 * byte + 4].any()
        used[2 * byte: 2 * byte + 4] = True
    # every other nibble is padding holding code 0
    nib = np.stack([bits & 0xF, bits >> 4], axis=1).reshape(-1)
    assert np.all(nib[~used] == 8)


def test_int4_part_sizes_against_the_pages_count():
    """For r a multiple of 8 (r = 8 .. 32; 24 in 3-byte rank units) a part
    holds exactly the pages' (P + d) r / 2 code bytes plus its 16-bit scales
    (keys: d + r, values: P + d), rounded up to 64 bytes."""
    for r in (8, 16, 24, 32):
        codes = (64 + 128) * r // 2
        k = pkv.factor_part_bytes(pkv.KEYS, r, pkv.BF16_INT4)
        v = pkv.factor_part_bytes(pkv.VALUES, r, pkv.BF16_INT4)
        assert k == -(-(codes + 2 * (128 + r)) // 64) * 64, r
        assert v == -(-(codes + 2 * (64 + 128)) // 64) * 64, r
    # the qwen-shaped rank 24: 5312 bytes per page pair (the pages' count:
    # 5296, before the 64-byte rounding of the key part) against 18432 for bf16
    assert pkv.factor_part_bytes(pkv.KEYS, 24, pkv.BF16_INT4) + \
        pkv.factor_part_bytes(pkv.VALUES, 24, pkv.BF16_INT4) == 5312
    assert 2 * pkv.factor_part_bytes(pkv.KEYS, 24, pkv.BF16) == 18432


def test_int4_part_sizes_of_32_token_pages():
    """P = 32 parts hold the (32 + d) r / 2 code bytes of the pages' count
    for r = 16, 32 (no compacted tile) plus the 16-bit scales, rounded up to
    64 bytes."""
    for r in (16, 32):
        codes = (32 + 128) * r // 2
        k = pkv.factor_part_bytes(pkv.KEYS, r, pkv.BF16_INT4, P=32)
        v = pkv.factor_part_bytes(pkv.VALUES, r, pkv.BF16_INT4, P=32)
        assert k == -(-(codes + 2 * (128 + r)) // 64) * 64
        assert v == -(-(codes + 2 * (32 + 128)) // 64) * 64


def test_int4_cache_at_the_pages_operating_point():
    """P = 32, (r_K, r_V) = (16, 14), one sink page and one window page: the
    whole cache comes within the part padding (r_V padded to 16, parts to 64
    bytes) of the pages' INT4 accounting, 0.187 at long contexts (oracle,
    pinned against the printed figure)."""
    T, rk, rv = 16384, 16, 14
    lay = pkv.cache_layout(pkv.make_shape(batch=1, n_q_heads=8, n_kv_heads=1, rank_k=rk, rank_v=rv, sink=32,
                                          window=32, max_tokens=T, dtype=pkv.BF16_INT4, page_len=32))
    assert lay["factor_k_bytes"] == pkv.factor_part_bytes(pkv.KEYS, rk, pkv.BF16_INT4, P=32)
    assert lay["factor_v_bytes"] == pkv.factor_part_bytes(pkv.VALUES, rv, pkv.BF16_INT4, P=32)
    n_pages = T // 32
    dense = 2 * 32 * 128 * 2
    ours = (lay["max_fact_pages"] * lay["factor_page_bytes"] + 2 * dense) / (n_pages * dense)
    ref = oracle.int4_storage_ratio(T, 32, 128, rk, rv, 2)
    assert ref <= ours <= ref * 1.12, (ours, ref)
    # unequal padded ranks: each part in its own rank's layout
    lay = pkv.cache_layout(pkv.make_shape(1, 8, 1, 8, 24, 32, 32, T, pkv.BF16_INT4, page_len=32))
    assert lay["factor_k_bytes"] == pkv.factor_part_bytes(pkv.KEYS, 8, pkv.BF16_INT4, P=32)
    assert lay["factor_v_bytes"] == pkv.factor_part_bytes(pkv.VALUES, 24, pkv.BF16_INT4, P=32)
    assert lay["factor_page_bytes"] == lay["factor_k_bytes"] + lay["factor_v_bytes"]


def test_int4_cache_layout_and_storage_ratio():
    """An INT4 cache: bf16 dense pages, parts of pkv_factor_part_bytes; at the
    pages' operating point (r_K, r_V) = (16, 14) its whole-cache storage comes
    within the part padding of the pages' 0.187 accounting (oracle)."""
    T, rk, rv = 16384, 16, 14
    sh = pkv.make_shape(batch=1, n_q_heads=8, n_kv_heads=1, rank_k=rk, rank_v=rv, sink=64,
                        window=64, max_tokens=T, dtype=pkv.BF16_INT4)
    lay = pkv.cache_layout(sh)
    assert lay["elem_bytes"] == 2
    assert lay["factor_k_bytes"] == pkv.factor_part_bytes(pkv.KEYS, rk, pkv.BF16_INT4)
    assert lay["factor_v_bytes"] == pkv.factor_part_bytes(pkv.VALUES, rv, pkv.BF16_INT4)
    assert lay["factor_page_bytes"] == lay["factor_k_bytes"] + lay["factor_v_bytes"]
    n_pages = T // 64
    dense = 2 * 64 * 128 * 2
    ours = (lay["max_fact_pages"] * lay["factor_page_bytes"] + 2 * dense) / (n_pages * dense)
    # P = 64 here; the pages' ratio is quoted at P = 32, so compare like with like
    ref = oracle.int4_storage_ratio(T, 64, 128, rk, rv, 2)
    assert ref <= ours <= ref * 1.12, (ours, ref)


def test_int4_validation_without_gpu():
    L = pkv.lib()
    for r, st in ((33, 2), (64, 2)):
        with pytest.raises(pkv.PKVError) as ei:
            pkv.cache_layout(pkv.make_shape(1, 8, 1, r, 16, 64, 128, 4096, pkv.BF16_INT4))
        assert ei.value.status == st
        with pytest.raises(pkv.PKVError) as ei:
            pkv.factor_part_bytes(pkv.KEYS, r, pkv.BF16_INT4)
        assert ei.value.status == st
    g = np.random.default_rng(3)
    Lq, Ls, Rq, Rs = _random_part(g, pkv.KEYS, 8)
    Lq[3, 2] = 8  # outside -7..7
    with pytest.raises(pkv.PKVError) as ei:
        pkv.pack_factors_int4(pkv.KEYS, 8, Lq, Ls, Rq, Rs)
    assert ei.value.status == 1
    n = ctypes.c_int64()
    assert L.pkv_factor_part_bytes(5, 64, 128, 8, pkv.BF16_INT4, ctypes.byref(n)) == 1
    assert L.pkv_pack_factors_int4(0, 64, 128, 8, None, None, None, None, None) == 1


def test_nibble_operand_identity():
    """The attention kernel turns code nibbles n = c + 8 into matrix-core
    operands by an and-or: bf16 bits 0x3f80 | (n << 3) (n in mantissa bits
    3..6 of 1.0) is exactly 1 + n/16 = 1.5 + c/16; the pair of elements
    (2k, 2k + 1) of a packed dword is ((u << 3) >> 4k) & 0x00780078 | 0x3f803f80."""
    n = np.arange(16, dtype=np.uint32)
    bits = (0x3F80 | (n << 3)).astype(np.uint32) << 16
    vals = bits.view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(vals, 1.5 + (n.astype(np.float64) - 8) / 16)
    g = np.random.default_rng(11)
    codes = g.integers(-7, 8, (1000, 8))
    # a dword unit of 8 codes, element e at bit 4 ((e % 2) 4 + e // 2)
    u = np.zeros(1000, np.uint64)
    for e in range(8):
        u |= (codes[:, e] + 8).astype(np.uint64) << np.uint64(_nib(8, e))
    u = u.astype(np.uint32)
    for k in range(4):
        sh = (u << np.uint32(3)) if k == 0 else (u >> np.uint32(4 * k - 3))
        w = (sh & np.uint32(0x00780078)) | np.uint32(0x3F803F80)
        lo = (w << np.uint32(16)).view(np.float32).astype(np.float64)
        hi = (w & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
        np.testing.assert_array_equal(lo, 1.5 + codes[:, 2 * k] / 16)
        np.testing.assert_array_equal(hi, 1.5 + codes[:, 2 * k + 1] / 16)
