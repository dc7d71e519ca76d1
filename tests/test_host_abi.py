"""CPU tests of the C-ABI library: it loads without a GPU, exports every
symbol include/pkv.h declares, and its host-only logic (classification, slot
policy, packed factor layout, storage accounting, argument validation) agrees
with the oracle or with closed forms.  No device compute is called here."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import oracle
import long_context_decode_pkv_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session", autouse=True)
def _built():
    if not os.path.exists(pkv.LIB_PATH):
        from long_context_decode_pkv_amd import build
        build.build()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 15
    L = ctypes.CDLL(pkv.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_classify_matches_oracle_exhaustive():
    for P in (16, 32, 64):
        for s, w in itertools.product((0, P, 2 * P), (0, P, 2 * P, 3 * P)):
            for T in list(range(0, 12 * P + 3)) + [64 * P + 1, 100 * P]:
                cls, slot = pkv.classify(T, P, s, w)
                ocls, oslot = oracle.classify(T, P, s, w)
                np.testing.assert_array_equal(cls, ocls, err_msg=f"{T} {P} {s} {w}")
                np.testing.assert_array_equal(slot, oslot, err_msg=f"{T} {P} {s} {w}")


def test_classify_pending_state_matches_oracle():
    P, s, w = 64, 64, 128
    for T in (8192 + 64 * k for k in range(1, 4)):
        steady = (T // P) - 1 - 2
        cls, slot = pkv.classify(T, P, s, w, n_fact=steady - 1)
        ocls, oslot = oracle.classify(T, P, s, w, n_fact=steady - 1)
        np.testing.assert_array_equal(cls, ocls)
        np.testing.assert_array_equal(slot, oslot)


def test_classify_rejects_bad_arguments():
    with pytest.raises(pkv.PKVError):
        pkv.classify(100, 64, 32, 128)
    with pytest.raises(pkv.PKVError):
        pkv.classify(100, 64, 64, 100)
    with pytest.raises(pkv.PKVError):
        pkv.classify(-1, 64, 64, 128, n_pages=1)


def test_storage_ratio_is_eq3_and_agrees_with_oracle():
    for P, rk, rv, d in ((32, 16, 14, 128), (64, 16, 16, 128), (64, 24, 24, 128), (16, 9, 9, 128)):
        assert abs(pkv.storage_ratio(P, rk, rv, d) - oracle.storage_ratio(P, rk, rv, d)) < 1e-15


def _part_elems(kind, r, P):
    """Key parts r8 (P + d); value parts r8 P + r2 d, their Rf at r rounded
    up to even (r8 above 32)."""
    r8 = -(-r // 8) * 8
    r2 = r + r % 2 if r8 <= 32 else r8
    return r8 * P + r2 * 128 if kind == pkv.VALUES else r8 * (P + 128)


@pytest.mark.parametrize("r", [1, 7, 8, 10, 13, 14, 16, 20, 24, 25, 30, 32, 40, 48, 56, 64])
def test_packed_layout_is_a_bijection(r):
    """Every (operand, row, col) of the two factor parts maps to a distinct
    slot inside the part (value parts at their exact, even-rounded rank),
    and pack and unpack are inverse."""
    r8 = -(-r // 8) * 8
    for kind in (pkv.KEYS, pkv.VALUES, pkv.KEYS_PRE_ROPE):
        n = pkv.factor_part_elems(kind, r)
        assert n == _part_elems(kind, r, 64)
        # encode each entry's identity in its value, pack, and check coverage
        Lf = np.arange(64 * r8, dtype=np.float32).reshape(64, r8)[:, :r] + 1
        Rf = np.arange(r8 * 128, dtype=np.float32).reshape(r8, 128)[:r] + 1 + 64 * r8
        packed = pkv.pack_factors(kind, r, pkv.F32, Lf, Rf)
        assert packed.size == n
        vals = packed[packed != 0]
        assert len(np.unique(vals)) == len(vals) == 64 * r + r * 128
        Lb, Rb = pkv.unpack_factors(kind, r, pkv.F32, packed)
        np.testing.assert_array_equal(Lb, Lf)
        np.testing.assert_array_equal(Rb, Rf)


def test_pack_bf16_rounds_nearest_even():
    g = np.random.default_rng(0)
    r = 24
    Lf = g.standard_normal((64, r)).astype(np.float32)
    Rf = g.standard_normal((r, 128)).astype(np.float32)
    packed = pkv.pack_factors(pkv.KEYS, r, pkv.BF16, Lf, Rf)
    Lb, Rb = pkv.unpack_factors(pkv.KEYS, r, pkv.BF16, packed)
    np.testing.assert_array_equal(Lb, oracle.round_to(Lf, "bf16").astype(np.float32))
    np.testing.assert_array_equal(Rb, oracle.round_to(Rf, "bf16").astype(np.float32))


def test_operand_order_of_packed_parts():
    """Spot-check the documented lane order: K part starts with Rf_K tile 0,
    reduction step 0, lane l -> row l % 16 (rank 2*n8*(l%16//4) + l%4),
    channels 8*(l//16) .. +7."""
    r = 24  # n8 = 3, six ranks per lane quad
    Lf = np.zeros((64, r), np.float32)
    Rf = np.arange(r * 128, dtype=np.float32).reshape(r, 128)
    packed = pkv.pack_factors(pkv.KEYS, r, pkv.F32, Lf, Rf)
    for lane in (0, 5, 17, 63):
        rho, qk = lane % 16, lane // 16
        rank = 6 * (rho // 4) + rho % 4
        np.testing.assert_array_equal(packed[lane * 8: lane * 8 + 8], Rf[rank, 8 * qk: 8 * qk + 8])


def _shape(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, rank_k=16, rank_v=16, sink=64, window=128,
                max_tokens=4096, dtype=pkv.BF16)
    base.update(kw)
    return pkv.make_shape(**base)


def test_layout_sizes():
    lay = pkv.cache_layout(_shape())
    assert lay["max_pages"] == 64
    assert lay["max_fact_pages"] == 64 - 1 - 2
    assert lay["factor_page_bytes"] == 2 * (16 * 192) * 2
    assert lay["dense_page_bytes"] == 64 * 128 * 2
    for k in ("sink_k", "sink_v", "win_k", "win_v", "factors", "page_table", "total_bytes"):
        assert lay[k] % 256 == 0
    assert lay["factors"] >= lay["win_v"] + 2 * 2 * 3 * lay["dense_page_bytes"]
    assert lay["total_bytes"] >= lay["page_table"] + 4 * lay["max_pages"]


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 2), (dict(page_len=16), 2),
    (dict(page_len=128, sink=128, window=128), 2), (dict(page_len=32, rank_k=33), 1), (dict(n_q_heads=32, n_kv_heads=2), 2),
    (dict(sink=32), 1), (dict(window=100), 1), (dict(rank_k=0), 1), (dict(rank_v=65), 1),
    (dict(n_q_heads=7), 1), (dict(max_tokens=0), 1), (dict(dtype=5), 1),
])
def test_layout_validation(kw, status):
    with pytest.raises(pkv.PKVError) as ei:
        pkv.cache_layout(_shape(**kw))
    assert ei.value.status == status


def test_layout_of_32_token_pages():
    """P = 32 (the pages' default page length) at (r_K, r_V) = (16, 14): the
    key part holds r8 (P + d) elements, the value part r8 P + r2 d with its
    Rf_V at the exact rank 14 (only Lf_V^T keeps two zero rank rows).  A
    factorized page pair then takes 0.594 of its dense bytes, against Sec. 3.3
    Eq. 3's 0.586 at (16, 14) and 0.625 with both ranks padded to 16."""
    lay = pkv.cache_layout(_shape(page_len=32, rank_k=16, rank_v=14, sink=32, window=32))
    assert lay["dense_page_bytes"] == 32 * 128 * 2
    assert lay["factor_k_elems"] == 16 * (32 + 128) and lay["factor_v_elems"] == 16 * 32 + 14 * 128
    assert lay["max_pages"] == 4096 // 32 and lay["max_fact_pages"] == 4096 // 32 - 2
    ratio = lay["factor_page_bytes"] / (2 * lay["dense_page_bytes"])
    assert ratio == (16 * 160 + 16 * 32 + 14 * 128) / (2 * 32 * 128) == 0.59375
    assert pkv.storage_ratio(32, 16, 16, 128) == 0.625
    assert abs(pkv.storage_ratio(32, 16, 14, 128) - 0.586) < 5e-4


@pytest.mark.parametrize("r", [1, 7, 8, 10, 13, 14, 16, 20, 24, 25, 30, 32])
def test_packed_layout_of_32_token_pages_is_a_bijection(r):
    """Every (operand, row, col) of a P = 32 part maps to a distinct slot,
    and pack and unpack are inverse."""
    P = 32
    r8 = -(-r // 8) * 8
    for kind in (pkv.KEYS, pkv.VALUES, pkv.KEYS_PRE_ROPE):
        n = pkv.factor_part_elems(kind, r, P)
        assert n == _part_elems(kind, r, P)
        Lf = np.arange(P * r8, dtype=np.float32).reshape(P, r8)[:, :r] + 1
        Rf = np.arange(r8 * 128, dtype=np.float32).reshape(r8, 128)[:r] + 1 + P * r8
        packed = pkv.pack_factors(kind, r, pkv.F32, Lf, Rf, P=P)
        assert packed.size == n
        vals = packed[packed != 0]
        assert len(np.unique(vals)) == len(vals) == P * r + r * 128
        Lb, Rb = pkv.unpack_factors(kind, r, pkv.F32, packed, P=P)
        np.testing.assert_array_equal(Lb, Lf)
        np.testing.assert_array_equal(Rb, Rf)
        assert pkv.factor_part_bytes(kind, r, pkv.BF16, P=P) == 2 * n
    L = pkv.lib()
    nb = ctypes.c_int64()
    assert L.pkv_factor_part_bytes(pkv.KEYS, P, 128, r, pkv.BF16_INT4, ctypes.byref(nb)) == 0
    assert nb.value == pkv.factor_part_bytes(pkv.KEYS, r, pkv.BF16_INT4, P=P)  # INT4 parts at P = 32
    assert L.pkv_factor_part_elems(pkv.VALUES, P, 128, P + 1, ctypes.byref(nb)) == 1
    assert L.pkv_factor_part_elems(pkv.KEYS, 16, 128, 8, ctypes.byref(nb)) == 2
    assert L.pkv_factor_part_elems(7, P, 128, 8, ctypes.byref(nb)) == 1  # no such kind


def test_operand_order_of_32_token_parts():
    """Spot-check the compacted operands of a P = 32 part against the P = 64
    order: K1 and V2 (rank x channel) are the same; K2 keeps lane
    lam = 8 (l // 16) + l % 16 of the lanes l % 16 < 8, V1 lanes 0..31."""
    r = 16  # n8 = 2: A = 4 ranks per lane quad, one rank tile
    g = np.random.default_rng(5)
    Lf32 = g.standard_normal((32, r)).astype(np.float32)
    Rf = g.standard_normal((r, 128)).astype(np.float32)
    Lf64 = np.concatenate([Lf32, np.zeros((32, r), np.float32)])
    for kind in (pkv.KEYS, pkv.VALUES):
        p32 = pkv.pack_factors(kind, r, pkv.F32, Lf32, Rf, P=32)
        p64 = pkv.pack_factors(kind, r, pkv.F32, Lf64, Rf)
        if kind == pkv.KEYS:
            k1 = 16 * 128
            np.testing.assert_array_equal(p32[:k1], p64[:k1])
            A = 4
            for mt in range(4):
                t32 = p32[k1 + mt * 32 * A: k1 + (mt + 1) * 32 * A].reshape(32, A)
                t64 = p64[k1 + mt * 64 * A: k1 + (mt + 1) * 64 * A].reshape(64, A)
                keep = [l for l in range(64) if l % 16 < 8]
                np.testing.assert_array_equal(t32, t64[keep])
                assert not t64[[l for l in range(64) if l % 16 >= 8]].any()
        else:
            v1_32, v1_64 = 16 * 32, 16 * 64
            t32 = p32[:v1_32].reshape(2, 32, 8)
            t64 = p64[:v1_64].reshape(2, 64, 8)
            np.testing.assert_array_equal(t32, t64[:, :32])
            assert not t64[:, 32:].any()
            np.testing.assert_array_equal(p32[v1_32:], p64[v1_64:])


def test_create_validation_without_gpu():
    L = pkv.lib()
    sh = _shape()
    lay = pkv.cache_layout(sh)
    h = ctypes.c_void_p()
    # misaligned buffer pointer and a buffer that is too small
    assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 1000 + 8), lay["total_bytes"],
                              ctypes.byref(h)) == 1
    assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 1000), lay["total_bytes"] - 1,
                              ctypes.byref(h)) == 3
    # a handle over a fake address: host-side state calls work, no GPU touched
    assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 1000), lay["total_bytes"],
                              ctypes.byref(h)) == 0
    T, nf, pend = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    assert L.pkv_cache_state(h, ctypes.byref(T), ctypes.byref(nf), ctypes.byref(pend)) == 0
    assert (T.value, nf.value, pend.value) == (0, 0, 0)
    assert L.pkv_promote_page(h, None) == 4          # nothing waiting
    assert L.pkv_prefill(h, None, None, 10, None) == 1
    assert L.pkv_prefill(h, ctypes.c_void_p(4096), ctypes.c_void_p(4096), 5000, None) == 3
    ws = ctypes.c_uint64()
    assert L.pkv_decode_workspace_bytes(h, 4, ctypes.byref(ws)) == 0
    assert ws.value >= 2 * 8 * 4 * 130 * 4
    # empty cache: attention is refused before any launch
    assert L.pkv_decode_attn(h, ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                             ws.value, 4, None) == 1
    assert L.pkv_cache_set_aux_stream(h, None) == 0  # off by default; clearing is a no-op
    assert L.pkv_cache_set_aux_stream(None, None) == 1
    L.pkv_cache_destroy(h)


def test_compress_validation_without_gpu():
    L = pkv.lib()
    p = ctypes.c_void_p(4096)
    assert L.pkv_compress_pages(p, 4, 16, 128, 8, 0, 0, p, p, None, None) == 2
    assert L.pkv_compress_pages(p, 4, 32, 128, 33, 0, 0, p, p, None, None) == 1
    assert L.pkv_compress_pages(p, 4, 64, 128, 0, 0, 0, p, p, None, None) == 1
    assert L.pkv_compress_pages(p, 4, 64, 128, 65, 0, 0, p, p, None, None) == 1
    assert L.pkv_compress_pages(None, 4, 64, 128, 8, 0, 0, p, p, None, None) == 1
    assert L.pkv_compress_pages(p, 0, 64, 128, 8, 0, 0, p, p, None, None) == 0
    assert L.pkv_compress_pages(ctypes.c_void_p(4098), 4, 64, 128, 8, 0, 0, p, p, None, None) == 1


def test_time_next_kernel_validation_without_gpu():
    """Both handles or neither; a call that launches nothing leaves the
    request pending, and (NULL, NULL) clears it."""
    L = pkv.lib()
    p = ctypes.c_void_p(4096)
    assert L.pkv_time_next_kernel(p, None) == 1
    assert L.pkv_time_next_kernel(None, p) == 1
    assert L.pkv_time_next_kernel(p, p) == 0
    assert L.pkv_compress_pages(p, 0, 64, 128, 8, 0, 0, p, p, None, None) == 0  # no launch
    assert L.pkv_time_next_kernel(None, None) == 0


def test_prefill_chunk_validation_without_gpu():
    """Argument and state checks of pkv_prefill_chunk fire before any launch."""
    L = pkv.lib()
    sh = _shape(max_tokens=256)
    lay = pkv.cache_layout(sh)
    h = ctypes.c_void_p()
    assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 1000), lay["total_bytes"],
                              ctypes.byref(h)) == 0
    fake = ctypes.c_void_p(256 * 5000)
    try:
        assert L.pkv_prefill_chunk(None, fake, fake, 1, None) == 1
        assert L.pkv_prefill_chunk(h, fake, fake, -1, None) == 1
        assert L.pkv_prefill_chunk(h, fake, fake, 0, None) == 0           # nothing to do
        assert L.pkv_prefill_chunk(h, None, fake, 4, None) == 1
        assert L.pkv_prefill_chunk(h, ctypes.c_void_p(256 * 5000 + 2), fake, 4, None) == 1
        assert L.pkv_prefill_chunk(h, fake, fake, 257, None) == 3         # beyond max_tokens
        T, nf, pend = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        assert L.pkv_cache_state(h, ctypes.byref(T), ctypes.byref(nf), ctypes.byref(pend)) == 0
        assert (T.value, nf.value, pend.value) == (0, 0, 0)
    finally:
        L.pkv_cache_destroy(h)


@pytest.mark.parametrize("r", [8, 16, 24, 40])
def test_pre_rope_key_part_is_channel_major(r):
    """A pre-RoPE key part holds Rf_K in the value part's Rf order at its
    start, and Lf_K where a key part holds it."""
    g = np.random.default_rng(r)
    Lf = g.standard_normal((64, r)).astype(np.float32)
    Rf = g.standard_normal((r, 128)).astype(np.float32)
    n8 = -(-r // 8)
    k1 = 8 * n8 * 128  # Rf elements of a part
    pre = pkv.pack_factors(pkv.KEYS_PRE_ROPE, r, pkv.F32, Lf, Rf)
    val = pkv.pack_factors(pkv.VALUES, r, pkv.F32, np.zeros_like(Lf), Rf)
    key = pkv.pack_factors(pkv.KEYS, r, pkv.F32, Lf, np.zeros_like(Rf))
    v1 = 8 * n8 * 64
    np.testing.assert_array_equal(pre[:k1], val[v1:])
    np.testing.assert_array_equal(pre[k1:], key[k1:])
    assert pkv.factor_part_bytes(pkv.KEYS_PRE_ROPE, r, pkv.BF16) == pkv.factor_part_bytes(pkv.KEYS, r, pkv.BF16)


def test_set_key_rope_validation_without_gpu():
    L = pkv.lib()
    f = np.full(64, 0.5, np.float32)
    fp = f.ctypes.data_as(ctypes.c_void_p)
    assert L.pkv_cache_set_key_rope(None, fp, 64) == 1
    for dtype, ok in ((pkv.BF16, 0), (pkv.F32, 0), (pkv.BF16_INT4, 2)):
        sh = _shape(dtype=dtype)
        lay = pkv.cache_layout(sh)
        h = ctypes.c_void_p()
        assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 1000), lay["total_bytes"],
                                  ctypes.byref(h)) == 0
        try:
            assert L.pkv_cache_set_key_rope(h, fp, 64) == ok
            if ok == 0:
                assert L.pkv_cache_set_key_rope(h, fp, 63) == 1
                bad = f.copy()
                bad[7] = np.nan
                assert L.pkv_cache_set_key_rope(h, bad.ctypes.data_as(ctypes.c_void_p), 64) == 1
                assert L.pkv_cache_set_key_rope(h, None, 0) == 0
        finally:
            L.pkv_cache_destroy(h)


def test_batch_validation_without_gpu():
    """pkv_decode_batch_workspace_bytes / pkv_decode_attn_batch reject bad
    batches before any launch: null or out-of-range arguments, empty caches."""
    L = pkv.lib()
    nb = ctypes.c_uint64()
    sh = _shape(batch=1, max_tokens=256)
    lay = pkv.cache_layout(sh)
    h = ctypes.c_void_p()
    assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 1000), lay["total_bytes"],
                              ctypes.byref(h)) == 0
    try:
        hs = (ctypes.c_void_p * 2)(h, h)
        assert L.pkv_decode_batch_workspace_bytes(None, 1, 0, ctypes.byref(nb)) == 1
        assert L.pkv_decode_batch_workspace_bytes(hs, 0, 0, ctypes.byref(nb)) == 1
        assert L.pkv_decode_batch_workspace_bytes(hs, 33, 0, ctypes.byref(nb)) == 1
        assert L.pkv_decode_batch_workspace_bytes(hs, 2, 0, None) == 1
        assert L.pkv_decode_batch_workspace_bytes(hs, 2, 0, ctypes.byref(nb)) == 0  # empty caches: sized
        assert nb.value > 0
        fake = ctypes.c_void_p(256 * 5000)
        assert L.pkv_decode_attn_batch(hs, 2, fake, fake, fake, 1 << 20, 0, None) == 1  # nothing to attend
        assert L.pkv_decode_step_batch(hs, 2, None, fake, fake, fake, fake, 1 << 20, 0, None) == 1
        assert L.pkv_decode_step_batch(hs, 2, fake, fake, fake, fake, fake, 16, 0, None) == 3
    finally:
        L.pkv_cache_destroy(h)
