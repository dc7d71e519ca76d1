"""The size formulas include/pkv.h states, restated here, against what the
library returns (host only): factor part elements and bytes in every
storage format, the INT4 part sizes, the cache layout's regions, and the
decode workspace -- at both page lengths and every rank."""
import ctypes

import pytest

import long_context_decode_pkv_amd as pkv

D = 128


def roundup(x, a):
    return -(-x // a) * a


def r8(r):
    return 8 * (-(-r // 8))


def r2(r):
    """Ranks a value part's Rf operand stores: r rounded up to even up to
    r8 = 32, r8 above."""
    return r + r % 2 if r8(r) <= 32 else r8(r)


def part_elems(kind, P, r):
    return r8(r) * P + r2(r) * D if kind == pkv.VALUES else r8(r) * (P + D)


def int4_part_bytes(kind, P, r):
    """The INT4 part sizes as the header gives them at pkv_factor_part_bytes."""
    A = r8(r) // 4
    ub = A // 2  # a rank unit: A codes, one nibble each
    h = 1 if P == 64 else 2
    if kind == pkv.VALUES:
        return roundup(r8(r) * P // 2 + 4 * D * ub + 2 * P + 2 * D, 64)
    return roundup(r8(r) * D // 2 + (256 // h) * ub + 2 * D + 2 * r8(r), 64)


@pytest.mark.parametrize("P", [32, 64])
def test_factor_part_sizes_follow_the_header(P):
    for r in range(1, P + 1):
        for kind in (pkv.KEYS, pkv.VALUES, pkv.KEYS_PRE_ROPE):
            n = part_elems(kind, P, r)
            assert pkv.factor_part_elems(kind, r, P) == n, (P, r, kind)
            assert pkv.factor_part_bytes(kind, r, pkv.BF16, P=P) == 2 * n
            assert pkv.factor_part_bytes(kind, r, pkv.F32, P=P) == 4 * n
        if r <= 32:
            for kind in (pkv.KEYS, pkv.VALUES):
                assert pkv.factor_part_bytes(kind, r, pkv.BF16_INT4, P=P) == int4_part_bytes(kind, P, r), \
                    (P, r, kind)


@pytest.mark.parametrize("P,dtype", [(P, dt) for P in (32, 64) for dt in (pkv.BF16, pkv.F32, pkv.BF16_INT4)])
def test_cache_layout_follows_the_header(P, dtype):
    B, Hq, H = 3, 12, 2
    for r in range(1, (32 if dtype == pkv.BF16_INT4 else P) + 1):
        for s, w, Tmax in ((P, 2 * P, 40 * P + 7), (0, 0, 5 * P), (2 * P, P, 3 * P - 1)):
            r_v = r  # INT4 at P = 32 needs equal padded ranks
            sh = pkv.make_shape(B, Hq, H, r, r_v, s, w, Tmax, dtype, page_len=P)
            L = pkv.cache_layout(sh)
            esz = 4 if dtype == pkv.F32 else 2
            n_s, n_w = s // P, w // P
            assert L["elem_bytes"] == esz
            assert L["n_sink_slots"] == n_s and L["n_ring_slots"] == n_w + 1
            assert L["max_pages"] == -(-Tmax // P)
            assert L["max_fact_pages"] == max(0, Tmax // P - n_s - n_w)
            assert L["dense_page_bytes"] == P * D * esz
            if dtype == pkv.BF16_INT4:  # (codes: the padded count)
                assert L["factor_k_elems"] == r8(r) * (P + D) and L["factor_v_elems"] == r8(r_v) * (P + D)
                kb, vb = int4_part_bytes(pkv.KEYS, P, r), int4_part_bytes(pkv.VALUES, P, r_v)
            else:
                assert L["factor_k_elems"] == part_elems(pkv.KEYS, P, r)
                assert L["factor_v_elems"] == part_elems(pkv.VALUES, P, r_v)
                kb, vb = part_elems(pkv.KEYS, P, r) * esz, part_elems(pkv.VALUES, P, r_v) * esz
            assert (L["factor_k_bytes"], L["factor_v_bytes"]) == (kb, vb)
            assert L["factor_page_bytes"] == kb + vb
            # regions in order, each starting at the previous end rounded up to 256
            sink = B * H * n_s * P * D * esz
            ring = B * H * (n_w + 1) * P * D * esz
            off = 0
            for name, size in (("sink_k", sink), ("sink_v", sink), ("win_k", ring), ("win_v", ring),
                               ("factors", B * H * L["max_fact_pages"] * (kb + vb)),
                               ("page_table", 4 * L["max_pages"])):
                assert L[name] == off, (name, P, dtype, r, s, w)
                off = roundup(off + size, 256)
            assert L["total_bytes"] == off


def test_decode_workspace_follows_the_header():
    L = pkv.lib()
    for P in (32, 64):
        sh = pkv.make_shape(3, 24, 4, 16, 16, P, 2 * P, 50 * P, pkv.BF16, page_len=P)
        lay = pkv.cache_layout(sh)
        h = ctypes.c_void_p()
        # a handle over a fake address: host-side calls only
        assert L.pkv_cache_create(ctypes.byref(sh), ctypes.c_void_p(256 * 4096), lay["total_bytes"],
                                  ctypes.byref(h)) == 0
        try:
            for ns in (1, 2, 7, 64, 511, 512):
                got = ctypes.c_uint64()
                assert L.pkv_decode_workspace_bytes(h, ns, ctypes.byref(got)) == 0
                rows = 3 * 24 * ns
                assert got.value == roundup(rows * D * 4, 256) + roundup(rows * 2 * 4, 256), (P, ns)
            got = ctypes.c_uint64()
            assert L.pkv_decode_workspace_bytes(h, 513, ctypes.byref(got)) == 1
        finally:
            L.pkv_cache_destroy(h)
