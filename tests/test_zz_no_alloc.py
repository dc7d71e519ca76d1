"""pkv_decode_attn_noalloc: decode attention with the library-held workspace
(for callers that cannot allocate).  Called through the C-ABI (ctypes
binding) and checked bit for bit against pkv_decode_attn with the caller's
workspace and the same split count, on two calls in a row -- the second on a
smaller cache, so it runs over the first call's leftover workspace contents --
and against the oracle at the bf16 tolerance.  A split count whose workspace
exceeds the library's array is refused before any device work."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _cache_and_query(T, B, kv_heads):
    d = synth.decode_inputs(2, T=T, B=B, kv_heads=kv_heads, with_f64=True)
    cache = make_cache(d)
    cache.prefill(to_dev(d["K"], "bf16"), to_dev(d["V"], "bf16"))
    return d, cache, to_dev(d["q"], "bf16")


@pytest.mark.parametrize("n_split", [0, 3])
def test_noalloc_matches_decode_attn_on_two_calls(n_split):
    import torch
    require_gpu()
    # first call: the larger cache (2 sequences x 4 KV heads, 37 pages)
    # second call: a smaller one (1 sequence x 2 KV heads, 19 pages)
    for T, B, H in ((64 * 36 + 17, 2, 4), (64 * 18 + 5, 1, 2)):
        d, cache, q = _cache_and_query(T, B, H)
        print(f"[noalloc] T={T} B={B} H_kv={H} n_split={n_split}", flush=True)
        ref = cache.decode(q, n_split=n_split)  # caller's workspace
        out = torch.full_like(ref, float("nan"))
        cache.decode_noalloc(q, out, n_split=n_split)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (T, B, H, n_split)
        o_ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, 64, d["cfg"]["s"], d["cfg"]["w"],
                              d["cfg"]["r_k"], d["cfg"]["r_v"], "bf16")["o_stored"]
        err = rel_err(to_f64(out), o_ref)
        print(f"[noalloc] vs oracle: {err:.3e}", flush=True)
        assert err <= TOL["bf16"]


def test_noalloc_refuses_a_workspace_beyond_its_array():
    import torch
    require_gpu()
    # 8 sequences x 32 query heads x 512 splits: 64 MiB of partial states,
    # above the library's array
    d, cache, q = _cache_and_query(64 * 4, 8, 8)
    need = cache.workspace_bytes(512)
    assert need > pkv.NOALLOC_WORKSPACE_BYTES
    out = torch.zeros((8, 8 * d["G"], 128), dtype=torch.float32, device="cuda:0")
    st = pkv.lib().pkv_decode_attn_noalloc(cache._h, ctypes.c_void_p(q.data_ptr()),
                                           ctypes.c_void_p(out.data_ptr()), 512,
                                           pkv._stream(cache.device))
    assert st == 3  # PKV_ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0  # nothing was launched
    # the largest count that fits still works and matches the caller's workspace
    ns = max(n for n in range(1, 513) if cache.workspace_bytes(n) <= pkv.NOALLOC_WORKSPACE_BYTES)
    assert cache.workspace_bytes(ns + 1) > pkv.NOALLOC_WORKSPACE_BYTES
    ref = cache.decode(q, n_split=ns)
    cache.decode_noalloc(q, out, n_split=ns)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert not np.isnan(to_f64(out)).any()
