"""Helpers shared by the GPU tests (not a test module)."""
import numpy as np
import pytest

import long_context_decode_pkv_amd as pkv


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    pkv.lib()  # raises loudly if libpkv.so is missing


def to_dev(a, dtype):
    """Stored numpy array (uint16 bf16 bits or float32) -> device tensor."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a.astype(np.float32)).to("cuda:0")


def to_f64(t):
    """Device tensor -> float64 numpy."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor (NaN refs ignored)."""
    m = ~np.isnan(ref)
    return float(np.abs(got[m] - ref[m]).max() / np.abs(ref[m]).max())


def make_cache(d, r_k=None, r_v=None, max_tokens=None, s=None, w=None, store=None, P=64):
    """Cache for decode_inputs d (pages of P tokens); store "int4" keeps INT4
    factor pages (the inputs' dtype must then be bf16)."""
    cfg = d["cfg"]
    return pkv.Cache(batch=d["B"], n_q_heads=d["Hq"], n_kv_heads=d["Hkv"],
                     rank_k=cfg["r_k"] if r_k is None else r_k,
                     rank_v=cfg["r_v"] if r_v is None else r_v,
                     sink=cfg["s"] if s is None else s, window=cfg["w"] if w is None else w,
                     max_tokens=max_tokens or d["T"], dtype=store or cfg["dtype"], page_len=P)


# Tolerances (relative to max |o_ref| over the tensor): bf16 storage 1e-2,
# fp32 storage 1e-4; INT4 factor pages against the oracle's own INT4 factors,
# the bf16 gate (the two sides may round a code differently where the exact
# factor sits on a rounding boundary).
TOL = {"bf16": 1e-2, "f32": 1e-4, "int4": 1e-2}


def valid_dense_rows(cache, T):
    """{(b, h, page): (K rows, V columns)} of every dense page's valid rows."""
    import torch
    L, sh = cache.layout, cache.shape
    B, H, P, d = sh.batch, sh.n_kv_heads, sh.page_len, 128
    esz = L["elem_bytes"]
    n_s, ring = L["n_sink_slots"], L["n_ring_slots"]
    cls, slot = cache.page_table(-(-T // P))
    buf = cache.buffer
    out = {}
    for p in range(len(cls)):
        if cls[p] == pkv.FACT:
            continue
        nv = min(P, T - p * P)
        for b in range(B):
            for h in range(H):
                if cls[p] == pkv.SINK:
                    base_k = L["sink_k"] + ((b * H + h) * n_s + slot[p]) * P * d * esz
                    base_v = L["sink_v"] + ((b * H + h) * n_s + slot[p]) * P * d * esz
                else:
                    base_k = L["win_k"] + ((b * H + h) * ring + slot[p]) * P * d * esz
                    base_v = L["win_v"] + ((b * H + h) * ring + slot[p]) * P * d * esz
                k = buf[base_k: base_k + P * d * esz].view(P, d * esz)[:nv].clone()
                v = buf[base_v: base_v + P * d * esz].view(d, P * esz)[:, :nv * esz].clone()
                out[(b, h, p)] = (k, v)
    torch.cuda.synchronize()
    return out


def assert_same_cache(a, b, label):
    """Two caches agree exactly: host state, page table, every factorized
    page's packed factors and every valid dense row."""
    import torch
    assert a.state() == b.state(), (label, a.state(), b.state())
    T, nf, _ = a.state()
    n = -(-T // a.shape.page_len)
    for x, y in zip(a.page_table(n), b.page_table(n)):
        np.testing.assert_array_equal(x, y, err_msg=label)
    L, sh = a.layout, a.shape
    for bb in range(sh.batch):
        for h in range(sh.n_kv_heads):
            for f in range(nf):
                for kind in (pkv.KEYS, pkv.VALUES):
                    assert torch.equal(a.factor_part(bb, h, f, kind), b.factor_part(bb, h, f, kind)), \
                        (label, bb, h, f, kind)
    da, db = valid_dense_rows(a, T), valid_dense_rows(b, T)
    assert da.keys() == db.keys()
    for key in da:
        assert torch.equal(da[key][0], db[key][0]) and torch.equal(da[key][1], db[key][1]), (label, key)
