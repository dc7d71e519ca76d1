"""GPU parity of value parts stored at their exact rank.

A bf16 / fp32 value part keeps Rf_V (the V2 operand) at r rounded up to
even, not at r8 = 8 ceil(r / 8), for r8 <= 32: each 16-channel tile holds the
partial lane quad's ranks first, then the full quads (include/pkv.h, the
layout note).  Key parts are unchanged.  The attention kernels read such a
part through each lane's own offset; a slot of a rank the part does not
hold reads a neighbouring entry and meets a zero rank weight (the padded
rank rows of Lf_V^T are zero).

- The decomposition writes that layout: every element of a GPU-written key
  and value part is what the host packer writes for the part's own factors
  (pack(unpack(part)) reproduces the part exactly).
- Attention on the oracle's own bf16 factors written into the pool agrees
  with the oracle's attention over the same factors within 2e-4 max |o_ref|
  (the cfg-3 recipe, sigma_i = i^-1.2: every kept rank shows in the output).
- End to end at the gates of the cache dtype, at P = 64 and 32, on the
  matrix-core kernels (equal and unequal padded ranks, pre-RoPE keys) and
  the vector-ALU path (fp32 storage; pre-RoPE keys at unequal ranks above
  32), including value parts written by the Jacobi route of a cache whose
  key rank is above 32.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu

KIND = {pkv.KEYS: "K", pkv.VALUES: "V"}


def _prefilled(cfg_id, T, r_k, r_v, P, B=1, kv=2, rope=None):
    d = synth.decode_inputs(cfg_id, T=T, B=B, kv_heads=kv, with_f64=True)
    cache = make_cache(d, r_k=r_k, r_v=r_v, P=P, s=P, w=2 * P)
    if rope is not None:
        cache.set_key_rope(rope)
    dt = d["cfg"]["dtype"]
    cache.prefill(to_dev(d["K"], dt), to_dev(d["V"], dt))
    return d, cache


def _fact_pages(d, cache, b, h, kind):
    T, nf, _ = cache.state()
    P = cache.shape.page_len
    n_s = cache.shape.sink // P
    src = d["K64"] if kind == pkv.KEYS else d["V64"]
    return src[b, h, P * n_s: P * (n_s + nf)].reshape(nf, P, 128)


@pytest.mark.parametrize("P,rk,rv", [
    (64, 16, 14), (64, 24, 20), (64, 32, 30), (64, 8, 5), (64, 16, 13),
    (32, 16, 14), (32, 24, 22), (32, 32, 26), (32, 8, 1),
])
def test_gpu_parts_are_the_host_layout(P, rk, rv):
    require_gpu()
    import torch
    d, cache = _prefilled(3, P * 12 + 5, rk, rv, P)
    n_v = pkv.factor_part_elems(pkv.VALUES, rv, P)
    r8 = -(-rv // 8) * 8
    assert n_v == r8 * P + (rv + rv % 2) * 128
    for h in range(2):
        for f in range(cache.state()[1]):
            for kind, r in ((pkv.KEYS, rk), (pkv.VALUES, rv)):
                part = cache.factor_part(0, h, f, kind).cpu().numpy().view(np.uint16)
                torch.cuda.synchronize()
                assert part.size == pkv.factor_part_elems(kind, r, P)
                Lf, Rf = pkv.unpack_factors(kind, r, pkv.BF16, part, P=P)
                again = pkv.pack_factors(kind, r, pkv.BF16, Lf, Rf, P=P)
                np.testing.assert_array_equal(part, again, err_msg=f"h{h} page {f} {KIND[kind]}")


@pytest.mark.parametrize("P,rk,rv,splits", [
    (64, 16, 14, (0, 3)),   # A = 4: partial quad of 2 ranks
    (64, 24, 22, (0, 5)),   # A = 6: partial quad of 4
    (64, 32, 30, (0,)),     # A = 8: partial quad of 6
    (64, 8, 5, (0, 2)),     # A = 2: r2 = 6, the fourth quad empty
    (64, 8, 14, (0,)),      # unequal padded ranks
    (64, 32, 22, (0,)),     # unequal padded ranks (r8 32 / 24)
    (64, 48, 22, (0, 2)),   # key rank above 32: two reduction steps
    (32, 16, 14, (0, 3)),   # the pages' operating point
    (32, 24, 20, (0,)),
    (32, 32, 26, (0, 2)),
    (32, 16, 9, (0,)),      # A = 4: r2 = 10
])
def test_attention_on_oracle_factors(P, rk, rv, splits):
    require_gpu()
    import torch
    T = P * 40 + 17
    d, cache = _prefilled(3, T, rk, rv, P)
    for b in range(d["B"]):
        for h in range(d["Hkv"]):
            for kind, r in ((pkv.KEYS, rk), (pkv.VALUES, rv)):
                X = _fact_pages(d, cache, b, h, kind)
                U, S, Wt = oracle.svd_batch(X)
                Lf, Rf = oracle.stored_factors(U, S, Wt, r, "bf16", KIND[kind])
                for f in range(X.shape[0]):
                    part = pkv.pack_factors(kind, r, pkv.BF16, Lf[f], Rf[f], P=P)
                    cache.factor_part(b, h, f, kind).copy_(torch.from_numpy(part.view(np.uint8)))
    torch.cuda.synchronize()
    cfg = d["cfg"]
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, P, P, 2 * P, rk, rv, cfg["dtype"])
    q = to_dev(d["q"], cfg["dtype"])
    for ns in splits:
        o = to_f64(cache.decode(q, n_split=ns))
        torch.cuda.synchronize()
        err = rel_err(o, ref["o_stored"])
        print(f"[exact-rank oracle factors P={P} r=({rk},{rv}) split={ns}] err={err:.3e}")
        assert err <= 2e-4, (ns, err)


@pytest.mark.parametrize("cfg_id,P,rk,rv,rope", [
    (2, 64, 16, 14, None),
    (2, 32, 16, 14, None),
    (3, 64, 24, 23, None),
    (2, 64, 16, 14, 5e5),    # pre-RoPE keys, matrix-core kernel
    (3, 32, 24, 22, 1e6),    # pre-RoPE keys at 32-token pages
    (2, 64, 48, 13, None),   # key rank above 32: the job's Jacobi route writes the exact-rank value part
    (2, 64, 40, 13, 5e5),    # ... read by the vector-ALU kernel (pre-RoPE, unequal ranks above 32)
    (1, 64, 16, 13, None),   # fp32 storage: vector-ALU kernel
    (1, 32, 16, 13, None),
])
def test_end_to_end_against_oracle(cfg_id, P, rk, rv, rope):
    require_gpu()
    import torch
    T = P * 30 + 9
    freqs = synth.rope_inv_freq(rope) if rope else None
    d, cache = _prefilled(cfg_id, T, rk, rv, P, rope=freqs)
    cfg = d["cfg"]
    ref = oracle.decode(d["q64"], d["K64"], d["V64"], T, P, P, 2 * P, rk, rv, cfg["dtype"], key_rope=freqs)
    q = to_dev(d["q"], cfg["dtype"])
    for ns in (0, 3):
        o = to_f64(cache.decode(q, n_split=ns))
        torch.cuda.synchronize()
        err = rel_err(o, ref["o_stored"])
        print(f"[exact-rank cfg{cfg_id} P={P} r=({rk},{rv}) rope={rope} split={ns}] err={err:.3e}")
        assert err <= TOL[cfg["dtype"]], (ns, err)
