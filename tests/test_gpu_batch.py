"""GPU tests of pkv_decode_attn_batch: attention for a batch of sequences of
different lengths, one cache (own pools, own page table) per sequence.

Row i of the batched result must equal pkv_decode_attn on cache i with the
same split count bit for bit (the same kernel code runs on the same pages),
whatever the format: the batched matrix-core kernels and the per-cache
fallback (fp32, unequal padded ranks, INT4 with unequal ranks).  Against the
oracle each row meets the cache dtype's gate.
"""
import numpy as np
import pytest

import oracle
import synth
import long_context_decode_pkv_amd as pkv
from gpu_common import TOL, make_cache, rel_err, require_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu

# ragged lengths: sink only, all dense, page-aligned, long, one token past a page
LENGTHS = [64 * 20 + 5, 40, 64 * 3 + 1, 64 * 50, 130, 64 * 7 + 63]


def _batch(cfg_id, lengths, store=None, r_k=None, r_v=None, rope=None, kv_heads=2, with_f64=False):
    """One cache per length (sequence i: decode_inputs with seed offset i)."""
    caches, data = [], []
    for i, T in enumerate(lengths):
        d = synth.decode_inputs(cfg_id, T=T, B=1, kv_heads=kv_heads, with_f64=with_f64)
        if i:  # distinct sequences: shift the keys and values of sequence i
            d = synth.decode_inputs(cfg_id, T=T + 64 * i, B=1, kv_heads=kv_heads, with_f64=with_f64)
            for k in ("K", "V") + (("K64", "V64") if with_f64 else ()):
                d[k] = np.ascontiguousarray(d[k][:, :, 64 * i:64 * i + T])
            d["T"] = T
        dt = d["cfg"]["dtype"]
        c = make_cache(d, r_k=r_k, r_v=r_v, max_tokens=T + 64, store=store)
        if rope is not None:
            c.set_key_rope(rope)
        c.prefill(to_dev(d["K"], dt), to_dev(d["V"], dt))
        caches.append(c)
        data.append(d)
    return caches, data


def _queries(cfg_id, n, Hq, dtype):
    g = synth.rng(synth.CONFIGS[cfg_id]["seed"], 77, 0, 0, synth.KIND_Q)
    q = synth.to_storage(g.standard_normal((n, Hq, 128)), dtype)
    return q


def _check_equal_to_single(caches, q, n_split):
    import torch
    out = pkv.decode_batch(caches, q, n_split=n_split)
    torch.cuda.synchronize()
    for i, c in enumerate(caches):
        o = c.decode(q[i:i + 1].contiguous(), n_split=n_split)
        torch.cuda.synchronize()
        assert torch.equal(out[i:i + 1], o), (i, n_split)
    return out


@pytest.mark.parametrize("store,rk,rv", [
    (None, 16, 16), ("int4", 16, 16), (None, 24, 24),
    (None, 16, 13), (None, 24, 22), (None, 32, 30),  # value parts at the exact rank
])
def test_batch_equals_single_caches(store, rk, rv):
    require_gpu()
    caches, data = _batch(2, LENGTHS, store=store, r_k=rk, r_v=rv)
    dt = "bf16"
    q = to_dev(_queries(2, len(caches), data[0]["Hq"], dt), dt)
    for ns in (1, 4, 16):
        _check_equal_to_single(caches, q, ns)
    # the library's split count for the batch (that of its longest cache):
    # the per-cache results to fp32 rounding
    import torch
    out = to_f64(pkv.decode_batch(caches, q))
    for i, c in enumerate(caches):
        o = to_f64(c.decode(q[i:i + 1].contiguous()))
        torch.cuda.synchronize()
        assert rel_err(out[i:i + 1], o) <= 1e-5, i


@pytest.mark.parametrize("rk,rv", [(None, None), (48, 48), (24, 8)])
def test_batch_pre_rope_keys(rk, rv):
    """Pre-RoPE caches in one batched launch (r = 16; r = 48: the one-wave
    format above r = 32) or one launch per cache (unequal padded ranks)."""
    require_gpu()
    f = synth.rope_inv_freq(5e5)
    caches, data = _batch(2, LENGTHS, rope=f, r_k=rk, r_v=rv)
    q = to_dev(_queries(2, len(caches), data[0]["Hq"], "bf16"), "bf16")
    _check_equal_to_single(caches, q, 4)


@pytest.mark.parametrize("cfg_id,store,rk,rv", [
    (1, None, 16, 16),     # fp32: VALU kernel, one launch per cache
    (2, None, 24, 16),     # unequal padded ranks
    (2, None, 48, 22),     # unequal, one rank above 32
    (2, "int4", 24, 16),   # INT4 with unequal padded ranks
])
def test_batch_per_cache_fallback(cfg_id, store, rk, rv):
    require_gpu()
    caches, data = _batch(cfg_id, [64 * 9 + 3, 70, 64 * 12], store=store, r_k=rk, r_v=rv, kv_heads=1)
    dt = data[0]["cfg"]["dtype"]
    q = to_dev(_queries(cfg_id, len(caches), data[0]["Hq"], dt), dt)
    _check_equal_to_single(caches, q, 3)


def test_batch_against_oracle():
    import torch
    require_gpu()
    caches, data = _batch(3, [64 * 30 + 7, 64 * 4, 100], with_f64=True)
    dt = "bf16"
    qn = _queries(3, len(caches), data[0]["Hq"], dt)
    out = to_f64(pkv.decode_batch(caches, to_dev(qn, dt)))
    torch.cuda.synchronize()
    q64 = synth.storage_to_f64(qn, dt)
    for i, d in enumerate(data):
        cfg = d["cfg"]
        ref = oracle.decode(q64[i:i + 1], d["K64"], d["V64"], d["T"], 64, cfg["s"], cfg["w"], cfg["r_k"],
                            cfg["r_v"], dt)
        err = rel_err(out[i:i + 1], ref["o_stored"])
        print(f"[batch vs oracle] cache {i} T={d['T']}: err {err:.3e}")
        assert err <= TOL[dt]


def test_batch_of_32_caches():
    require_gpu()
    lengths = [65 + 97 * i for i in range(32)]
    caches, data = _batch(2, lengths, kv_heads=1)
    q = to_dev(_queries(2, 32, data[0]["Hq"], "bf16"), "bf16")
    _check_equal_to_single(caches, q, 2)


def test_batch_errors():
    import ctypes
    import torch
    require_gpu()
    caches, data = _batch(2, [300, 200], kv_heads=1)
    q = to_dev(_queries(2, 2, data[0]["Hq"], "bf16"), "bf16")
    L = pkv.lib()
    nb = ctypes.c_uint64()
    for n in (0, 33):
        hs = (ctypes.c_void_p * max(n, 1))(*([caches[0]._h] * max(n, 1)))
        assert L.pkv_decode_batch_workspace_bytes(hs, n, 0, ctypes.byref(nb)) == 1
    other = make_cache(data[0], r_k=8, r_v=8, max_tokens=400)
    other.prefill(to_dev(data[0]["K"], "bf16"), to_dev(data[0]["V"], "bf16"))
    with pytest.raises(pkv.PKVError) as ei:  # shapes differ
        pkv.decode_batch([caches[0], other], q)
    assert ei.value.status == 1
    empty = make_cache(data[0], max_tokens=400)
    empty.prefill(to_dev(data[0]["K"], "bf16")[:, :, :0].contiguous(),
                  to_dev(data[0]["V"], "bf16")[:, :, :0].contiguous())
    with pytest.raises(pkv.PKVError) as ei:  # an empty cache
        pkv.decode_batch([caches[0], empty], q)
    assert ei.value.status == 1
    small = torch.empty(64, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(pkv.PKVError) as ei:
        pkv.decode_batch(caches, q, workspace=small)
    assert ei.value.status == 3


def _step_twins(cfg_id, lengths, steps, kv_heads=2, store=None, rope=None, aux=False, w=None, headroom=0):
    """Two identical sets of caches (one per length) with `steps` further
    tokens per sequence: set a steps through pkv_decode_step_batch, set b
    through pkv_decode_step per cache.  `headroom` tokens of capacity beyond
    the run let the pages completed during it leave the window (a window
    page is factorized early only if it can leave within capacity)."""
    import torch
    seqs, A, Bs = [], [], []
    for i, T in enumerate(lengths):
        d = synth.decode_inputs(cfg_id, T=T + steps + 64 * i, B=1, kv_heads=kv_heads)
        dt = d["cfg"]["dtype"]
        Kd = to_dev(np.ascontiguousarray(d["K"][:, :, 64 * i:]), dt)
        Vd = to_dev(np.ascontiguousarray(d["V"][:, :, 64 * i:]), dt)
        for group in (A, Bs):
            c = make_cache(d, max_tokens=T + steps + headroom, store=store, w=w)
            if rope is not None:
                c.set_key_rope(rope)
            c.prefill(Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
            group.append(c)
        seqs.append((Kd, Vd, T))
    if aux:  # True, or one flag per cache
        mask = list(aux) if isinstance(aux, (list, tuple)) else [True] * len(lengths)
        st_a, st_b = torch.cuda.Stream(), torch.cuda.Stream()
        for c, m in zip(A, mask):
            if m:
                c.set_aux_stream(st_a)
        for c, m in zip(Bs, mask):
            if m:
                c.set_aux_stream(st_b)
    return seqs, A, Bs, d


def _run_step_twins(cfg_id, lengths, steps, n_split=4, expect_early=False, **kw):
    """expect_early: the batched caches with an aux stream must factorize
    completed window pages early -- a page's factor slot is written by the
    step that completes the page, before the page leaves the window, and
    holds after the promotion exactly what it held then -- and at least one
    such page must leave the window during the run."""
    import torch
    require_gpu()
    seqs, A, Bs, d = _step_twins(cfg_id, lengths, steps, **kw)
    dt = d["cfg"]["dtype"]
    n, Hq = len(lengths), d["Hq"]
    ws = pkv.batch_workspace(A, n_split)
    aux = kw.get("aux", False)
    mask = list(aux) if isinstance(aux, (list, tuple)) else [bool(aux)] * n
    P, n_s, n_w = 64, A[0].layout["n_sink_slots"], A[0].layout["n_ring_slots"] - 1
    early = {}  # (cache, slot) -> (slot before the completing step, right after it)
    if expect_early:
        # factor slots not yet written get a sentinel (the allocator may hand
        # out a buffer that already holds these very factors)
        for c in A:
            L, nf = c.layout, c.state()[1]
            for h in range(c.shape.n_kv_heads):
                lo = L["factors"] + (h * L["max_fact_pages"] + nf) * L["factor_page_bytes"]
                hi = L["factors"] + (h + 1) * L["max_fact_pages"] * L["factor_page_bytes"]
                c.buffer[lo:hi].fill_(0xFF)
    for t in range(steps):
        k = torch.stack([Kd[0, :, T + t] for Kd, _, T in seqs]).contiguous()
        v = torch.stack([Vd[0, :, T + t] for _, Vd, T in seqs]).contiguous()
        q = to_dev(synth.step_queries(cfg_id, t, n, Hq, 128, dt), dt)
        watch = []
        if expect_early:
            torch.cuda.synchronize()
            for i, c in enumerate(A):
                T1 = c.state()[0] + 1
                p = T1 // P - 1  # the page this step completes
                if mask[i] and n_w > 0 and T1 % P == 0 and p >= n_s and p - n_s < c.layout["max_fact_pages"]:
                    watch.append((i, p - n_s, c.factor_part(0, 0, p - n_s, pkv.KEYS).clone()))
        oa = pkv.step_batch(A, k, v, q, n_split=n_split, workspace=ws)
        for i, c in enumerate(Bs):
            ob = c.step(k[i:i + 1].contiguous(), v[i:i + 1].contiguous(), q[i:i + 1].contiguous(), n_split=n_split)
            torch.cuda.synchronize()
            assert torch.equal(oa[i:i + 1], ob), (t, i)
        for i, f, before in watch:  # the aux stream's work is done (device synchronized)
            assert A[i].state()[1] <= f, "the completed page must still be in the window"
            early[(i, f)] = (before, A[i].factor_part(0, 0, f, pkv.KEYS).clone())
    torch.cuda.synchronize()
    if expect_early:
        left = [(i, f) for (i, f) in early if A[i].state()[1] > f]
        assert left, "no early-factorized page left the window during the run"
        for i, f in left:
            before, after_step = early[(i, f)]
            assert not torch.equal(before, after_step), ("slot not written early", i, f)
            assert torch.equal(after_step, A[i].factor_part(0, 0, f, pkv.KEYS)), ("slot changed at promotion", i, f)
        print(f"[early factorization] {len(left)} early-factorized pages left the window during the run")
    for a, b in zip(A, Bs):
        assert a.state() == b.state()
        T, nf, _ = a.state()
        for x, y in zip(a.page_table(-(-T // 64)), b.page_table(-(-T // 64))):
            np.testing.assert_array_equal(x, y)
        for h in range(a.shape.n_kv_heads):
            for f in range(nf):
                for kind in (pkv.KEYS, pkv.VALUES):
                    assert torch.equal(a.factor_part(0, h, f, kind), b.factor_part(0, h, f, kind))
    return A


# steps and capacity of the aux-stream cases: early-factorized pages (those
# completed during the run) leave the window inside it, (n_w + 1) P = 192
# tokens after completing
EARLY = dict(steps=230, headroom=192, expect_early=True)


@pytest.mark.parametrize("label,cfg_id,kw", [
    ("bf16", 2, {}),
    ("int4", 2, dict(store="int4")),
    ("pre-RoPE", 2, dict(rope=synth.rope_inv_freq(5e5))),
    ("aux stream", 2, dict(aux=True, **EARLY)),
    ("fp32", 1, dict(kv_heads=1)),
])
def test_step_batch_equals_per_cache_steps(label, cfg_id, kw):
    # an empty cache, one in the sink, and caches whose pages complete and
    # leave the window at different steps
    kw = dict(kw)
    steps = kw.pop("steps", 70)
    _run_step_twins(cfg_id, [0, 5, 64 * 3 + 60, 64 * 10 + 63, 64 * 20 + 1], steps, **kw)


@pytest.mark.parametrize("label,cfg_id,kw", [
    ("bf16", 2, {}),
    ("int4", 2, dict(store="int4")),
    ("pre-RoPE", 2, dict(rope=synth.rope_inv_freq(5e5))),
    # caches with an aux stream only wait for their early factorization; the
    # others share the one decomposition launch
    ("mixed aux", 2, dict(aux=[True, False, True, False], **EARLY)),
    # every cache on one aux stream: their early factorizations share a launch
    ("aux together", 2, dict(aux=True, **EARLY)),
])
def test_step_batch_promotes_together(label, cfg_id, kw):
    # every cache completes a page at the same steps, so the pages leaving the
    # windows are decomposed by one launch (which also sets their entries)
    kw = dict(kw)
    steps = kw.pop("steps", 90)
    _run_step_twins(cfg_id, [64 * 5 + 40, 64 * 9 + 40, 64 * 3 + 40, 64 * 12 + 40], steps, **kw)


def test_step_batch_without_window():
    # w = 0: a completed page is promoted by the step that completes it (the
    # caches step one by one)
    _run_step_twins(2, [64 * 2 + 62, 64 * 5 + 10], 70, w=0)


def test_step_batch_against_oracle():
    import torch
    require_gpu()
    cfg_id, steps = 4, 80
    lengths = [64 * 6 + 3, 64 * 2 + 50, 17]
    seqs, A, _, d = _step_twins(cfg_id, lengths, steps, kv_heads=1)
    cfg = d["cfg"]
    dt = cfg["dtype"]
    incs = []
    for Kd, Vd, T in seqs:
        K64 = synth.storage_to_f64(Kd.view(torch.int16).cpu().numpy().view(np.uint16), dt)
        V64 = synth.storage_to_f64(Vd.view(torch.int16).cpu().numpy().view(np.uint16), dt)
        incs.append(oracle.IncrementalDecoder(K64, V64, 64, cfg["s"], cfg["w"], cfg["r_k"], cfg["r_v"], dt))
    worst = 0.0
    for t in range(steps):
        k = torch.stack([Kd[0, :, T + t] for Kd, _, T in seqs]).contiguous()
        v = torch.stack([Vd[0, :, T + t] for _, Vd, T in seqs]).contiguous()
        qn = synth.step_queries(cfg_id, t, len(seqs), d["Hq"], 128, dt)
        o = to_f64(pkv.step_batch(A, k, v, to_dev(qn, dt)))
        torch.cuda.synchronize()
        q64 = synth.storage_to_f64(qn, dt)
        for i, (inc, (_, _, T)) in enumerate(zip(incs, seqs)):
            ref, _ = inc.step(q64[i:i + 1], T + t + 1)
            err = rel_err(o[i:i + 1], ref)
            worst = max(worst, err)
            assert err <= TOL[dt], (t, i, err)
    print(f"[step batch vs oracle] {steps} steps x {len(seqs)} caches, worst err {worst:.3e}")
