"""Benchmark of the PuzzleKV hot path on one MI355X.

Default workload (qwen3-32b-layer-128k): one layer of a Qwen3-32B-shaped cache,
B = 1, 64 query heads, 8 KV heads, d = 128, T = 131072 bf16 tokens, P = 64,
r = 24, sink 64, window 128; 2045 factorized pages per KV head.  A layer step
is one decode step of the hot path on one layer: append the new token's K/V
row, promote the page leaving the window when one is due (page
decomposition), and run mixed decode attention for every query head (the
partial-state kernel, then the cross-split merge).  Four independent layer
caches of this shape are stepped in rotation, as the layers of a model would
be, so no cache's 302 MB is served from the 256 MB Infinity Cache on reuse.
Inputs are seeded synthetic pages with the sigma_i = i^-1.2 spectrum
(synth.py), resident in HBM before timing.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  Other workloads: llama3.1-8b-layer (B = 8, T = 32768,
r = 16), llama3.1-8b-layer-p32 (the same tokens in 32-token pages at
(r_K, r_V) = (16, 14), sink 32, window 32: PuzzleKV Sec. 4.1; -p32-int4 and
-p32-prerope with INT4 factors or pre-RoPE keys), the same layers with
pre-RoPE keys (-prerope), qwen3-32b-layer-128k-int4 and llama3.1-8b-layer-int4 (the same
layers with INT4 factor pages, PuzzleKV Sec. 4.3), incremental (workload 4:
the Llama-shaped layer decoded for 512 steps from T = 8192 with its
promotions), and compress (batched page decomposition, 524288 distinct pages,
r in {8,16,32}).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CACHE_DIR = os.environ.get("PKV_BENCH_CACHE", "/tmp/pkv_bench_inputs")


# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs of
# this script (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled
# by what the same counter reads for the 1 GiB device copy of `--workload copy`
# (FETCH_SIZE reads 524301.6 KiB for 2^30 bytes read -> x1.99995; WRITE_SIZE
# reads 1048576 KiB for 2^30 bytes written -> x1.0).  A figure holds only for
# the kernel sources whose hash it carries; any change to them makes it null.
PMC_TRAFFIC = {
    "qwen3-32b-layer-128k": {"sha256": "3024b2ca48695e27f815c8ea88ab3a2437e597fb35b9ba98f715ee15fac9ab7c",
                           "fetch": 303085466, "write": 1114112},
    "qwen3-32b-layer-128k-int4": {"sha256": "3024b2ca48695e27f815c8ea88ab3a2437e597fb35b9ba98f715ee15fac9ab7c",
                                "fetch": 88847381, "write": 2228224},
    "llama3.1-8b-layer-p32": {"sha256": "3024b2ca48695e27f815c8ea88ab3a2437e597fb35b9ba98f715ee15fac9ab7c",
                            "fetch": 640461063, "write": 1114112},
}
TRAFFIC_SOURCES = ("long_context_decode_pkv_amd/csrc/pkv_decode.hip",
                   "long_context_decode_pkv_amd/csrc/pkv_internal.h")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def pmc_traffic(workload):
    t = PMC_TRAFFIC.get(workload)
    if not t or t["sha256"] is None or t["sha256"] != kernel_sources_sha256():
        return None
    return t


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cached_inputs(cfg_id, T, workers):
    import synth
    os.makedirs(CACHE_DIR, exist_ok=True)
    path = os.path.join(CACHE_DIR, f"cfg{cfg_id}_T{T}.npz")
    if os.path.exists(path):
        z = np.load(path, allow_pickle=False)
        return dict(K=z["K"], V=z["V"], q=z["q"])
    t = time.time()
    d = synth.decode_inputs(cfg_id, T=T, workers=workers)
    log(f"generated workload {cfg_id} inputs T={T} in {time.time() - t:.1f}s")
    np.savez(path, K=d["K"], V=d["V"], q=d["q"])
    return dict(K=d["K"], V=d["V"], q=d["q"])


def to_dev(a, dtype):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.astype(np.float32)).cuda()


def decode_bytes(cfg, B, Hkv, Hq, T, n_fact, store=None):
    """Algorithmic bytes one mixed-attention launch must move: factors of every
    factorized page (r (P + d) elements per K and per V page; INT4 pages:
    (r_K + r_V)(P + d) / 2 code bytes and the 16-bit scales of their four
    factors, 2 (r_K + d + P + d)), the valid rows of every dense page (K and
    V), q in, o out (fp32)."""
    esz = 2 if cfg["dtype"] == "bf16" else 4
    P, d = cfg["P"], cfg["d"]
    if store == "int4":
        fact = n_fact * ((cfg["r_k"] + cfg["r_v"]) * (P + d) // 2 + 2 * (cfg["r_k"] + d + P + d))
    else:
        fact = n_fact * (cfg["r_k"] + cfg["r_v"]) * (P + d) * esz
    dense = (T - n_fact * P) * d * 2 * esz
    return B * Hkv * (fact + dense) + B * Hq * d * esz + B * Hq * d * 4


def host_cpu():
    """The host the oracle runs on: CPU model and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}


def one_core(fn):
    """Run fn with the oracle's OpenMP core and numpy's BLAS on one thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return fn()


def cpu_baseline_decode(cfg, K, V, q, T, store=None, key_rope=None):
    """The oracle on a bounded sample: KV head 0 of the same cache.  The
    oracle reconstructs that head (Jacobi SVD of its factorized pages,
    truncation, storage rounding; timed -> pages/s), then its naive float64
    attention for the head's query heads is timed and scaled to the full step
    (all (sequence, KV head) pairs) -> tokens/s.  Both are timed on all the
    host's cores and again on one core (the SVD on a 128-page share of the
    head's pages there)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    P, s, w = cfg["P"], cfg["s"], cfg["w"]
    n_pairs = K.shape[0] * K.shape[1]
    G = q.shape[1] // K.shape[1]
    k64 = synth.storage_to_f64(K[0, 0, :T], cfg["dtype"])
    v64 = synth.storage_to_f64(V[0, 0, :T], cfg["dtype"])
    q64 = synth.storage_to_f64(q[0, :G], cfg["dtype"])
    n_fact = int((oracle.classify(T, P, s, w)[0] == oracle.FACT).sum())
    t = time.perf_counter()
    st = store or cfg["dtype"]
    Khat = oracle.reconstruct_cache(k64, T, P, s, w, cfg["r_k"], st, kind="K")[0]
    Vhat = oracle.reconstruct_cache(v64, T, P, s, w, cfg["r_v"], st, kind="V")[0]
    t_rec = time.perf_counter() - t
    reps = 3
    t = time.perf_counter()
    for _ in range(reps):
        Ka = Khat if key_rope is None else oracle.rope_rotate(Khat, np.arange(T), key_rope)
        oracle.attention(q64, Ka, Vhat)
    t_att = (time.perf_counter() - t) / reps
    step = t_att * n_pairs

    def timed_one_core():
        t0 = time.perf_counter()
        Ka = Khat if key_rope is None else oracle.rope_rotate(Khat, np.arange(T), key_rope)
        oracle.attention(q64, Ka, Vhat)
        t_att1 = time.perf_counter() - t0
        n1 = min(128, n_fact)
        pages = np.stack([k64[p * P:(p + 1) * P] for p in
                          np.nonzero(oracle.classify(T, P, s, w)[0] == oracle.FACT)[0][:n1]])
        t0 = time.perf_counter()
        oracle.svd_batch(pages)
        return t_att1, n1 / (time.perf_counter() - t0)

    t_att1, svd1 = one_core(timed_one_core)
    return dict(value=K.shape[0] / step, unit="tokens/s", cores=int(max(blas, oracle.num_threads())),
                kind="oracle",
                sample=(f"KV head 0 of the same cache: naive float64 attention of its {G} query "
                        f"heads over T={T} reconstructed tokens took {t_att * 1e3:.1f} ms, scaled "
                        f"by {n_pairs} (sequence, KV head) pairs per step; the oracle's "
                        f"reconstruction of that head ({2 * n_fact} Jacobi SVDs) ran at "
                        f"{2 * n_fact / t_rec:.1f} pages/s"),
                one_core={"value": K.shape[0] / (t_att1 * n_pairs), "unit": "tokens/s",
                          "svd_pages_per_s": svd1,
                          "sample": f"the same attention on one core ({t_att1 * 1e3:.1f} ms), "
                                    f"the Jacobi SVD of {min(128, n_fact)} of the head's pages"},
                host=host_cpu(),
                svd_pages_per_s=2 * n_fact / t_rec)


ROPE_BASE = {2: 5e5, 3: 1e6}  # rotary bases of the Llama 3.1 and Qwen3 checkpoints


# The pages' own operating point (Sec. 4.1): 32-token pages, (r_K, r_V) =
# (16, 14), one sink page and one window page.
P32_POINT = dict(P=32, r_k=16, r_v=14, s=32, w=32)


def bench_decode(args, cfg_id, name, store=None, rope=False, overrides=None):
    """One decode step of the workload's layer, on NL independent layer caches
    in rotation (a decode step of an NL-layer stack), so that no cache is
    re-read from the 256 MB Infinity Cache between its uses.  `overrides`
    replaces cache parameters of the workload (page length, ranks, sink,
    window) over the same input tokens."""
    import torch
    import synth
    import long_context_decode_pkv_amd as pkv

    cfg = dict(synth.CONFIGS[cfg_id])
    cfg.update(overrides or {})
    B, Hq, Hkv, T0 = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"]
    NL = args.layers
    # timed pass, an instrumented pass, then up to P steps to a promotion per layer
    total = T0 + args.warmup + 2 * args.steps + cfg["P"]
    inp = cached_inputs(cfg_id, total, workers=args.workers)
    dt = cfg["dtype"]
    Kd, Vd = to_dev(inp["K"], dt), to_dev(inp["V"], dt)
    caches = [pkv.Cache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, rank_k=cfg["r_k"], rank_v=cfg["r_v"],
                        sink=cfg["s"], window=cfg["w"], max_tokens=total, dtype=store or dt,
                        page_len=cfg["P"])
              for _ in range(NL)]
    freqs = synth.rope_inv_freq(ROPE_BASE[cfg_id]) if rope else None
    if rope:  # pre-RoPE keys, rotated at attention (App. D.3)
        for c in caches:
            c.set_key_rope(freqs)
    K0 = Kd[:, :, :T0].contiguous()
    V0 = Vd[:, :, :T0].contiguous()
    rows_k = [Kd[:, :, t].contiguous() for t in range(T0, total)]
    rows_v = [Vd[:, :, t].contiguous() for t in range(T0, total)]
    qs = [to_dev(synth.step_queries(cfg_id, t, B, Hq, cfg["d"], dt), dt) for t in range(total - T0)]
    out = torch.empty((B, Hq, cfg["d"]), dtype=torch.float32, device="cuda:0")
    del Kd, Vd
    torch.cuda.synchronize()

    # prefill (dense pools + decomposition of every factorized page); the
    # other layer caches first, so that the timed prefill of layer 0 runs
    # warm (its kernels loaded)
    for c in caches[1:]:
        c.prefill(K0, V0)
    if NL == 1:
        caches[0].prefill(K0, V0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    caches[0].prefill(K0, V0)
    e1.record()
    torch.cuda.synchronize()
    t_prefill = e0.elapsed_time(e1) * 1e-3
    n_fact0 = caches[0].state()[1]
    pages0 = B * Hkv * n_fact0 * 2
    log(f"prefill T={T0}: {pages0} pages decomposed in {t_prefill * 1e3:.2f} ms; {NL} layer caches")
    wss = [c.workspace(512) for c in caches]  # fits every split count
    P, n_s, n_w = cfg["P"], cfg["s"] // cfg["P"], cfg["w"] // cfg["P"]
    aux = torch.cuda.Stream() if args.aux else None  # default priority
    if aux is not None:
        for c in caches:  # completed window pages are factorized early, on aux
            c.set_aux_stream(aux)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def layer_step(c, ws, i, rec=None):
        """pkv_decode_step: promotion when a page leaves the window, attention
        over the cached tokens, then the merge, which adds the new token's
        state and writes the token into the cache (no append launch)."""
        if rec is None:
            c.step(rows_k[i], rows_v[i], qs[i], out=out, workspace=ws)
            return None
        T, nf, _ = c.state()
        due = (T + 1) // P - n_s - n_w > nf
        # the partial kernel's own duration, or (synchronous promotions) the
        # decomposition's, which is then the first kernel of the step
        timed_promo = due and aux is None
        pkv.time_next_kernel(*(rec["promote"] if timed_promo else rec["partial"]))
        rec["promoted"] = timed_promo
        c.step(rows_k[i], rows_v[i], qs[i], out=out, workspace=ws)
        rec["merge"][1].record()
        return T + 1, nf + (1 if due else 0)

    for i in range(args.warmup):
        for c, ws in zip(caches, wss):
            layer_step(c, ws, i)
    torch.cuda.synchronize()
    # timed pass: exactly `steps` layer steps per layer cache, nothing but the
    # library calls inside the timed region
    nf_timed0 = sum(c.state()[1] for c in caches)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for j in range(args.steps):
        for c, ws in zip(caches, wss):
            layer_step(c, ws, args.warmup + j)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    promos_timed = sum(c.state()[1] for c in caches) - nf_timed0  # promotions inside `value`

    # instrumented pass (not part of `value`): the same steps on the next
    # tokens, each attention launch bracketed by its kernel's own events
    recs = [[{"partial": (ev(), ev()), "merge": (None, ev()), "promote": (ev(), ev())}
             for _ in range(NL)] for _ in range(args.steps)]
    for e in (e for step in recs for r in step for pair in r.values() for e in pair if e is not None):
        e.record()  # creates the event before the pass
    states = []
    torch.cuda.synchronize()
    t = time.perf_counter()
    for j in range(args.steps):
        for li, (c, ws) in enumerate(zip(caches, wss)):
            states.append(layer_step(c, ws, args.warmup + args.steps + j, recs[j][li]))
    torch.cuda.synchronize()
    elapsed_instr = time.perf_counter() - t
    layer_steps = args.steps * NL
    # one promotion per layer cache whatever the step count: step on to the
    # first step at which a page leaves the window and time its decomposition
    # (the first kernel of that step)
    i = args.warmup + 2 * args.steps
    extra = []
    while not extra and i < total - T0:
        T, nf, _ = caches[0].state()  # every cache has the same length
        due = (T + 1) // P - n_s - n_w > nf
        for c, ws in zip(caches, wss):
            if due and aux is None:
                pair = (ev(), ev())
                pkv.time_next_kernel(*pair)
                extra.append(pair)
            c.step(rows_k[i], rows_v[i], qs[i], out=out, workspace=ws)
        i += 1
    torch.cuda.synchronize()
    flat = [r for step in recs for r in step]
    keep = [k for k, r in enumerate(flat) if not r["promoted"]]
    durs = np.array([flat[k]["partial"][0].elapsed_time(flat[k]["partial"][1]) * 1e-3 for k in keep])
    merges = np.array([flat[k]["partial"][1].elapsed_time(flat[k]["merge"][1]) * 1e-3 for k in keep])
    promos = [r["promote"][0].elapsed_time(r["promote"][1]) * 1e-3 for r in flat if r["promoted"]]
    promos += [a.elapsed_time(b) * 1e-3 for a, b in extra]
    if aux is not None:
        # early factorizations overlap later steps; time the same launch
        # (one page of every (sequence, KV head, K/V)) on its own
        pages = np.ascontiguousarray(inp["K"][:, :, :2 * P].reshape(-1, P, cfg["d"])[:2 * B * Hkv])
        Xp = to_dev(pages, dt)
        for _ in range(6):
            a, b = ev(), ev()
            a.record()
            b.record()
            pkv.time_next_kernel(a, b)
            pkv.compress_pages(Xp, cfg["r_k"], with_sigma=False)
            torch.cuda.synchronize()
            promos.append(a.elapsed_time(b) * 1e-3)
        promos = promos[1:]
    # the attention call alone (pkv_decode_attn: the split partials and the
    # merge, no append or promotion), `steps` calls per layer cache over the
    # tokens the caches now hold
    T_call, nf_call, _ = caches[0].state()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for j in range(args.steps):
        for c, ws in zip(caches, wss):
            c.decode(qs[j], out=out, workspace=ws)
    torch.cuda.synchronize()
    t_call = (time.perf_counter() - t) / layer_steps
    bytes_call = decode_bytes(cfg, B, Hkv, Hq, T_call, nf_call, store)
    log(f"attention call (pkv_decode_attn) at T={T_call}: {t_call * 1e6:.1f} us per layer, "
        f"{bytes_call / t_call / 1e9:.0f} GB/s ({bytes_call / t_call / 1e9 / HBM_PEAK_GBS * 100:.1f}% of peak)")
    # early factorization in steady state (without --aux): the caches refilled
    # through pkv_prefill_chunk with a second stream, which factorizes the
    # window's complete pages there, then P steps per layer -- one page
    # completion (its decomposition on the second stream) and one promotion
    # (which only waits for that work) per layer
    step_early = None
    if aux is None:
        aux2 = torch.cuda.Stream()  # default priority
        empty = K0[:, :, :0].contiguous()
        for c in caches:
            c.set_aux_stream(aux2)
            c.prefill(empty, empty)
            c.prefill_chunk(K0, V0)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for j in range(P):
            for c, ws in zip(caches, wss):
                c.step(rows_k[j], rows_v[j], qs[j], out=out, workspace=ws)
        torch.cuda.synchronize()
        step_early = (time.perf_counter() - t) / (P * NL)
        log(f"early factorization on a second stream, steady state: {step_early * 1e6:.1f} us per layer step "
            f"over {P} steps x {NL} layers (one page completion and one promotion per layer)")
    del K0, V0
    states = [states[k] for k in keep]
    nbytes = np.array([decode_bytes(cfg, B, Hkv, Hq, T, nf, store) for T, nf in states], dtype=np.float64)
    achieved = nbytes.sum() / durs.sum() / 1e9
    traffic = pmc_traffic(name)
    # promotions at their rate: one per P steps of a layer; the timed pass
    # holds promos_timed of them
    t_promo = float(np.mean(promos)) if promos else 0.0
    step_amortized = (elapsed - promos_timed * t_promo) / layer_steps + t_promo / P
    log(f"partial kernel: mean {durs.mean() * 1e6:.2f} us (median {np.median(durs) * 1e6:.2f}), "
        f"{nbytes.mean() / 1e6:.1f} MB -> {achieved:.0f} GB/s; partial end to merge end "
        f"{merges.mean() * 1e6:.2f} us; "
        f"{len(promos)} promotions, mean {np.mean(promos) * 1e6 if promos else 0:.1f} us; "
        f"layer step {elapsed / layer_steps * 1e6:.1f} us "
        f"({elapsed_instr / layer_steps * 1e6:.1f} us with per-launch events); "
        f"{promos_timed} promotions in the timed pass; with one promotion per {P} steps "
        f"{step_amortized * 1e6:.1f} us per layer step")

    res = {
        "metric": "decode-attn tokens/s (one layer: batch tokens per second of a layer decode step)",
        "value": B * layer_steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / layer_steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 dense pages + int4 factor pages (bf16 scales), f32 math" if store == "int4"
                  else "bf16 storage, f32 math" if dt == "bf16" else "f32"),
        "data": "synthetic (seeded generator, workload recipe)",
        "config": {"workload": name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": cfg["d"],
                   "context_tokens": T0, "page_len": cfg["P"], "rank_k": cfg["r_k"],
                   "rank_v": cfg["r_v"], "sink": cfg["s"], "window": cfg["w"],
                   "layer_caches_rotated": NL, "factor_store": store or dt,
                   "keys": (f"pre-RoPE, rotated at attention (base {ROPE_BASE[cfg_id]:g})" if rope
                            else "as given"),
                   "step": "pkv_decode_step per layer: promotion when a page leaves the window, "
                           "decode partial, merge with the appended token folded in",
                   "early_factorization": bool(args.aux)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     # the whole layer step (partial, merge and the gaps
                     # between launches) against the same bytes
                     "frac_step": nbytes.mean() / (elapsed / layer_steps) / 1e9 / HBM_PEAK_GBS,
                     "frac_step_promotions_amortized": nbytes.mean() / step_amortized / 1e9 / HBM_PEAK_GBS,
                     # the attention call (pkv_decode_attn: partial + merge)
                     "frac_call": bytes_call / t_call / 1e9 / HBM_PEAK_GBS,
                     "traffic": None if traffic is None else traffic["fetch"] + traffic["write"],
                     "kernel": ("decode_mfma_kernel (pkv_decode_partial)" if cfg["P"] == 64
                                else "decode_valu_kernel (pkv_decode_partial)"),
                     "launch_us_mean": durs.mean() * 1e6,
                     "bytes_per_launch": float(nbytes.mean()),
                     "traffic_read_write": None if traffic is None else [traffic["fetch"],
                                                                         traffic["write"]]},
        "breakdown_us": {"decode_partial": durs.mean() * 1e6,
                         "partial_end_to_merge_end": merges.mean() * 1e6,
                         "promote_mean": float(np.mean(promos) * 1e6) if promos else None,
                         "promotions_timed": len(promos),
                         "promotions_in_value": promos_timed,
                         "promote_amortized_per_step": t_promo / P * 1e6,
                         "layer_step_promotions_amortized": step_amortized * 1e6,
                         "layer_step_early_factorization": None if step_early is None else step_early * 1e6,
                         "attention_call": t_call * 1e6,
                         "layer_step_with_events": elapsed_instr / layer_steps * 1e6},
        "ms_per_step_promotions_amortized": step_amortized * 1e3,
        "decode_effective_GBps": achieved,
        "pages_compressed_per_s": pages0 / t_prefill,
        "prefill_ms": t_prefill * 1e3,
    }
    del caches, wss
    torch.cuda.empty_cache()
    if args.with_compress:
        # the third figure of the metric: batched compression of workload 5
        # (524288 pages, r = 16), measured after the decode steps
        c5 = synth.CONFIGS[5]
        n_total = c5["layers"] * c5["Hkv"] * 2 * c5["pages_per_head"]
        X = compress_pool(n_total)
        cres = measure_compress(X, n_total, [c5["ranks"][1]], 3, 1)
        del X
        res["compress"] = {"workload": "batched-prefill-compression", "pages": n_total,
                           "rank": c5["ranks"][1], "pages_per_s": cres[c5["ranks"][1]]["pages_per_s"],
                           "roofline": compress_summary(cres, c5["ranks"][1])}
    if args.cpu_baseline:
        log("timing the oracle on a bounded sample (cpu_baseline)")
        cb = cpu_baseline_decode(cfg, inp["K"], inp["V"], inp["q"], T0, store, freqs)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample", "one_core", "host")}
        res["cpu_baseline_svd_pages_per_s"] = cb["svd_pages_per_s"]
    return res


VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (256 CUs x 2.4 GHz, packed FMA)
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


def compress_flops(r, P=64, d=128):
    """Algorithmic flops of one page decomposition by the tridiagonal route:
    Gram 2P^2d and R = Q_r^T X 2rPd on the matrix cores; Householder
    reduction (4/3)P^3, accumulation of its orthogonal factor (4/3)P^3 and
    Q_r = Q_H Z 2P^2r on the vector ALUs (the eigenvalue and eigenvector
    recurrences of the tridiagonal matrix, O(P r) per round, are left out)."""
    return dict(mfma_bf16=2 * P * P * d, mfma_f32=2 * r * P * d,
                valu=(8 * P ** 3) // 3 + 2 * P * P * r)


def compress_pool(n_total):
    """The batched-compression workload's n_total distinct pages, drawn on
    the device (synth.compression_pool_device), as a bf16 device tensor."""
    import torch
    import synth
    t = time.time()
    X = synth.compression_pool_device(n_total, device="cuda:0").view(torch.bfloat16)
    torch.cuda.synchronize()
    log(f"drew {n_total} distinct pages on the device in {time.time() - t:.1f}s")
    return X


def measure_compress(X, n_total, ranks, steps, warmup):
    """Each rank: warm-up launches, then `steps` launches of pkv_compress_pages
    over all n_total pages, each timed by its own kernel events."""
    import torch
    import long_context_decode_pkv_amd as pkv
    out = {}
    stream = torch.cuda.current_stream().cuda_stream
    for r in ranks:
        Lf = torch.empty((n_total, 64, r), dtype=torch.bfloat16, device="cuda:0")
        Rf = torch.empty((n_total, r, 128), dtype=torch.bfloat16, device="cuda:0")
        for _ in range(warmup):
            assert pkv.lib().pkv_compress_pages(X.data_ptr(), n_total, 64, 128, r, 0, 0, Lf.data_ptr(),
                                                Rf.data_ptr(), None, stream) == 0
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record()
            b.record()
        torch.cuda.synchronize()
        for a, b in evs:
            pkv.time_next_kernel(a, b)  # the kernel's own duration
            assert pkv.lib().pkv_compress_pages(X.data_ptr(), n_total, 64, 128, r, 0, 0, Lf.data_ptr(),
                                                Rf.data_ptr(), None, stream) == 0
        torch.cuda.synchronize()
        t = sum(a.elapsed_time(b) for a, b in evs) * 1e-3 / steps
        fl = compress_flops(r)
        out[r] = dict(ms=t * 1e3, pages_per_s=n_total / t,
                      valu_tflops=fl["valu"] * n_total / t / 1e12,
                      mfma_bf16_tflops=fl["mfma_bf16"] * n_total / t / 1e12,
                      mfma_f32_tflops=fl["mfma_f32"] * n_total / t / 1e12)
        log(f"compress r={r}: {t * 1e3:.2f} ms per {n_total} pages -> {n_total / t:.3e} pages/s")
        del Lf, Rf
    return out


def cpu_baseline_compress(X, n_sample):
    """The oracle's Jacobi SVD (double precision, OpenMP) on a sample of the
    workload's pages -> pages/s, on all cores and on one core (a 256-page
    share).  The SVD cost does not depend on r."""
    import torch
    import oracle
    import synth
    X64 = synth.storage_to_f64(X[:n_sample].view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    t = time.perf_counter()
    oracle.svd_batch(X64)
    dt = time.perf_counter() - t

    def single():
        t0 = time.perf_counter()
        oracle.svd_batch(X64[:256])
        return 256 / (time.perf_counter() - t0)

    return dict(value=n_sample / dt, unit="pages/s", cores=int(oracle.num_threads()), kind="oracle",
                sample=f"Jacobi SVD of the first {n_sample} pages of the workload's page pool "
                       f"(same recipe: sigma_i = i^-1.2 spectrum plus 2% noise pages), {dt:.1f} s",
                one_core={"value": one_core(single), "unit": "pages/s",
                          "sample": "Jacobi SVD of the first 256 of those pages on one core"},
                host=host_cpu())


def compress_summary(res, r0):
    m = res[r0]
    return {"bound": "alu", "achieved": m["valu_tflops"], "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": m["valu_tflops"] / VALU_PEAK_TFLOPS, "traffic": None,
            "kernel": "compress_tri_kernel (pkv_compress_pages, r <= 32)",
            "mfma_bf16_frac": m["mfma_bf16_tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "mfma_f32_frac": m["mfma_f32_tflops"] / MFMA_F32_PEAK_TFLOPS,
            "launch_ms": m["ms"]}


def bench_compress(args):
    """Batched prefill compression (workload 5): 524288 pages per rank setting."""
    import synth
    cfg = synth.CONFIGS[5]
    n_total = cfg["layers"] * cfg["Hkv"] * 2 * cfg["pages_per_head"]
    X = compress_pool(n_total)
    steps = max(1, min(args.steps, 8))
    res = measure_compress(X, n_total, cfg["ranks"], steps, max(1, min(args.warmup, 2)))
    r0 = cfg["ranks"][1]
    out = {
        "metric": "pages compressed/s (batched page decomposition)",
        "value": res[r0]["pages_per_s"], "unit": "pages/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": res[r0]["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in/out, f32 eigen-solve",
        "data": f"synthetic: {n_total} distinct seeded pages drawn on the device",
        "config": {"workload": "batched-prefill-compression", "pages": n_total, "rank": r0,
                   "pages_per_s_by_rank": {r: m["pages_per_s"] for r, m in res.items()}},
        "roofline": compress_summary(res, r0),
    }
    if args.cpu_baseline:
        log("timing the oracle on a bounded sample (cpu_baseline)")
        out["cpu_baseline"] = cpu_baseline_compress(X, 4096)
    return out


def bench_incremental(args):
    """Workload 4: the Llama-3.1-8B-shaped layer (B = 8, 32 query heads, 8 KV
    heads, r = 16, sink 64, window 128) from T = 8192, 512 decode steps; each
    appends one token per (sequence, KV head) and every 64th promotes the page
    leaving the window (128 page decompositions), then attends.  NL layer
    caches are stepped in rotation (4 x 105-111 MB, above the 256 MB Infinity
    Cache).  Timed twice from the same prefilled state: once with nothing but
    the library calls inside the timed region (`value`), once with an event
    after every layer step, which splits the steps into promotion and
    non-promotion steps (the promotion overhead, cf. the pages' +0.18% TPOT,
    Sec. 4.5 Table 4) and times each promotion's decomposition kernel."""
    import torch
    import synth
    import long_context_decode_pkv_amd as pkv

    cfg = dict(synth.CONFIGS[4])
    B, Hq, Hkv, T0, n_steps, P = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["steps"], cfg["P"]
    dt, NL = cfg["dtype"], args.layers
    total = T0 + n_steps
    inp = cached_inputs(4, total, workers=args.workers)
    Kd, Vd = to_dev(inp["K"], dt), to_dev(inp["V"], dt)
    K0, V0 = Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous()
    rows_k = [Kd[:, :, t].contiguous() for t in range(T0, total)]
    rows_v = [Vd[:, :, t].contiguous() for t in range(T0, total)]
    qs = [to_dev(synth.step_queries(4, t, B, Hq, cfg["d"], dt), dt) for t in range(n_steps)]
    del Kd, Vd
    caches = [pkv.Cache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, rank_k=cfg["r_k"], rank_v=cfg["r_v"],
                        sink=cfg["s"], window=cfg["w"], max_tokens=total, dtype=dt) for _ in range(NL)]
    wss = [c.workspace(512) for c in caches]
    out = torch.empty((B, Hq, cfg["d"]), dtype=torch.float32, device="cuda:0")
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def prefill():
        for c in caches:
            c.prefill(K0, V0)
        torch.cuda.synchronize()

    # warm-up (kernels loaded, clocks up), then the timed pass from T0
    prefill()
    for t in range(min(args.warmup, n_steps)):
        for c, ws in zip(caches, wss):
            c.step(rows_k[t], rows_v[t], qs[t], out=out, workspace=ws)
    prefill()
    t0 = time.perf_counter()
    for t in range(n_steps):
        for c, ws in zip(caches, wss):
            c.step(rows_k[t], rows_v[t], qs[t], out=out, workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # instrumented pass: the same 512 steps again
    prefill()
    marks = [ev() for _ in range(n_steps * NL + 1)]
    promo = []  # (layer step index, decomposition events)
    for e in marks:
        e.record()
    torch.cuda.synchronize()
    marks[0].record()
    k = 0
    for t in range(n_steps):
        for c, ws in zip(caches, wss):
            T, nf, _ = c.state()
            if (T + 1) // P - cfg["s"] // P - cfg["w"] // P > nf:
                pair = (ev(), ev())
                pkv.time_next_kernel(*pair)
                promo.append((k, pair))
            c.step(rows_k[t], rows_v[t], qs[t], out=out, workspace=ws)
            k += 1
            marks[k].record()
    torch.cuda.synchronize()
    durs = np.array([marks[i].elapsed_time(marks[i + 1]) * 1e-3 for i in range(n_steps * NL)])
    is_promo = np.zeros(n_steps * NL, dtype=bool)
    is_promo[[k for k, _ in promo]] = True
    dec = np.array([a.elapsed_time(b) * 1e-3 for _, (a, b) in promo])
    plain, with_p = durs[~is_promo], durs[is_promo]
    overhead = with_p.mean() - plain.mean()
    amortized = overhead * is_promo.sum() / durs.size
    states = [(T0 + t, (T0 + t) // P - cfg["s"] // P - cfg["w"] // P) for t in range(n_steps)]
    nbytes = float(np.mean([decode_bytes(cfg, B, Hkv, Hq, T, nf) for T, nf in states]))
    step = elapsed / (n_steps * NL)
    log(f"incremental: {n_steps} steps x {NL} layers from T={T0}: {step * 1e6:.1f} us per layer step; "
        f"instrumented: plain steps {plain.mean() * 1e6:.1f} us, promotion steps {with_p.mean() * 1e6:.1f} us "
        f"({is_promo.sum()} of {durs.size}), decomposition of {2 * B * Hkv} pages {dec.mean() * 1e6:.1f} us; "
        f"promotion overhead {amortized / plain.mean() * 100:.2f}% per step")
    # early factorization: the same steps with a second stream per cache
    # (pkv_cache_set_aux_stream), on which each window page is factorized as
    # soon as a token completes it; the page's promotion, n_w pages later,
    # only waits for that work.  The caches are filled through
    # pkv_prefill_chunk, which factorizes the window's complete pages there
    # as well, so every promotion of the run is an early one.
    aux = torch.cuda.Stream()  # default priority
    empty = K0[:, :, :0].contiguous()

    def prefill_early():
        for c in caches:
            c.prefill(empty, empty)
            c.prefill_chunk(K0, V0)
        torch.cuda.synchronize()

    for c in caches:
        c.set_aux_stream(aux)
    prefill_early()
    for t in range(min(args.warmup, n_steps)):
        for c, ws in zip(caches, wss):
            c.step(rows_k[t], rows_v[t], qs[t], out=out, workspace=ws)
    prefill_early()
    t0 = time.perf_counter()
    for t in range(n_steps):
        for c, ws in zip(caches, wss):
            c.step(rows_k[t], rows_v[t], qs[t], out=out, workspace=ws)
    torch.cuda.synchronize()
    step_early = (time.perf_counter() - t0) / (n_steps * NL)
    # the same step without promotion work: the timed pass less its
    # promotions' overhead (measured per step in the instrumented pass)
    step_plain = step - amortized
    log(f"incremental with early factorization on a second stream: {step_early * 1e6:.1f} us per layer step "
        f"({B / step_early:.0f} tokens/s); promotion overhead {(step_early - step_plain) / step_plain * 100:.2f}% "
        f"per step against {amortized / step_plain * 100:.2f}% with promotions in the step")
    return {
        "metric": "decode-attn tokens/s (one layer: incremental decode steps with promotions)",
        "value": B * n_steps * NL / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": step * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 storage, f32 math",
        "data": "synthetic (seeded generator, workload-4 recipe)",
        "config": {"workload": "incremental-llama3.1-8b", "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": cfg["d"], "context_tokens": [T0, total], "page_len": P,
                   "rank_k": cfg["r_k"], "rank_v": cfg["r_v"], "sink": cfg["s"], "window": cfg["w"],
                   "layer_caches_rotated": NL,
                   "step": "pkv_decode_step per layer: append, promotion when a page leaves the window, "
                           "decode partial, merge"},
        "roofline": {"bound": "hbm", "achieved": nbytes / step / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / step / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "whole layer step (algorithmic bytes of its attention / step time)",
                     "bytes_per_step": nbytes},
        "breakdown_us": {"plain_step": plain.mean() * 1e6, "promotion_step": with_p.mean() * 1e6,
                         "promotion_steps": int(is_promo.sum()), "steps": int(durs.size),
                         "decomposition_kernel": float(dec.mean() * 1e6),
                         "promotion_overhead_per_step": amortized * 1e6,
                         "promotion_overhead_frac": amortized / step_plain,
                         "instrumented_step": durs.mean() * 1e6},
        "early_factorization": {"ms_per_step": step_early * 1e3, "tokens_per_s": B / step_early,
                                "promotion_overhead_per_step_us": (step_early - step_plain) * 1e6,
                                "promotion_overhead_frac": (step_early - step_plain) / step_plain,
                                "how": "pkv_cache_set_aux_stream: each window page factorized on a second "
                                       "stream when a token completes it; promotions wait for that work"},
    }


RAGGED_LENGTHS = [32768, 28672, 24576, 20480, 16384, 12288, 8192, 4096]


def bench_ragged_batch(args):
    """Serving batch: 8 sequences of different lengths (32K down to 4K) of the
    Llama-3.1-8B-shaped layer, one cache each.  A step is one
    pkv_decode_step_batch per layer (each sequence appends a token, pages
    leaving a window are factorized, every sequence attends), on NL layer
    caches in rotation; compared with one pkv_decode_step per cache.  The
    attention alone (pkv_decode_attn_batch) is timed beside it."""
    import torch
    import synth
    import long_context_decode_pkv_amd as pkv

    cfg = dict(synth.CONFIGS[2])
    Hq, Hkv, d = cfg["Hq"], cfg["Hkv"], cfg["d"]
    NL = args.layers
    n = len(RAGGED_LENGTHS)
    extra = 2 * (args.warmup + args.steps)  # tokens the batched and the per-cache passes append
    inp = cached_inputs(2, max(RAGGED_LENGTHS) + extra, workers=args.workers)  # sequence i: batch row i
    dt = cfg["dtype"]
    layers = []
    for _ in range(NL):
        cs = []
        for i, T in enumerate(RAGGED_LENGTHS):
            c = pkv.Cache(batch=1, n_q_heads=Hq, n_kv_heads=Hkv, rank_k=cfg["r_k"], rank_v=cfg["r_v"],
                          sink=cfg["s"], window=cfg["w"], max_tokens=T + extra, dtype=dt)
            c.prefill(to_dev(np.ascontiguousarray(inp["K"][i:i + 1, :, :T]), dt),
                      to_dev(np.ascontiguousarray(inp["V"][i:i + 1, :, :T]), dt))
            cs.append(c)
        layers.append(cs)
    # the new tokens of step t: [n][H_kv][d]
    ks = [to_dev(np.ascontiguousarray(np.stack([inp["K"][i, :, T + t] for i, T in enumerate(RAGGED_LENGTHS)])), dt)
          for t in range(extra)]
    vs = [to_dev(np.ascontiguousarray(np.stack([inp["V"][i, :, T + t] for i, T in enumerate(RAGGED_LENGTHS)])), dt)
          for t in range(extra)]
    qs = [to_dev(synth.step_queries(2, t, n, Hq, d, dt), dt) for t in range(extra)]
    out = torch.empty((n, Hq, d), dtype=torch.float32, device="cuda:0")
    ws = pkv.batch_workspace(layers[0])
    wss = [c.workspace(512) for c in layers[0]]  # fits every split count
    torch.cuda.synchronize()
    t_next = [0]

    def batched_step():
        t = t_next[0]
        for cs in layers:
            pkv.step_batch(cs, ks[t], vs[t], qs[t], out=out, workspace=ws)
        t_next[0] += 1

    def separate_steps():
        t = t_next[0]
        for cs in layers:
            for i, c in enumerate(cs):
                c.step(ks[t][i:i + 1], vs[t][i:i + 1], qs[t][i:i + 1], out=out[i:i + 1], workspace=wss[i])
        t_next[0] += 1

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (args.steps * NL)

    t_batch = timed(batched_step)
    t_sep = timed(separate_steps)
    # attention alone, and the batched partial kernel's own duration
    q = qs[0]

    def attn():
        for cs in layers:
            pkv.decode_batch(cs, q, out=out, workspace=ws)

    t_attn = timed(attn)
    durs = []
    for _ in range(args.steps):
        for cs in layers:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            pkv.time_next_kernel(a, b)
            pkv.decode_batch(cs, q, out=out, workspace=ws)
            durs.append((a, b))
    torch.cuda.synchronize()
    dur = float(np.mean([a.elapsed_time(b) * 1e-3 for a, b in durs]))
    nbytes = sum(decode_bytes(cfg, 1, Hkv, Hq, c.state()[0], c.state()[1]) for c in layers[0])
    achieved = nbytes / dur / 1e9
    log(f"ragged batch of {n}: batched step {t_batch * 1e6:.1f} us, per-cache steps {t_sep * 1e6:.1f} us, "
        f"batched attention {t_attn * 1e6:.1f} us per layer; partial kernel {dur * 1e6:.1f} us, "
        f"{nbytes / 1e6:.1f} MB -> {achieved:.0f} GB/s")
    return {
        "metric": "decode-attn tokens/s (one layer: decode step of a batch of sequences of different lengths)",
        "value": n / t_batch, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_batch * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 storage, f32 math", "data": "synthetic (seeded generator, workload-2 recipe)",
        "config": {"workload": "llama3.1-8b-ragged-batch", "sequences": n, "lengths": RAGGED_LENGTHS,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "page_len": cfg["P"], "rank_k": cfg["r_k"],
                   "rank_v": cfg["r_v"], "sink": cfg["s"], "window": cfg["w"], "layer_caches_rotated": NL,
                   "step": "pkv_decode_step_batch per layer: append, promotion when due, attention"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_mfma_kernel (batched launch)", "launch_us_mean": dur * 1e6,
                     "bytes_per_launch": nbytes},
        "breakdown_us": {"per_cache_steps_per_layer": t_sep * 1e6, "batched_attention_per_layer": t_attn * 1e6},
    }


def bench_copy(args):
    """Plain device-to-device copy of a known size: the reference that scales
    the HBM traffic counters (FETCH_SIZE, WRITE_SIZE) read under rocprofv3."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / args.steps
    return {"metric": "device copy bandwidth (counter calibration)", "value": 2 * n / t / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 0, "ms_per_step": t * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
            "data": "synthetic", "config": {"workload": "copy", "bytes_read_per_copy": n,
                                            "bytes_written_per_copy": n}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen3-32b-layer-128k",
                    choices=["qwen3-32b-layer-128k", "llama3.1-8b-layer", "qwen3-32b-layer-128k-int4",
                             "llama3.1-8b-layer-int4", "qwen3-32b-layer-128k-prerope",
                             "llama3.1-8b-layer-prerope", "llama3.1-8b-layer-p32", "llama3.1-8b-layer-p32-prerope",
                             "llama3.1-8b-layer-p32-int4",
                             "llama3.1-8b-ragged-batch", "incremental",
                             "compress", "copy"])
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--workers", type=int, default=1)
    ap.add_argument("--layers", type=int, default=4,
                    help="independent layer caches decoded in rotation (defeats cache reuse)")
    ap.add_argument("--aux", action="store_true",
                    help="decode workloads: factorize completed window pages early on a second "
                         "stream (pkv_cache_set_aux_stream); measured slower on the 128K layer")
    ap.add_argument("--no-compress", dest="with_compress", action="store_false",
                    help="decode workloads: skip the batched-compression figure")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the hot path is measured on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    import long_context_decode_pkv_amd as pkv
    if not os.path.exists(pkv.LIB_PATH):
        from long_context_decode_pkv_amd import build
        build.build()
    pkv.lib()
    if args.workload == "compress":
        res = bench_compress(args)
    elif args.workload == "copy":
        res = bench_copy(args)
    elif args.workload == "llama3.1-8b-ragged-batch":
        res = bench_ragged_batch(args)
    elif args.workload == "incremental":
        res = bench_incremental(args)
    else:
        cfg_id = 2 if args.workload.startswith("llama3.1-8b-layer") else 3
        res = bench_decode(args, cfg_id, args.workload, "int4" if args.workload.endswith("-int4") else None,
                           rope=args.workload.endswith("-prerope"),
                           overrides=P32_POINT if "-p32" in args.workload else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
