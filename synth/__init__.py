"""Seeded synthetic inputs for the PuzzleKV hot path.

Shared by both sides (the oracle and the HIP path); holds none of the method's
arithmetic -- only random draws, the generator recipes below, and rounding of
the generated doubles to the storage dtype (nearest-even, one rounding).

The pages measure on RULER / LongBench / NIAH with trained models; none of that
is used here.  These recipes stand in for real KV pages with the shapes the
pages and the workload list name (head_dim 128, 8 KV heads, GQA, P = 64):

* ``lowrank``  (workloads 1, 2, 4): per page A B + 0.1 N(0,1) with A ~ N(0,1)
  (64 x 8) and B ~ N(0, 1/8) (8 x 128) -- the second arguments are variances --
  plus one mean vector ~ N(0, 0.5) per (sequence, KV head) added to every row;
  keys additionally get 4 distinct outlier channels (per sequence and KV head)
  multiplied by 10 after the mean is added.  Values: same recipe, no outliers.
* ``spectrum`` (workloads 3, 5): per page X = U diag(i^-1.2) W^T, U Haar on
  O(64), W 128 x 64 with Haar-orthonormal columns (QR of a Gaussian with the
  sign of diag(R) fixed).  Values drawn the same way, independently.
* workload 5 adds exactly round(0.02 n) pages of N(0,1) noise, chosen by a
  seeded permutation.
* queries q ~ N(0,1).

Random streams: numpy Generator(SFC64) seeded by SeedSequence(entropy=seed,
spawn_key=(...)), one independent stream per (sequence, layer, KV head, kind) so
the bytes do not depend on thread count or generation order.
"""
from __future__ import annotations

import numpy as np

KIND_K, KIND_V, KIND_Q, KIND_META_K, KIND_META_V, KIND_PAGE = 0, 1, 2, 3, 4, 5

# The five workloads (shapes as named by the workload list; seeds 1..5).
CONFIGS = {
    1: dict(name="tiny-fp32", seed=1, B=1, Hq=1, Hkv=1, d=128, T=1024, dtype="f32", P=64,
            r_k=16, r_v=16, s=64, w=128, recipe="lowrank"),
    2: dict(name="llama3.1-8b-layer", seed=2, B=8, Hq=32, Hkv=8, d=128, T=32768, dtype="bf16",
            P=64, r_k=16, r_v=16, s=64, w=128, recipe="lowrank"),
    3: dict(name="qwen3-32b-layer-128k", seed=3, B=1, Hq=64, Hkv=8, d=128, T=131072,
            dtype="bf16", P=64, r_k=24, r_v=24, s=64, w=128, recipe="spectrum"),
    4: dict(name="incremental-llama3.1-8b", seed=4, B=8, Hq=32, Hkv=8, d=128, T=8192,
            steps=512, dtype="bf16", P=64, r_k=16, r_v=16, s=64, w=128, recipe="lowrank"),
    5: dict(name="batched-prefill-compression", seed=5, layers=64, Hkv=8, pages_per_head=512,
            d=128, dtype="bf16", P=64, ranks=(8, 16, 32), recipe="spectrum+noise",
            noise_frac=0.02),
}


def rng(seed: int, *key: int) -> np.random.Generator:
    """Independent stream for (seed, key...)."""
    ss = np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.SFC64(ss))


# --------------------------------------------------------------------------
# Storage dtype conversion (nearest, ties to even; exactly one rounding)
# --------------------------------------------------------------------------

def to_bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), nearest-even, one rounding."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    f, e = np.frexp(ax)                       # ax = f * 2^e, f in [0.5, 1)
    normal = np.ldexp(np.rint(f * 256.0), e - 8)
    sub = np.rint(ax * 2.0 ** 133) * 2.0 ** -133
    v = np.where(e - 1 < -126, sub, normal)
    v = np.where(ax == 0.0, 0.0, v)
    with np.errstate(over="ignore"):
        bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = bits | np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_storage(x, dtype: str) -> np.ndarray:
    """float64 -> stored array: uint16 bf16 bits, or float32."""
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def storage_to_f64(a, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Page recipes
# --------------------------------------------------------------------------

def lowrank_pages(g: np.random.Generator, n_pages: int, P: int, d: int, rank: int = 8,
                  noise: float = 0.1) -> np.ndarray:
    A = g.standard_normal((n_pages, P, rank))
    Bm = g.standard_normal((n_pages, rank, d)) * np.sqrt(1.0 / rank)
    N = g.standard_normal((n_pages, P, d)) * noise
    return A @ Bm + N


def haar_columns(Z: np.ndarray) -> np.ndarray:
    """Orthonormal columns from Gaussian Z (..., n, k): QR with diag(R) > 0."""
    import torch  # CPU only; batched LAPACK QR

    Q, R = torch.linalg.qr(torch.from_numpy(np.ascontiguousarray(Z)))
    sgn = torch.sign(torch.diagonal(R, dim1=-2, dim2=-1))
    sgn[sgn == 0] = 1.0
    return (Q * sgn[..., None, :]).numpy()


def spectrum_pages(g: np.random.Generator, n_pages: int, P: int, d: int,
                   decay: float = 1.2) -> np.ndarray:
    import torch

    k = min(P, d)
    U = haar_columns(g.standard_normal((n_pages, P, P)))[..., :, :k]
    W = haar_columns(g.standard_normal((n_pages, d, k)))
    sig = np.arange(1, k + 1, dtype=np.float64) ** (-decay)
    Us = torch.from_numpy(np.ascontiguousarray(U * sig[None, None, :]))
    return torch.matmul(Us, torch.from_numpy(W).transpose(-1, -2)).numpy()


def kv_head(cfg: dict, b: int, h: int, T: int, layer: int = 0):
    """float64 K and V (T, d) of one (sequence, layer, KV head)."""
    P, d, seed = cfg["P"], cfg["d"], cfg["seed"]
    n_pages = -(-T // P)
    out = []
    for kind in (KIND_K, KIND_V):
        g = rng(seed, b, layer, h, kind)
        if cfg["recipe"] == "lowrank":
            X = lowrank_pages(g, n_pages, P, d).reshape(n_pages * P, d)
            gm = rng(seed, b, layer, h, KIND_META_K if kind == KIND_K else KIND_META_V)
            X = X + gm.standard_normal(d) * np.sqrt(0.5)
            if kind == KIND_K:
                ch = gm.permutation(d)[:4]
                X[:, ch] *= 10.0
        elif cfg["recipe"] == "spectrum":
            X = spectrum_pages(g, n_pages, P, d).reshape(n_pages * P, d)
        else:
            raise ValueError(cfg["recipe"])
        out.append(X[:T])
    return out[0], out[1]


def _stored_head(args):
    cfg, b, h, T = args
    k, v = kv_head(cfg, b, h, T)
    return to_storage(k, cfg["dtype"]), to_storage(v, cfg["dtype"])


def decode_inputs(cfg_id: int, T: int | None = None, B: int | None = None,
                  kv_heads: int | None = None, with_f64: bool = False, workers: int = 1):
    """Stored K, V (B, H_kv, T, d) and q (B, H_q, d) for workload cfg_id.

    T, B and kv_heads may shrink a workload for quick tests (the recipe and
    streams are unchanged, so a shrunk input is a prefix/subset of the full
    one).  Stored arrays are uint16 (bf16 bits) or float32.  workers > 1
    generates (sequence, KV head) streams on that many threads; the
    bytes do not depend on it.
    """
    cfg = dict(CONFIGS[cfg_id])
    if T is None:
        T = cfg["T"] + cfg.get("steps", 0)
    B = cfg["B"] if B is None else B
    Hkv = cfg["Hkv"] if kv_heads is None else kv_heads
    G = cfg["Hq"] // cfg["Hkv"]
    Hq = Hkv * G
    d = cfg["d"]
    sdt = np.uint16 if cfg["dtype"] == "bf16" else np.float32
    K = np.empty((B, Hkv, T, d), dtype=sdt)
    V = np.empty((B, Hkv, T, d), dtype=sdt)
    jobs = [(cfg, b, h, T) for b in range(B) for h in range(Hkv)]
    if workers > 1 and len(jobs) > 1:
        import concurrent.futures as cf

        # bulk numpy draws and torch QR / matmul release the GIL
        with cf.ThreadPoolExecutor(max_workers=min(workers, len(jobs))) as ex:
            results = list(ex.map(_stored_head, jobs))
    else:
        results = [_stored_head(j) for j in jobs]
    for (_, b, h, _), (ks, vs) in zip(jobs, results):
        K[b, h] = ks
        V[b, h] = vs
    q = np.empty((B, Hq, d), dtype=sdt)
    for b in range(B):
        q[b] = to_storage(rng(cfg["seed"], b, 0, 0, KIND_Q).standard_normal((Hq, d)),
                          cfg["dtype"])
    res = dict(cfg=cfg, K=K, V=V, q=q, T=T, B=B, Hkv=Hkv, Hq=Hq, G=G)
    if with_f64:
        res.update(K64=storage_to_f64(K, cfg["dtype"]), V64=storage_to_f64(V, cfg["dtype"]),
                   q64=storage_to_f64(q, cfg["dtype"]))
    return res


def rope_inv_freq(base: float, d: int = 128) -> np.ndarray:
    """Rotary frequencies base^(-2m/d), m < d/2, as float32 (the values both
    sides receive; Qwen3 checkpoints use base 1e6, Llama 3.1 5e5 before its
    frequency scaling)."""
    return (float(base) ** (-np.arange(0, d, 2, dtype=np.float64) / d)).astype(np.float32)


def step_queries(cfg_id: int, step: int, B: int, Hq: int, d: int, dtype: str):
    """Query of decode step `step` (workload 4)."""
    g = rng(CONFIGS[cfg_id]["seed"], 1000 + step, 0, 0, KIND_Q)
    return to_storage(g.standard_normal((B, Hq, d)), dtype)


def noise_page_ids(seed: int, n_pages: int, frac: float) -> np.ndarray:
    """Indices of the full-rank noise pages of a batch: exactly
    round(frac * n_pages) of them, from a seeded permutation."""
    n_noise = int(round(frac * n_pages))
    perm = rng(seed, 7, 7, 7, KIND_PAGE).permutation(n_pages)
    return np.sort(perm[:n_noise])


def bf16_bits_torch(x):
    """float64 torch tensor (any device) -> int16 tensor of bfloat16 bit
    patterns, nearest-even with exactly one rounding (as to_bf16_bits): the
    float32 step rounds to odd (exact float32, else its magnitude truncated
    and the last bit set), which makes the following nearest-even step
    round as if from the double.  Finite inputs only."""
    import torch

    x32 = x.to(torch.float32)                     # nearest-even
    back = x32.to(torch.float64)
    inexact = back != x
    u = x32.view(torch.int32)
    u = torch.where(inexact & (back.abs() > x.abs()), u - 1, u)  # toward zero
    u = torch.where(inexact, u | 1, u)                            # odd
    u = u + 0x7FFF + ((u >> 16) & 1)              # float32 -> bf16 nearest-even
    return (u >> 16).to(torch.int16)


def _haar_columns_torch(Z):
    """Orthonormal columns of Gaussian Z (n, rows, k) float64 on Z's device by
    classical Gram-Schmidt applied twice per column (batched matrix-vector
    products only): column j is Z_j minus its projection on columns < j,
    divided by its norm, so R_jj > 0 -- the Q of the QR with diag(R) > 0,
    the construction of haar_columns.  The basis is kept in both orders so no
    product reads a transposed view."""
    import torch

    n, m, k = Z.shape
    Q = torch.empty_like(Z)                      # (n, m, k)
    Qt = torch.empty((n, k, m), dtype=Z.dtype, device=Z.device)
    for j in range(k):
        v = Z[:, :, j:j + 1].contiguous()
        for _ in range(2 if j else 0):
            c = torch.bmm(Qt[:, :j, :], v)       # (n, j, 1)
            v = v - torch.bmm(Q[:, :, :j], c)
        v = v / torch.linalg.vector_norm(v, dim=1, keepdim=True)
        Q[:, :, j:j + 1] = v
        Qt[:, j:j + 1, :] = v.transpose(1, 2)
    return Q


def compression_pool_device(n_total: int | None = None, device="cuda:0", cfg_id: int = 5,
                            chunk: int = 16384):
    """The batched-compression workload drawn on a torch device: int16
    tensor (n_total, P, d) of bfloat16 bit patterns (view it as bfloat16).

    Same recipe as compression_pages -- page i is U diag(i^-1.2) W^T with U
    Haar on O(64) and W 128 x 64 with Haar columns, or N(0,1) noise when i is
    one of noise_page_ids -- generated in float64 and rounded once, but drawn
    from torch's device generator: chunk c (pages c*chunk ..) from a
    generator seeded from (seed, c).  The bytes are fixed by the seed, the
    chunk size and torch's generator; they differ from compression_pages'
    per-page streams.  For pools too large to draw on the host in seconds."""
    import torch

    cfg = CONFIGS[cfg_id]
    P, d, seed = cfg["P"], cfg["d"], cfg["seed"]
    if n_total is None:
        n_total = cfg["layers"] * cfg["Hkv"] * 2 * cfg["pages_per_head"]
    noise = torch.from_numpy(noise_page_ids(seed, n_total, cfg["noise_frac"]))
    k = min(P, d)
    sig = torch.arange(1, k + 1, dtype=torch.float64, device=device) ** -1.2
    out = torch.empty((n_total, P, d), dtype=torch.int16, device=device)
    for c0 in range(0, n_total, chunk):
        n = min(chunk, n_total - c0)
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(c0 // chunk, KIND_PAGE, 99))
        g = torch.Generator(device=device)
        g.manual_seed(int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1)))
        U = _haar_columns_torch(torch.randn((n, P, P), generator=g, dtype=torch.float64, device=device))
        W = _haar_columns_torch(torch.randn((n, d, k), generator=g, dtype=torch.float64, device=device))
        X = torch.bmm((U[:, :, :k] * sig).contiguous(), W.transpose(-1, -2).contiguous())
        del U, W
        nz = noise[(noise >= c0) & (noise < c0 + n)] - c0
        if nz.numel():
            X[nz.to(device)] = torch.randn((nz.numel(), P, d), generator=g, dtype=torch.float64,
                                           device=device)
        out[c0:c0 + n] = bf16_bits_torch(X)
        del X
    return out


def compression_pages(page_ids, n_total: int | None = None, cfg_id: int = 5) -> np.ndarray:
    """float64 pages (len(page_ids), P, d) of the batched-compression workload.
    Page i is drawn from its own stream; noise pages are N(0,1)."""
    cfg = CONFIGS[cfg_id]
    P, d, seed = cfg["P"], cfg["d"], cfg["seed"]
    if n_total is None:
        n_total = cfg["layers"] * cfg["Hkv"] * 2 * cfg["pages_per_head"]
    noise = set(noise_page_ids(seed, n_total, cfg["noise_frac"]).tolist())
    ids = [int(i) for i in page_ids]
    k = min(P, d)
    Zu = np.empty((len(ids), P, P))
    Zw = np.empty((len(ids), d, k))
    Zn = {}
    for j, i in enumerate(ids):
        g = rng(seed, i, 0, 0, KIND_PAGE)
        if i in noise:
            Zn[j] = g.standard_normal((P, d))
            Zu[j] = np.eye(P)
            Zw[j] = np.eye(d, k)
        else:
            Zu[j] = g.standard_normal((P, P))
            Zw[j] = g.standard_normal((d, k))
    U = haar_columns(Zu)[..., :, :k]
    W = haar_columns(Zw)
    sig = np.arange(1, k + 1, dtype=np.float64) ** -1.2
    X = (U * sig[None, None, :]) @ np.swapaxes(W, -1, -2)
    for j, z in Zn.items():
        X[j] = z
    return X
