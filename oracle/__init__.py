"""PuzzleKV CPU oracle -- plain, slow, double-precision reference.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP path (``long_context_decode_pkv_amd``) and neither imports the other.

Source of every formula: the page "PuzzleKV: Page-Wise Low-Rank Decomposition for
KV Cache Compression" (arXiv 2608.23843).  Section / equation numbers below refer
to that page.

What the oracle computes is the plain definition of the method's result:

    o = softmax(q K^T / sqrt(d)) V                      (Sec. 3.2, Eq. 1)

where K and V equal the dense cache except that every page classified as
factorized is replaced by its rank-r truncated SVD U_r Sigma_r W_r^T (Sec. 3.2
"Truncated SVD"; Sec. 3.3 Eq. 2).  It uses no Gram matrix, no online softmax and
no split-K: those are the method's machinery, which the GPU path implements.
The page-wise Eq. 4 / Eq. 5 states are provided separately
(``page_state_factored``, ``page_state_dense``, ``merge_states``) so that a test
can show they reproduce the plain definition.

Readings taken where the pages are silent (each is listed in the design doc):
  * the sink is the first s/P pages, the window the w/P most recently completed
    pages plus the page still being filled (Sec. 3.3 (1)-(3); Sec. 4.1
    "Implementation");
  * the factor placement is Lf = U_r Sigma_r (P x r), Rf = W_r^T (r x d); the
    page's Eq. 2 puts Sigma on the right factor, the product is identical;
  * the "stored" variant rounds Lf and Rf to the cache dtype, nearest-even;
  * query head h reads KV head floor(h / G) (contiguous GQA groups);
  * no causal mask: the single decode query sees every cached token;
  * pre-RoPE keys (App. D.3 compares them with post-RoPE keys and gives no
    procedure): the cache stores and factorizes keys before rotation, and the
    attention rotates every key at its token index with the half-split channel
    pairing; the query arrives rotated.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv_oracle.so")
_LIB = None

# Page classes.  Their numeric values are the ones the C-ABI's page table
# reports (an interface value both sides must agree on, not shared code).
SINK, FACT, WIN, PART = 1, 2, 3, 4


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _build  # noqa: WPS433 (build once, on demand)
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.pkvo_svd.argtypes = [vp, ci, ci, vp, vp, vp]
        lib.pkvo_svd.restype = ci
        lib.pkvo_svd_batch.argtypes = [vp, i64, ci, ci, vp, vp, vp]
        lib.pkvo_svd_batch.restype = ci
        lib.pkvo_round_array.argtypes = [vp, i64, ci]
        lib.pkvo_round_array.restype = None
        lib.pkvo_bf16_encode.argtypes = [vp, vp, i64]
        lib.pkvo_bf16_encode.restype = None
        lib.pkvo_bf16_decode.argtypes = [vp, vp, i64]
        lib.pkvo_bf16_decode.restype = None
        lib.pkvo_num_threads.argtypes = []
        lib.pkvo_num_threads.restype = ci
        _LIB = lib
    return _LIB


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the C core uses (OMP_NUM_THREADS)."""
    return int(_lib().pkvo_num_threads())


# --------------------------------------------------------------------------
# Storage dtypes
# --------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """Nearest bfloat16 of each double, ties to even, as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _lib().pkvo_bf16_encode(_ptr(x), _ptr(out), x.size)
    return out


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _lib().pkvo_bf16_decode(_ptr(b), _ptr(out), b.size)
    return out


def round_to(x, dtype) -> np.ndarray:
    """Round to the storage dtype ('bf16', 'f32') nearest-even, back to float64.
    dtype None returns an unrounded float64 copy."""
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    mode = {"bf16": 0, "f32": 1, None: 2}[dtype]
    _lib().pkvo_round_array(_ptr(y), y.size, mode)
    return y


# --------------------------------------------------------------------------
# Truncated SVD of a page (Sec. 3.2 "Truncated SVD"; Sec. 3.3 Eq. 2)
# --------------------------------------------------------------------------

def svd(X):
    """X (n x m, n <= m) -> U (n x n), S (n,), Wt (n x m); X = U diag(S) Wt,
    S descending.  One-sided Jacobi in double; raises if it does not converge."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    n, m = X.shape
    U = np.empty((n, n))
    S = np.empty(n)
    Wt = np.empty((n, m))
    rc = _lib().pkvo_svd(_ptr(X), n, m, _ptr(U), _ptr(S), _ptr(Wt))
    if rc < 0:
        raise RuntimeError(f"oracle Jacobi SVD failed (status {rc})")
    return U, S, Wt


def svd_batch(X):
    """Batched svd over the leading axes of X (..., n, m)."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    lead = X.shape[:-2]
    n, m = X.shape[-2:]
    cnt = int(np.prod(lead)) if lead else 1
    U = np.empty(lead + (n, n))
    S = np.empty(lead + (n,))
    Wt = np.empty(lead + (n, m))
    if cnt:
        rc = _lib().pkvo_svd_batch(_ptr(X), cnt, n, m, _ptr(U), _ptr(S), _ptr(Wt))
        if rc < 0:
            raise RuntimeError(f"oracle Jacobi SVD failed (status {rc})")
    return U, S, Wt


def truncate(U, S, Wt, r):
    """Rank-r factors in the stored placement: Lf = U_r Sigma_r, Rf = W_r^T."""
    Lf = U[..., :, :r] * S[..., None, :r]
    Rf = Wt[..., :r, :].copy()
    return Lf, Rf


def factorize(X, r, store=None):
    """Rank-r factors of each page of X (..., P, d), optionally rounded to the
    storage dtype.  Returns (Lf, Rf, S) with S the page's full spectrum."""
    U, S, Wt = svd_batch(X)
    Lf, Rf = truncate(U, S, Wt, r)
    if store is not None:
        Lf = round_to(Lf, store)
        Rf = round_to(Rf, store)
    return Lf, Rf, S


# --------------------------------------------------------------------------
# INT4 factors (Sec. 4.3 "Quantization Compatibility")
# --------------------------------------------------------------------------

INT4_MAX = 7  # symmetric INT4: codes -7 .. 7


def quantize_int4(x, axis):
    """Symmetric INT4 quantization of x with one scale per group, a group
    being all entries along `axis` (Sec. 4.3).  Per group: s = max|x| / 7,
    rounded nearest-even to bfloat16 (the scale is stored at 16 bits);
    q = x / s rounded half to even, clamped to [-7, 7]; q = 0 where s = 0.
    Returns (q as int8, s as float64 with `axis` kept, length 1)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=axis, keepdims=True)
    s = round_to(amax / INT4_MAX, "bf16")
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(x / safe), -INT4_MAX, INT4_MAX)
    q = np.where(s > 0, q, 0.0)
    return q.astype(np.int8), s


def dequantize_int4(q, s):
    return q.astype(np.float64) * s


def int4_codes(U, S, Wt, r, kind):
    """Sec. 4.3: the singular values are split between the two factors,
    Lt = U_r Sigma_r^(1/2) (P x r) and Rt = Sigma_r^(1/2) W_r^T (r x d), and
    each factor is INT4-quantized: Lt column-wise for keys and row-wise for
    values, Rt column-wise for both.  Returns (Lt, Rt) unquantized and the
    codes and scales (lq, ls, rq, rs) of quantize_int4."""
    h = np.sqrt(S[..., :r])
    Lt = U[..., :, :r] * h[..., None, :]
    Rt = Wt[..., :r, :] * h[..., :, None]
    lq, ls = quantize_int4(Lt, axis=-2 if kind == "K" else -1)
    rq, rs = quantize_int4(Rt, axis=-2)
    return Lt, Rt, lq, ls, rq, rs


def int4_factors(U, S, Wt, r, kind):
    """The dequantized INT4 factors (Lt, Rt) of int4_codes."""
    _, _, lq, ls, rq, rs = int4_codes(U, S, Wt, r, kind)
    return dequantize_int4(lq, ls), dequantize_int4(rq, rs)


def stored_factors(U, S, Wt, r, store, kind):
    """The rank-r factors a cache stores: bf16 / f32 / exact (store None)
    placements of Eq. 2 (Lf = U_r Sigma_r, Rf = W_r^T, rounded), or the INT4
    factors of Sec. 4.3 (store 'int4'), as float64."""
    if store == "int4":
        return int4_factors(U, S, Wt, r, kind)
    Lf, Rf = truncate(U, S, Wt, r)
    if store:
        Lf, Rf = round_to(Lf, store), round_to(Rf, store)
    return Lf, Rf


def int4_storage_ratio(T, P, d, r_k, r_v, n_dense_pages):
    """Whole-cache storage of a T-token cache (T a multiple of P) with INT4
    factors and 16-bit scales, over its dense bf16 storage (Sec. 4.3): a
    factorized K/V page pair holds (r_K + r_V)(P + d) four-bit codes and the
    scales of its four factors (r_K per column of Lt_K, d per column of Rt_K,
    P per row of Lt_V, d per column of Rt_V); dense pages keep 2 P d bf16."""
    n_pages = T // P
    n_fact = n_pages - n_dense_pages
    fact_bytes = (r_k + r_v) * (P + d) / 2 + 2 * (r_k + d + P + d)
    dense_bytes = 2 * P * d * 2
    return (n_fact * fact_bytes + n_dense_pages * dense_bytes) / (n_pages * dense_bytes)


def optimal_error(S, r):
    """Eckart-Young-Mirsky: the best rank-r Frobenius error from the spectrum."""
    tail = np.asarray(S)[..., r:]
    return np.sqrt(np.sum(tail * tail, axis=-1))


# --------------------------------------------------------------------------
# Page classification (Sec. 3.3 (1)-(3) and "Incremental Cache Update (5)")
# --------------------------------------------------------------------------

def classify(T, P, s, w, n_fact=None):
    """Class and slot of each logical page of a T-token cache.

    Sink: the first s/P pages.  Window: the w/P most recently completed pages
    (and, while a promotion is pending, the page that has just left it).  The
    page still being filled is PART.  Every other completed page is FACT.
    n_fact=None is the steady state in which every eligible page has been
    factorized; otherwise exactly the first n_fact eligible pages are FACT.

    Slots: SINK -> p, FACT -> p - n_s (factor storage is filled in page
    order), WIN/PART -> (p - n_s) mod (n_w + 1) (a ring of window buffers).
    """
    if P <= 0 or s % P or w % P or T < 0:
        raise ValueError("s and w must be multiples of P")
    n_s, n_w = s // P, w // P
    n_pages = -(-T // P)
    cls = np.zeros(n_pages, dtype=np.int32)
    slot = np.zeros(n_pages, dtype=np.int32)
    completed = [p for p in range(n_pages) if (p + 1) * P <= T]
    non_sink_done = [p for p in completed if p >= n_s]
    if n_fact is None:
        n_elig = max(0, len(non_sink_done) - n_w)
    else:
        n_elig = n_fact
    fact_set = set(non_sink_done[:n_elig])
    for p in range(n_pages):
        if p < n_s:
            cls[p], slot[p] = SINK, p
        elif p in fact_set:
            cls[p], slot[p] = FACT, p - n_s
        elif p in completed:
            cls[p], slot[p] = WIN, (p - n_s) % (n_w + 1)
        else:
            cls[p], slot[p] = PART, (p - n_s) % (n_w + 1)
    return cls, slot


# --------------------------------------------------------------------------
# Attention (Sec. 3.2 Eq. 1) and the page-wise states (Sec. 3.3 Eq. 4, Eq. 5)
# --------------------------------------------------------------------------

def attention(q, K, V):
    """softmax(q K^T / sqrt(d)) V for q (G, d), K and V (T, d), in float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = q.shape[-1]
    scores = (q @ K.T) / math.sqrt(d)
    scores = scores - scores.max(axis=-1, keepdims=True)
    wts = np.exp(scores)
    wts = wts / wts.sum(axis=-1, keepdims=True)
    return wts @ V


def page_state_factored(q, LfK, RfK, LfV, RfV):
    """Eq. 4: (m_p, l_p, o_p) of one factorized page, contracting q with the
    small factors first: s = (q RfK^T) LfK^T / sqrt(d), o = (e^(s-m) LfV) RfV."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    s = ((q @ RfK.T) @ LfK.T) / math.sqrt(d)
    m = s.max(axis=-1)
    e = np.exp(s - m[..., None])
    return m, e.sum(axis=-1), (e @ LfV) @ RfV


def page_state_dense(q, Kp, Vp):
    """Eq. 4's state for a dense page (same triple, from stored K_p and V_p)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    s = (q @ np.asarray(Kp, dtype=np.float64).T) / math.sqrt(d)
    m = s.max(axis=-1)
    e = np.exp(s - m[..., None])
    return m, e.sum(axis=-1), e @ np.asarray(Vp, dtype=np.float64)


def merge_states(states):
    """Eq. 5: m = max_p m_p;  o = sum e^(m_p-m) o_p / sum e^(m_p-m) l_p.
    An empty state (l = 0, m = -inf) contributes nothing."""
    ms = np.stack([st[0] for st in states])
    m = ms.max(axis=0)
    num = 0.0
    den = 0.0
    for mp, lp, op in states:
        wgt = np.where(np.isneginf(mp), 0.0, np.exp(np.where(np.isneginf(mp), 0.0, mp - m)))
        num = num + wgt[..., None] * op
        den = den + wgt * lp
    return num / den[..., None]


# --------------------------------------------------------------------------
# Pre-RoPE keys (App. D.3 "RoPE Key Analysis"; rotary embedding of RoFormer,
# the page's ref. [15])
# --------------------------------------------------------------------------

def rope_rotate(X, positions, inv_freq):
    """Rotary position embedding of the rows of X (n, d): row t turns each
    channel pair (m, m + d/2) by the angle a = positions[t] * inv_freq[m]
    (the pairing of the Llama / Qwen checkpoints):
        x_m <- x_m cos a - x_{m+d/2} sin a,   x_{m+d/2} <- x_{m+d/2} cos a + x_m sin a.
    Angles and rotation in float64; inv_freq holds d/2 frequencies."""
    X = np.asarray(X, dtype=np.float64)
    h = X.shape[-1] // 2
    a = np.asarray(positions, dtype=np.float64)[:, None] * np.asarray(inv_freq, dtype=np.float64)[None, :]
    c, sn = np.cos(a), np.sin(a)
    x1, x2 = X[..., :h], X[..., h:]
    return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1)


# --------------------------------------------------------------------------
# Whole-cache decode (the quantity the GPU path is checked against)
# --------------------------------------------------------------------------

def reconstruct_cache(X, T, P, s, w, r, store, n_fact=None, with_metrics=False, kind="K"):
    """X: (T, d) dense pages of one (sequence, KV head, K or V: `kind`).
    Returns (Xhat_stored, Xhat_exact, metrics) where FACT pages are replaced
    by their rank-r truncated SVD (stored = the factors the cache keeps, see
    stored_factors)."""
    X = np.asarray(X, dtype=np.float64)[:T]
    cls, _ = classify(T, P, s, w, n_fact)
    fact = np.nonzero(cls == FACT)[0]
    Xs = X.copy()
    Xe = X.copy()
    metrics = None
    if len(fact):
        pages = np.stack([X[p * P:(p + 1) * P] for p in fact])
        U, S, Wt = svd_batch(pages)
        Lf, Rf = truncate(U, S, Wt, r)
        exact = Lf @ Rf
        Lfs, Rfs = stored_factors(U, S, Wt, r, store, kind)
        stored = Lfs @ Rfs
        for k, p in enumerate(fact):
            Xs[p * P:(p + 1) * P] = stored[k]
            Xe[p * P:(p + 1) * P] = exact[k]
        if with_metrics:
            metrics = dict(
                pages=fact,
                S=S,
                opt=optimal_error(S, r),
                norm=np.sqrt((pages ** 2).sum(axis=(-2, -1))),
                err_exact=np.sqrt(((pages - exact) ** 2).sum(axis=(-2, -1))),
                err_stored=np.sqrt(((pages - stored) ** 2).sum(axis=(-2, -1))),
            )
    return Xs, Xe, metrics


def decode(q, K, V, T, P, s, w, r_k, r_v, store, n_fact=None, kv_heads=None, key_rope=None):
    """Attention output of one decode step over a hybrid cache.

    q: (B, H_q, d); K, V: (B, H_kv, >=T, d) holding the stored (already
    dtype-rounded) values.  Returns dict(o_stored, o_exact) of shape
    (B, H_q, d); query heads of KV heads not in `kv_heads` are left NaN.

    key_rope (d/2 frequencies, or None): the cache holds pre-RoPE keys (App.
    D.3) -- pages are factorized as stored, and every key, dense or
    reconstructed, is rotated at its own position t (its token index) before
    the scores; q is taken as already rotated.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    o_s = np.full((B, Hq, d), np.nan)
    o_e = np.full((B, Hq, d), np.nan)
    heads = range(Hkv) if kv_heads is None else kv_heads
    for b in range(B):
        for h in heads:
            Ks, Ke, _ = reconstruct_cache(K[b, h], T, P, s, w, r_k, store, n_fact, kind="K")
            Vs, Ve, _ = reconstruct_cache(V[b, h], T, P, s, w, r_v, store, n_fact, kind="V")
            if key_rope is not None:
                Ks = rope_rotate(Ks, np.arange(T), key_rope)
                Ke = rope_rotate(Ke, np.arange(T), key_rope)
            qs = q[b, h * G:(h + 1) * G]
            o_s[b, h * G:(h + 1) * G] = attention(qs, Ks, Vs)
            o_e[b, h * G:(h + 1) * G] = attention(qs, Ke, Ve)
    return dict(o_stored=o_s, o_exact=o_e)


# --------------------------------------------------------------------------
# Storage accounting (Sec. 1; Sec. 3.3 Eq. 3; App. D.1 Eq. 6)
# --------------------------------------------------------------------------

def storage_ratio(P, r_k, r_v, d):
    """Eq. 3: elements of a factorized K/V page pair over its dense elements,
    counted from the factor shapes: Lf is P x r, Rf is r x d."""
    factor_elems = (P * r_k + r_k * d) + (P * r_v + r_v * d)
    dense_elems = 2 * P * d
    return factor_elems / dense_elems


def kv_cache_elements(n_layers, n_kv_heads, T, d):
    """Sec. 1: K and V of every layer and KV head, T tokens of d each."""
    return 2 * n_layers * n_kv_heads * T * d


class IncrementalDecoder:
    """Decode-step oracle for a growing cache (Sec. 3.3 (5)): a page is
    factorized once, when it becomes FACT, and never revisited, so the result
    at length T equals ``decode`` at length T; caching only saves time.

    K, V: (B, H_kv, T_max, d) float64 stored values of every token that will
    ever be appended.
    """

    def __init__(self, K, V, P, s, w, r_k, r_v, store, kv_heads=None, key_rope=None):
        self.K = np.asarray(K, dtype=np.float64)
        self.V = np.asarray(V, dtype=np.float64)
        self.key_rope = key_rope  # pre-RoPE keys, rotated at attention (see decode)
        self.P, self.s, self.w = P, s, w
        self.r = (r_k, r_v)
        self.store = store
        B, Hkv = self.K.shape[:2]
        self.heads = [(b, h) for b in range(B) for h in (range(Hkv) if kv_heads is None else kv_heads)]
        self.done = {}  # (b, h, kind, p) -> (stored, exact) reconstructions

    def _factorize_new(self, fact_pages):
        todo = [(b, h, kind, p) for (b, h) in self.heads for kind in (0, 1) for p in fact_pages
                if (b, h, kind, p) not in self.done]
        if not todo:
            return
        P = self.P
        for kind in (0, 1):
            items = [t for t in todo if t[2] == kind]
            if not items:
                continue
            src = self.K if kind == 0 else self.V
            pages = np.stack([src[b, h, p * P:(p + 1) * P] for (b, h, _, p) in items])
            U, S, Wt = svd_batch(pages)
            Lf, Rf = truncate(U, S, Wt, self.r[kind])
            exact = Lf @ Rf
            Ls, Rs = stored_factors(U, S, Wt, self.r[kind], self.store, "K" if kind == 0 else "V")
            stored = Ls @ Rs
            for k, key in enumerate(items):
                self.done[key] = (stored[k], exact[k])

    def step(self, q, T):
        """Attention outputs (o_stored, o_exact), shape (B, H_q, d), at length T
        (query heads of KV heads outside `kv_heads` are NaN)."""
        q = np.asarray(q, dtype=np.float64)
        B, Hq, d = q.shape
        Hkv = self.K.shape[1]
        G = Hq // Hkv
        cls, _ = classify(T, self.P, self.s, self.w)
        fact = [int(p) for p in np.nonzero(cls == FACT)[0]]
        self._factorize_new(fact)
        o_s = np.full((B, Hq, d), np.nan)
        o_e = np.full((B, Hq, d), np.nan)
        P = self.P
        for (b, h) in self.heads:
            Ks, Vs = self.K[b, h, :T].copy(), self.V[b, h, :T].copy()
            Ke, Ve = Ks.copy(), Vs.copy()
            for p in fact:
                Ks[p * P:(p + 1) * P], Ke[p * P:(p + 1) * P] = self.done[(b, h, 0, p)]
                Vs[p * P:(p + 1) * P], Ve[p * P:(p + 1) * P] = self.done[(b, h, 1, p)]
            if self.key_rope is not None:
                Ks = rope_rotate(Ks, np.arange(T), self.key_rope)
                Ke = rope_rotate(Ke, np.arange(T), self.key_rope)
            qs = q[b, h * G:(h + 1) * G]
            o_s[b, h * G:(h + 1) * G] = attention(qs, Ks, Vs)
            o_e[b, h * G:(h + 1) * G] = attention(qs, Ke, Ve)
        return o_s, o_e
