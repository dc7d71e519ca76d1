"""PuzzleKV page-wise low-rank KV cache for MI355X (gfx950).

Thin Python binding of ``libpkv.so`` (C-ABI in ``include/pkv.h``): argument
marshalling only.  Every step of the hot path -- page decomposition, dense
pool maintenance, append / promotion and mixed decode attention -- runs in the
library's HIP kernels; torch provides device memory and streams.  There is no
fallback: if the library is not built, every call raises.

Method: "PuzzleKV: Page-Wise Low-Rank Decomposition for KV Cache Compression"
(Sec. 3.3 steps (1)-(5), Eq. 2-5).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "capacity exceeded",
          4: "no page waiting for promotion", 5: "promotion pending", 6: "device error"}
BF16, F32, BF16_INT4 = 0, 1, 2
KEYS, VALUES, KEYS_PRE_ROPE = 0, 1, 2
UNUSED, SINK, FACT, WIN, PART = 0, 1, 2, 3, 4
PAGE_LEN, HEAD_DIM = 64, 128
NOALLOC_WORKSPACE_BYTES = 16 << 20  # PKV_NOALLOC_WORKSPACE_BYTES of include/pkv.h


class PKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "page_len", "rank_k", "rank_v", "sink",
        "window", "max_tokens", "dtype")]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "sink_k", "sink_v", "win_k", "win_v", "factors", "page_table", "total_bytes")] + \
        [(n, ctypes.c_int64) for n in (
            "n_sink_slots", "n_ring_slots", "max_fact_pages", "max_pages", "elem_bytes",
            "dense_page_bytes", "factor_k_elems", "factor_v_elems", "factor_page_bytes",
            "factor_k_bytes", "factor_v_bytes")]


_LIB = None


def lib():
    """The loaded libpkv.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_context_decode_pkv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    P = ctypes.POINTER
    sig = {
        "pkv_status_string": ([i32], ctypes.c_char_p),
        "pkv_version": ([], ctypes.c_char_p),
        "pkv_storage_ratio": ([i32, i32, i32, i32], ctypes.c_double),
        "pkv_classify": ([i64, i32, i32, i32, i64, vp, vp, i64], i32),
        "pkv_factor_part_elems": ([i32, i32, i32, i32, P(i64)], i32),
        "pkv_pack_factors": ([i32, i32, i32, i32, i32, vp, vp, vp], i32),
        "pkv_unpack_factors": ([i32, i32, i32, i32, i32, vp, vp, vp], i32),
        "pkv_factor_part_bytes": ([i32, i32, i32, i32, i32, P(i64)], i32),
        "pkv_pack_factors_int4": ([i32, i32, i32, i32, vp, vp, vp, vp, vp], i32),
        "pkv_unpack_factors_int4": ([i32, i32, i32, i32, vp, vp, vp, vp, vp], i32),
        "pkv_cache_layout": ([P(Shape), P(Layout)], i32),
        "pkv_cache_create": ([P(Shape), vp, u64, P(vp)], i32),
        "pkv_cache_destroy": ([vp], None),
        "pkv_cache_state": ([vp, P(i64), P(i64), P(i32)], i32),
        "pkv_compress_pages": ([vp, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp], i32),
        "pkv_prefill": ([vp, vp, vp, i64, vp], i32),
        "pkv_prefill_chunk": ([vp, vp, vp, i64, vp], i32),
        "pkv_append": ([vp, vp, vp, P(i32), vp], i32),
        "pkv_promote_page": ([vp, vp], i32),
        "pkv_decode_workspace_bytes": ([vp, i32, P(u64)], i32),
        "pkv_decode_attn": ([vp, vp, vp, vp, u64, i32, vp], i32),
        "pkv_decode_attn_noalloc": ([vp, vp, vp, i32, vp], i32),
        "pkv_decode_partial": ([vp, vp, vp, u64, i32, vp], i32),
        "pkv_decode_merge": ([vp, vp, u64, i32, vp, vp], i32),
        "pkv_read_page_table": ([vp, vp, vp, i64, vp], i32),
        "pkv_time_next_kernel": ([vp, vp], i32),
        "pkv_decode_step": ([vp, vp, vp, vp, vp, vp, u64, i32, vp], i32),
        "pkv_cache_set_aux_stream": ([vp, vp], i32),
        "pkv_cache_set_key_rope": ([vp, vp, i32], i32),
        "pkv_decode_attn_batch": ([vp, i32, vp, vp, vp, u64, i32, vp], i32),
        "pkv_decode_batch_workspace_bytes": ([vp, i32, i32, vp], i32),
        "pkv_decode_step_batch": ([vp, i32, vp, vp, vp, vp, vp, u64, i32, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = L
    return L


def _check(status: int, what: str):
    if status != PKV_OK:
        raise PKVError(status, what)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t}")


def _dev_ptr(t, dtype_code=None, what="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype_code is not None and _dtype_code(t.dtype) != dtype_code:
        raise ValueError(f"{what} has dtype {t.dtype}, cache dtype differs")
    return ctypes.c_void_p(t.data_ptr())


def time_next_kernel(start=None, stop=None):
    """Bracket the next decode-partial or page-decomposition kernel that this
    thread launches with two timing events (torch.cuda.Event with
    enable_timing=True): afterwards start.elapsed_time(stop) is that kernel's
    own execution time.  No arguments clears a pending request."""
    if start is None and stop is None:
        _check(lib().pkv_time_next_kernel(None, None), "pkv_time_next_kernel")
        return
    for e in (start, stop):
        if not e.cuda_event:  # torch creates the event at its first record
            e.record()
    _check(lib().pkv_time_next_kernel(ctypes.c_void_p(start.cuda_event),
                                      ctypes.c_void_p(stop.cuda_event)), "pkv_time_next_kernel")


# ------------------------------------------------------------------ host-only

def version() -> str:
    return lib().pkv_version().decode()


def storage_ratio(P: int, r_k: int, r_v: int, d: int) -> float:
    """Eq. 3: (r_K + r_V)(P + d) / (2 P d)."""
    return float(lib().pkv_storage_ratio(P, r_k, r_v, d))


def classify(T: int, P: int, s: int, w: int, n_fact: int = -1, n_pages: int | None = None):
    """(cls, slot) int32 arrays of the logical pages of a T-token cache."""
    if n_pages is None:
        n_pages = -(-T // P) if P > 0 else 0
    cls = np.zeros(n_pages, dtype=np.int32)
    slot = np.zeros(n_pages, dtype=np.int32)
    _check(lib().pkv_classify(T, P, s, w, n_fact, _np_ptr(cls), _np_ptr(slot), n_pages),
           "pkv_classify")
    return cls, slot


def factor_part_elems(kind: int, r: int, P: int = PAGE_LEN, d: int = HEAD_DIM) -> int:
    """Elements of one packed factor part of `kind` (KEYS, VALUES, KEYS_PRE_ROPE)."""
    n = ctypes.c_int64()
    _check(lib().pkv_factor_part_elems(kind, P, d, r, ctypes.byref(n)), "pkv_factor_part_elems")
    return n.value


def pack_factors(kind: int, r: int, dtype: int, Lf, Rf, P: int = PAGE_LEN) -> np.ndarray:
    """Row-major float32 Lf (P x r), Rf (r x d) -> one packed factor part
    (uint16 bf16 bits or float32)."""
    Lf = np.ascontiguousarray(Lf, dtype=np.float32)
    Rf = np.ascontiguousarray(Rf, dtype=np.float32)
    if Lf.shape != (P, r) or Rf.shape != (r, HEAD_DIM):
        raise ValueError("factor shapes do not match the part")
    n = factor_part_elems(kind, r, P)
    out = np.zeros(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    _check(lib().pkv_pack_factors(kind, P, HEAD_DIM, r, dtype, _np_ptr(Lf), _np_ptr(Rf),
                                  _np_ptr(out)), "pkv_pack_factors")
    return out


def unpack_factors(kind: int, r: int, dtype: int, packed, P: int = PAGE_LEN):
    """One packed factor part -> float32 Lf (P x r), Rf (r x d)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint16 if dtype == BF16 else np.float32)
    if packed.size < factor_part_elems(kind, r, P):
        raise ValueError("packed part too small")
    Lf = np.zeros((P, r), dtype=np.float32)
    Rf = np.zeros((r, HEAD_DIM), dtype=np.float32)
    _check(lib().pkv_unpack_factors(kind, P, HEAD_DIM, r, dtype, _np_ptr(packed),
                                    _np_ptr(Lf), _np_ptr(Rf)), "pkv_unpack_factors")
    return Lf, Rf


def factor_part_bytes(kind: int, r: int, dtype: int, P: int = PAGE_LEN, d: int = HEAD_DIM) -> int:
    n = ctypes.c_int64()
    _check(lib().pkv_factor_part_bytes(kind, P, d, r, dtype, ctypes.byref(n)), "pkv_factor_part_bytes")
    return n.value


def pack_factors_int4(kind: int, r: int, Lq, Ls, Rq, Rs, P: int = PAGE_LEN) -> np.ndarray:
    """Host packing of INT4 codes (Lq (P, r), Rq (r, 128), values -7..7) and
    scales (Ls (r,) for keys / (P,) for values, Rs (128,)) into one part
    (uint8)."""
    Lq = np.ascontiguousarray(Lq, dtype=np.int8)
    Rq = np.ascontiguousarray(Rq, dtype=np.int8)
    Ls = np.ascontiguousarray(Ls, dtype=np.float32)
    Rs = np.ascontiguousarray(Rs, dtype=np.float32)
    if Lq.shape != (P, r) or Rq.shape != (r, HEAD_DIM) or Rs.shape != (HEAD_DIM,) or \
            Ls.shape != ((r,) if kind == KEYS else (P,)):
        raise ValueError("code / scale shapes do not match the part")
    out = np.zeros(factor_part_bytes(kind, r, BF16_INT4, P=P), dtype=np.uint8)
    _check(lib().pkv_pack_factors_int4(kind, P, HEAD_DIM, r, _np_ptr(Lq), _np_ptr(Ls),
                                       _np_ptr(Rq), _np_ptr(Rs), _np_ptr(out)),
           "pkv_pack_factors_int4")
    return out


def unpack_factors_int4(kind: int, r: int, packed, P: int = PAGE_LEN):
    """Inverse of pack_factors_int4: (Lq, Ls, Rq, Rs)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size < factor_part_bytes(kind, r, BF16_INT4, P=P):
        raise ValueError("packed part too small")
    Lq = np.zeros((P, r), dtype=np.int8)
    Rq = np.zeros((r, HEAD_DIM), dtype=np.int8)
    Ls = np.zeros(r if kind == KEYS else P, dtype=np.float32)
    Rs = np.zeros(HEAD_DIM, dtype=np.float32)
    _check(lib().pkv_unpack_factors_int4(kind, P, HEAD_DIM, r, _np_ptr(packed), _np_ptr(Lq),
                                         _np_ptr(Ls), _np_ptr(Rq), _np_ptr(Rs)),
           "pkv_unpack_factors_int4")
    return Lq, Ls, Rq, Rs


def make_shape(batch, n_q_heads, n_kv_heads, rank_k, rank_v, sink, window, max_tokens, dtype,
               head_dim=HEAD_DIM, page_len=PAGE_LEN) -> Shape:
    return Shape(batch, n_q_heads, n_kv_heads, head_dim, page_len, rank_k, rank_v, sink, window,
                 max_tokens, dtype)


def cache_layout(shape: Shape) -> dict:
    lay = Layout()
    _check(lib().pkv_cache_layout(ctypes.byref(shape), ctypes.byref(lay)), "pkv_cache_layout")
    return {name: getattr(lay, name) for name, _ in Layout._fields_}


# ------------------------------------------------------------------ device

def compress_pages(X, r: int, out_dtype=None, with_sigma: bool = True):
    """Batched page decomposition: X (n, P, 128) bf16 / f32 device tensor,
    P = 64 or 32 -> Lf (n, P, r), Rf (n, r, 128) in out_dtype (default X's),
    sigma (n, r) f32."""
    import torch
    if X.dim() != 3 or X.shape[2] != HEAD_DIM:
        raise ValueError("X must be (n_pages, P, 128)")
    P = X.shape[1]
    out_dtype = X.dtype if out_dtype is None else out_dtype
    n = X.shape[0]
    Lf = torch.empty((n, P, r), dtype=out_dtype, device=X.device)
    Rf = torch.empty((n, r, HEAD_DIM), dtype=out_dtype, device=X.device)
    sg = torch.empty((n, r), dtype=torch.float32, device=X.device) if with_sigma else None
    _check(lib().pkv_compress_pages(_dev_ptr(X, what="X"), n, P, HEAD_DIM, r,
                                    _dtype_code(X.dtype), _dtype_code(out_dtype),
                                    ctypes.c_void_p(Lf.data_ptr()), ctypes.c_void_p(Rf.data_ptr()),
                                    ctypes.c_void_p(sg.data_ptr()) if sg is not None else None,
                                    _stream(X.device)), "pkv_compress_pages")
    return Lf, Rf, sg


class Cache:
    """One layer's hybrid PuzzleKV cache over a torch-owned device buffer."""

    def __init__(self, batch, n_q_heads, n_kv_heads, rank_k, rank_v, sink, window, max_tokens,
                 dtype="bf16", device="cuda:0", page_len=PAGE_LEN):
        import torch
        self.device = torch.device(device)
        if dtype in ("bf16", torch.bfloat16):
            self.dtype_code = BF16
        elif dtype in ("f32", torch.float32):
            self.dtype_code = F32
        elif dtype == "int4":  # bf16 dense pages, INT4 factor pages (Sec. 4.3)
            self.dtype_code = BF16_INT4
        else:
            raise ValueError(f"unsupported cache dtype {dtype}")
        # element type of K, V, q and the dense pages
        self.elem_code = F32 if self.dtype_code == F32 else BF16
        self.torch_dtype = torch.float32 if self.dtype_code == F32 else torch.bfloat16
        self.shape = make_shape(batch, n_q_heads, n_kv_heads, rank_k, rank_v, sink, window,
                                max_tokens, self.dtype_code, page_len=page_len)
        self.layout = cache_layout(self.shape)
        self.buffer = torch.empty(self.layout["total_bytes"], dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(lib().pkv_cache_create(ctypes.byref(self.shape), ctypes.c_void_p(self.buffer.data_ptr()),
                                      self.layout["total_bytes"], ctypes.byref(h)), "pkv_cache_create")
        self._h = h
        self._ws = None
        self._aux = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _LIB is not None:
            _LIB.pkv_cache_destroy(h)
            self._h = None

    # -- state
    def state(self):
        T, nf, pend = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib().pkv_cache_state(self._h, ctypes.byref(T), ctypes.byref(nf), ctypes.byref(pend)),
               "pkv_cache_state")
        return T.value, nf.value, bool(pend.value)

    @property
    def T(self):
        return self.state()[0]

    # -- hot path
    def prefill(self, K, V):
        """Build the cache from dense K, V [B][H_kv][T][d] (T may be 0)."""
        T = K.shape[2]
        kp = _dev_ptr(K, self.elem_code, "K") if T else None
        vp = _dev_ptr(V, self.elem_code, "V") if T else None
        _check(lib().pkv_prefill(self._h, kp, vp, T, _stream(self.device)), "pkv_prefill")

    def prefill_chunk(self, K, V):
        """Extend the cache by the chunk K, V [B][H_kv][C][d] (chunked prefill)."""
        if tuple(K.shape) != tuple(V.shape) or tuple(K.shape[:2]) != (self.shape.batch, self.shape.n_kv_heads):
            raise ValueError("K, V must both be [B][H_kv][C][d]")
        _check(lib().pkv_prefill_chunk(self._h, _dev_ptr(K, self.elem_code, "K"), _dev_ptr(V, self.elem_code, "V"),
                                       K.shape[2], _stream(self.device)), "pkv_prefill_chunk")
        if self._aux is not None and K.shape[2] > 0:
            # the aux stream may still read the chunk: torch's allocator must
            # not hand its memory out again before that work has passed
            K.record_stream(self._aux)
            V.record_stream(self._aux)

    def append(self, k, v) -> bool:
        pend = ctypes.c_int32()
        _check(lib().pkv_append(self._h, _dev_ptr(k, self.elem_code, "k"),
                                _dev_ptr(v, self.elem_code, "v"), ctypes.byref(pend),
                                _stream(self.device)), "pkv_append")
        return bool(pend.value)

    def promote(self):
        _check(lib().pkv_promote_page(self._h, _stream(self.device)), "pkv_promote_page")

    def workspace_bytes(self, n_split: int = 0) -> int:
        n = ctypes.c_uint64()
        _check(lib().pkv_decode_workspace_bytes(self._h, n_split, ctypes.byref(n)),
               "pkv_decode_workspace_bytes")
        return n.value

    def workspace(self, n_split: int = 0):
        import torch
        need = self.workspace_bytes(n_split)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode(self, q, out=None, n_split: int = 0, workspace=None):
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        ws = self.workspace(n_split) if workspace is None else workspace
        _check(lib().pkv_decode_attn(self._h, _dev_ptr(q, self.elem_code, "q"),
                                     _dev_ptr(out, None, "out"), ctypes.c_void_p(ws.data_ptr()),
                                     ws.numel(), n_split, _stream(self.device)), "pkv_decode_attn")
        return out

    def decode_noalloc(self, q, out, n_split: int = 0):
        """pkv_decode_attn_noalloc: decode attention into the caller's `out`
        with the library-held workspace (no allocation by the call)."""
        _check(lib().pkv_decode_attn_noalloc(self._h, _dev_ptr(q, self.elem_code, "q"),
                                             _dev_ptr(out, None, "out"), n_split,
                                             _stream(self.device)), "pkv_decode_attn_noalloc")
        return out

    def decode_partial(self, q, n_split: int = 0, workspace=None):
        """Eq. 4 states merged within each split, left in the workspace."""
        ws = self.workspace(n_split) if workspace is None else workspace
        _check(lib().pkv_decode_partial(self._h, _dev_ptr(q, self.elem_code, "q"),
                                        ctypes.c_void_p(ws.data_ptr()), ws.numel(), n_split,
                                        _stream(self.device)), "pkv_decode_partial")
        return ws

    def decode_merge(self, out, n_split: int = 0, workspace=None):
        """Eq. 5 merge of the workspace's partial states into out."""
        ws = self.workspace(n_split) if workspace is None else workspace
        _check(lib().pkv_decode_merge(self._h, ctypes.c_void_p(ws.data_ptr()), ws.numel(), n_split,
                                      _dev_ptr(out, None, "out"), _stream(self.device)),
               "pkv_decode_merge")
        return out

    def set_aux_stream(self, stream=None):
        """Factorize completed window pages early on `stream` (a
        torch.cuda.Stream at default priority), overlapping later steps;
        None turns it off (pkv_cache_set_aux_stream)."""
        ptr = ctypes.c_void_p(stream.cuda_stream) if stream is not None else None
        _check(lib().pkv_cache_set_aux_stream(self._h, ptr), "pkv_cache_set_aux_stream")
        self._aux = stream  # keep the stream alive while the cache uses it

    def set_key_rope(self, inv_freq=None):
        """Keys given from now on are pre-RoPE (App. D.3): they are stored and
        factorized unrotated, and attention rotates each key at its token
        index with these d/2 frequencies (None: off).  Only on an empty
        cache (pkv_cache_set_key_rope)."""
        if inv_freq is None:
            _check(lib().pkv_cache_set_key_rope(self._h, None, 0), "pkv_cache_set_key_rope")
            return
        f = np.ascontiguousarray(inv_freq, dtype=np.float32)
        _check(lib().pkv_cache_set_key_rope(self._h, _np_ptr(f), f.size), "pkv_cache_set_key_rope")

    def step(self, k, v, q, out=None, n_split: int = 0, workspace=None):
        """One decode step (pkv_decode_step): append (k, v), promote the page
        leaving the window when due, attend q over all tokens -> out."""
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        # auto split counts never exceed 512: that workspace fits any length
        ws = self.workspace(n_split or 512) if workspace is None else workspace
        _check(lib().pkv_decode_step(self._h, _dev_ptr(k, self.elem_code, "k"),
                                     _dev_ptr(v, self.elem_code, "v"),
                                     _dev_ptr(q, self.elem_code, "q"), _dev_ptr(out, None, "out"),
                                     ctypes.c_void_p(ws.data_ptr()), ws.numel(), n_split,
                                     _stream(self.device)), "pkv_decode_step")
        return out

    # -- inspection
    def page_table(self, n: int | None = None):
        if n is None:
            n = self.layout["max_pages"]
        cls = np.zeros(n, dtype=np.int32)
        slot = np.zeros(n, dtype=np.int32)
        _check(lib().pkv_read_page_table(self._h, _np_ptr(cls), _np_ptr(slot), n,
                                         _stream(self.device)), "pkv_read_page_table")
        return cls, slot

    def factor_part(self, b: int, h: int, slot: int, kind: int):
        """Device view (uint8) of one packed factor part of the pool."""
        L = self.layout
        base = L["factors"] + ((b * self.shape.n_kv_heads + h) * L["max_fact_pages"] + slot) * \
            L["factor_page_bytes"]
        kbytes = L["factor_k_bytes"]
        if kind == KEYS:
            return self.buffer[base: base + kbytes]
        return self.buffer[base + kbytes: base + L["factor_page_bytes"]]


def batch_workspace(caches, n_split: int = 0):
    """Device workspace for decode_batch / step_batch on these caches."""
    import torch
    n = len(caches)
    handles = (ctypes.c_void_p * n)(*[c._h for c in caches])
    nb = ctypes.c_uint64()
    _check(lib().pkv_decode_batch_workspace_bytes(handles, n, n_split, ctypes.byref(nb)),
           "pkv_decode_batch_workspace_bytes")
    return torch.empty(max(int(nb.value), 1), dtype=torch.uint8, device=caches[0].device)


def step_batch(caches, k, v, q, out=None, n_split: int = 0, workspace=None):
    """One decode step for a batch of sequences of different lengths, one
    Cache of batch 1 each (pkv_decode_step_batch): k, v [n][H_kv][d], q
    [n][H_q][d] -> out [n][H_q][d] float32."""
    import torch
    n = len(caches)
    handles = (ctypes.c_void_p * n)(*[c._h for c in caches])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=caches[0].device)
    if workspace is None:
        workspace = batch_workspace(caches, n_split)
    ec = caches[0].elem_code
    _check(lib().pkv_decode_step_batch(handles, n, _dev_ptr(k, ec, "k"), _dev_ptr(v, ec, "v"), _dev_ptr(q, ec, "q"),
                                       _dev_ptr(out, None, "out"), ctypes.c_void_p(workspace.data_ptr()),
                                       workspace.numel(), n_split, _stream(caches[0].device)),
           "pkv_decode_step_batch")
    return out


def decode_batch(caches, q, out=None, n_split: int = 0, workspace=None):
    """Attention for a batch of sequences of different lengths, one Cache of
    batch 1 each (pkv_decode_attn_batch): q [n][H_q][d] -> out [n][H_q][d]
    float32, row i over caches[i]."""
    import torch
    n = len(caches)
    handles = (ctypes.c_void_p * n)(*[c._h for c in caches])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=caches[0].device)
    if workspace is None:
        nb = ctypes.c_uint64()
        _check(lib().pkv_decode_batch_workspace_bytes(handles, n, n_split, ctypes.byref(nb)),
               "pkv_decode_batch_workspace_bytes")
        workspace = torch.empty(max(int(nb.value), 1), dtype=torch.uint8, device=caches[0].device)
    _check(lib().pkv_decode_attn_batch(handles, n, _dev_ptr(q, caches[0].elem_code, "q"),
                                       _dev_ptr(out, None, "out"), ctypes.c_void_p(workspace.data_ptr()),
                                       workspace.numel(), n_split, _stream(caches[0].device)),
           "pkv_decode_attn_batch")
    return out
