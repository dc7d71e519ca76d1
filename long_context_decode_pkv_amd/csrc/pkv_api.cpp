// C-ABI entry points of libpkv (declared in include/pkv.h).
//
// Host side of the hybrid cache: argument validation, device-buffer layout,
// the length / promotion state machine of PuzzleKV's incremental update
// (Sec. 3.3 "Incremental Cache Update (5)"), and kernel dispatch.  No entry
// point allocates device memory; none throws.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "pkv.h"
#include "pkv_internal.h"

using namespace pkv;

// Early factorization (pkv_cache_set_aux_stream): a window page is factorized
// on the caller's auxiliary stream as soon as its last token is written; the
// step at which it leaves the window then waits for that work and flips its
// table entry.  Pages [early_lo, early_hi) are factorized or in flight;
// ready[ring slot] marks the completion of each.
constexpr int kMaxRing = 64;

struct pkv_cache {
  pkv_shape shape;
  pkv_layout lay;
  uint8_t* base;
  int64_t T;
  int64_t n_fact;
  int32_t pending;  // a completed page waits for promotion
  hipStream_t aux = nullptr;
  hipEvent_t written = nullptr;
  hipEvent_t ready[kMaxRing] = {};
  int n_ready = 0;
  int64_t early_lo = 0, early_hi = 0;
  // pkv_prefill_chunk with an aux stream: the chunk's page decompositions run
  // there; the next call that reads the factor pool waits for chunk_ready
  hipEvent_t chunk_ready = nullptr;
  mutable bool chunk_pending = false;
  // pre-RoPE keys (pkv_cache_set_key_rope): rotary frequencies of pair (m, m + d/2)
  int rope = 0;
  float rope_freq[kD / 2] = {};
};

namespace {

thread_local KernelEvents t_kernel_events;

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int32_t check_shape(const pkv_shape* s) {
  if (!s) return PKV_ERR_INVALID_ARG;
  if (s->batch < 1 || s->n_kv_heads < 1 || s->n_q_heads < 1) return PKV_ERR_INVALID_ARG;
  if (s->n_q_heads % s->n_kv_heads) return PKV_ERR_INVALID_ARG;
  if (s->dtype != PKV_BF16 && s->dtype != PKV_F32 && s->dtype != PKV_BF16_INT4)
    return PKV_ERR_INVALID_ARG;
  if (s->page_len < 1 || s->head_dim < 1) return PKV_ERR_INVALID_ARG;
  if (s->sink < 0 || s->window < 0 || s->sink % s->page_len || s->window % s->page_len)
    return PKV_ERR_INVALID_ARG;
  const int rmax = s->page_len < s->head_dim ? s->page_len : s->head_dim;
  if (s->rank_k < 1 || s->rank_v < 1 || s->rank_k > rmax || s->rank_v > rmax)
    return PKV_ERR_INVALID_ARG;
  if (s->max_tokens < 1) return PKV_ERR_INVALID_ARG;
  if (s->head_dim != kD || (s->page_len != kP && s->page_len != kMinP)) return PKV_ERR_UNSUPPORTED;
  if (s->n_q_heads / s->n_kv_heads > kMaxG) return PKV_ERR_UNSUPPORTED;
  if (s->dtype == PKV_BF16_INT4 && (s->rank_k > kQ4MaxRank || s->rank_v > kQ4MaxRank))
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

void make_layout(const pkv_shape* s, pkv_layout* L) {
  std::memset(L, 0, sizeof(*L));
  const int64_t P = s->page_len, d = s->head_dim, B = s->batch, H = s->n_kv_heads;
  const int64_t n_s = s->sink / P, n_w = s->window / P;
  L->elem_bytes = s->dtype == PKV_F32 ? 4 : 2;
  L->n_sink_slots = n_s;
  L->n_ring_slots = n_w + 1;
  L->max_pages = (s->max_tokens + P - 1) / P;
  const int64_t fmax = s->max_tokens / P - n_s - n_w;
  L->max_fact_pages = fmax > 0 ? fmax : 0;
  L->dense_page_bytes = P * d * L->elem_bytes;
  L->factor_k_elems = part_elems(PKV_KEYS, s->rank_k, (int)P);
  // (INT4 value parts keep the padded code count of their own layout)
  L->factor_v_elems = part_elems(s->dtype == PKV_BF16_INT4 ? PKV_KEYS : PKV_VALUES, s->rank_v, (int)P);
  if (s->dtype == PKV_BF16_INT4) {
    L->factor_k_bytes = q4_dims(s->rank_k, (int)P).k_bytes;
    L->factor_v_bytes = q4_dims(s->rank_v, (int)P).v_bytes;
  } else {
    L->factor_k_bytes = L->factor_k_elems * L->elem_bytes;
    L->factor_v_bytes = L->factor_v_elems * L->elem_bytes;
  }
  L->factor_page_bytes = L->factor_k_bytes + L->factor_v_bytes;
  uint64_t off = 0;
  const uint64_t sink_bytes = (uint64_t)B * H * n_s * L->dense_page_bytes;
  const uint64_t ring_bytes = (uint64_t)B * H * (n_w + 1) * L->dense_page_bytes;
  L->sink_k = off;
  off = align_up(off + sink_bytes);
  L->sink_v = off;
  off = align_up(off + sink_bytes);
  L->win_k = off;
  off = align_up(off + ring_bytes);
  L->win_v = off;
  off = align_up(off + ring_bytes);
  L->factors = off;
  off = align_up(off + (uint64_t)B * H * L->max_fact_pages * L->factor_page_bytes);
  L->page_table = off;
  off = align_up(off + (uint64_t)L->max_pages * 4);
  L->total_bytes = off;
}

CacheGeom geom_of(const pkv_cache* c) {
  CacheGeom g;
  g.B = c->shape.batch;
  g.Hkv = c->shape.n_kv_heads;
  g.Hq = c->shape.n_q_heads;
  g.G = g.Hq / g.Hkv;
  g.P = c->shape.page_len;
  g.n_s = c->shape.sink / c->shape.page_len;
  g.n_w = c->shape.window / c->shape.page_len;
  g.F_max = c->lay.max_fact_pages;
  g.max_pages = c->lay.max_pages;
  g.dtype = c->shape.dtype;
  g.r_k = c->shape.rank_k;
  g.r_v = c->shape.rank_v;
  g.base = c->base;
  g.lay = c->lay;
  g.rope = c->rope;
  std::memcpy(g.rope_freq, c->rope_freq, sizeof(g.rope_freq));
  return g;
}

int32_t dev_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_DEVICE; }

// Steady-state number of factorized pages at length T.
int64_t steady_fact(int64_t T, int64_t P, int64_t n_s, int64_t n_w) {
  const int64_t f = T / P - n_s - n_w;
  return f > 0 ? f : 0;
}

float bf16_round_host(float x, uint16_t* bits) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  uint16_t b;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    b = (uint16_t)((u >> 16) | 0x40u);
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    b = (uint16_t)(u >> 16);
  }
  *bits = b;
  uint32_t w = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return f;
}

// Pages [p_lo, ...) of the recent-window ring (page p in ring slot
// (p - n_s) mod (n_w + 1), value pages stored transposed), factorized into
// factor slots p - n_s.
CompressSrc ring_src(const pkv_cache* c, int64_t p_lo) {
  const CacheGeom g = geom_of(c);
  const int64_t ppg = (int64_t)g.P * kD;
  CompressSrc src;
  std::memset(&src, 0, sizeof(src));
  src.base[0] = c->base + c->lay.win_k;
  src.base[1] = c->base + c->lay.win_v;
  src.trans[0] = 0;
  src.trans[1] = 1;
  src.bh_stride = (int64_t)(g.n_w + 1) * ppg;
  src.f_stride = ppg;
  src.in_f0 = p_lo - g.n_s;
  src.f_mod = g.n_w + 1;
  src.out_f0 = p_lo - g.n_s;
  return src;
}

// Whole pages of caller-owned K, V [B][H_kv][T][d] from row `row0` on, the
// k-th factorized into factor slot out_f0 + k.
CompressSrc dense_src(const pkv_cache* c, const void* K, const void* V, int64_t T, int64_t row0,
                      int64_t out_f0) {
  const int64_t esz = c->lay.elem_bytes;
  CompressSrc src;
  std::memset(&src, 0, sizeof(src));
  src.base[0] = (const uint8_t*)K + row0 * kD * esz;
  src.base[1] = (const uint8_t*)V + row0 * kD * esz;
  src.bh_stride = T * kD;
  src.f_stride = (int64_t)c->shape.page_len * kD;
  src.out_f0 = out_f0;
  return src;
}

// The job that decomposes n0 pages of `a` then n1 pages of `b` into the
// factor pool.
CompressJob factor_job(const pkv_cache* c, const CompressSrc& a, int64_t n0, const CompressSrc& b, int64_t n1) {
  const CacheGeom g = geom_of(c);
  CompressJob job;
  std::memset(&job, 0, sizeof(job));
  job.n_kind = 2;
  job.page_rows = g.P;
  job.n_f = n0 + n1;
  job.n_f_src0 = n0;
  job.n_pages = (int64_t)g.B * g.Hkv * job.n_f * 2;
  job.src[0] = a;
  job.src[1] = b;
  job.in_dtype = dense_dtype(g.dtype);
  job.rank[0] = g.r_k;
  job.rank[1] = g.r_v;
  job.out_dtype = g.dtype;
  job.key_part_kind = c->rope ? PKV_KEYS_PRE_ROPE : PKV_KEYS;
  job.fac = c->base + c->lay.factors;
  job.fac_bh_pages = g.F_max;
  job.page_bytes = c->lay.factor_page_bytes;
  job.k_part_bytes = c->lay.factor_k_bytes;
  return job;
}

// Decomposition of n0 pages of `a` then n1 pages of `b` into the factor pool,
// one launch on `s` (nothing when n0 + n1 == 0).
hipError_t factorize(const pkv_cache* c, const CompressSrc& a, int64_t n0, const CompressSrc& b,
                     int64_t n1, hipStream_t s) {
  if (n0 < 0 || n1 < 0) return hipErrorInvalidValue;
  if (n0 + n1 == 0) return hipSuccess;
  return launch_compress(factor_job(c, a, n0, b, n1), s);
}

// Factorize window pages [p_lo, p_hi) from their ring slots on `s`.
hipError_t factorize_ring(const pkv_cache* c, int64_t p_lo, int64_t p_hi, hipStream_t s) {
  return factorize(c, ring_src(c, p_lo), p_hi - p_lo, ring_src(c, p_lo), 0, s);
}

// The page leaving the window (n_s + n_fact) becomes FACT: factorized now, or
// (early factorization) waited for on `stream`; then its table entry flips.
int32_t promote_now(pkv_cache* c, void* stream) {
  const CacheGeom g = geom_of(c);
  const int64_t f = c->n_fact;            // factor slot of the page
  const int64_t p_old = g.n_s + f;        // logical page leaving the window
  if (f >= g.F_max) return PKV_ERR_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  bool entry_set = false;
  if (c->early_lo <= p_old && p_old < c->early_hi) {
    e = hipStreamWaitEvent(s, c->ready[f % (g.n_w + 1)], 0);
    c->early_lo = p_old + 1;
  } else {
    // one launch: the decomposition also writes the page's table entry
    CompressBatch jb;
    std::memset(&jb, 0, sizeof(jb));
    jb.base = factor_job(c, ring_src(c, p_old), 1, ring_src(c, p_old), 0);
    jb.n = 1;
    jb.m[0] = CompressMember{c->base + c->lay.win_k, c->base + c->lay.win_v, c->base + c->lay.factors, g.F_max, f, f,
                             (int32_t*)(c->base + c->lay.page_table), p_old, table_entry(PKV_PAGE_FACT, (int)f)};
    e = launch_compress_batch(jb, s);
    if (e == hipErrorNotSupported) {  // ranks above 32: the decomposition, then the entry
      (void)hipGetLastError();
      e = factorize_ring(c, p_old, p_old + 1, s);
    } else {
      entry_set = true;
    }
  }
  if (e == hipSuccess && !entry_set) e = launch_table_set(g, p_old, table_entry(PKV_PAGE_FACT, (int)f), s);
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  c->n_fact += 1;
  return PKV_OK;
}

// After the launch that wrote the last token of window page p: factorize it
// on the auxiliary stream, ordered after that launch.
int32_t factorize_early(pkv_cache* c, int64_t p, hipStream_t main) {
  const CacheGeom g = geom_of(c);
  if (p - g.n_s >= g.F_max) return PKV_OK;  // never leaves the window within capacity
  hipError_t e = hipEventRecord(c->written, main);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->aux, c->written, 0);
  if (e == hipSuccess) e = factorize_ring(c, p, p + 1, c->aux);
  if (e == hipSuccess) e = hipEventRecord(c->ready[(p - g.n_s) % (g.n_w + 1)], c->aux);
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  if (c->early_lo == c->early_hi) c->early_lo = p;
  c->early_hi = p + 1;
  return PKV_OK;
}

void release_aux(pkv_cache* c) {
  if (c->written) (void)hipEventDestroy(c->written);
  if (c->chunk_ready) (void)hipEventDestroy(c->chunk_ready);
  for (int i = 0; i < c->n_ready; ++i) (void)hipEventDestroy(c->ready[i]);
  c->written = nullptr;
  c->chunk_ready = nullptr;
  c->chunk_pending = false;
  c->n_ready = 0;
  c->aux = nullptr;
  c->early_lo = c->early_hi = 0;
}

// Order `s` after the chunk decompositions still running on the aux stream
// (the factor slots they write are read by the caller's next work).
hipError_t wait_chunk(const pkv_cache* c, hipStream_t s) {
  if (!c->chunk_pending) return hipSuccess;
  const hipError_t e = hipStreamWaitEvent(s, c->chunk_ready, 0);
  if (e == hipSuccess) c->chunk_pending = false;
  return e;
}

// Order `s` after every early factorization still in flight (they read ring
// slots and write factor slots that a prefill or chunk overwrites).
hipError_t wait_early(const pkv_cache* c, hipStream_t s) {
  if (!c->aux || c->early_lo >= c->early_hi) return hipSuccess;
  for (int i = 0; i < c->n_ready; ++i) {
    const hipError_t e = hipStreamWaitEvent(s, c->ready[i], 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


}  // namespace

namespace pkv {
KernelEvents take_kernel_events() {
  const KernelEvents e = t_kernel_events;
  t_kernel_events = KernelEvents{};
  return e;
}
}  // namespace pkv

extern "C" {

const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PKV_ERR_CAPACITY: return "capacity exceeded";
    case PKV_ERR_NOT_ELIGIBLE: return "no page waiting for promotion";
    case PKV_ERR_PROMOTION_PENDING: return "promotion pending";
    case PKV_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

double pkv_storage_ratio(int32_t P, int32_t r_k, int32_t r_v, int32_t d) {
  if (P <= 0 || d <= 0) return NAN;
  return (double)(r_k + r_v) * (double)(P + d) / (2.0 * P * d);
}

int32_t pkv_classify(int64_t T, int32_t P, int32_t s, int32_t w, int64_t n_fact, int32_t* cls,
                     int32_t* slot, int64_t n_pages) {
  if (P < 1 || s < 0 || w < 0 || s % P || w % P || T < 0 || n_pages < 0) return PKV_ERR_INVALID_ARG;
  if (n_pages > 0 && (!cls || !slot)) return PKV_ERR_INVALID_ARG;
  const int64_t n_s = s / P, n_w = w / P;
  const int64_t n_full = T / P, used = (T + P - 1) / P;
  const int64_t nf = n_fact < 0 ? steady_fact(T, P, n_s, n_w) : n_fact;
  if (nf > (n_full - n_s > 0 ? n_full - n_s : 0)) return PKV_ERR_INVALID_ARG;
  for (int64_t p = 0; p < n_pages; ++p) {
    int32_t c, sl = 0;
    if (p >= used) {
      c = PKV_PAGE_UNUSED;
    } else if (p < n_s) {
      c = PKV_PAGE_SINK;
      sl = (int32_t)p;
    } else if (p < n_s + nf) {
      c = PKV_PAGE_FACT;
      sl = (int32_t)(p - n_s);
    } else {
      c = p < n_full ? PKV_PAGE_WIN : PKV_PAGE_PART;
      sl = (int32_t)((p - n_s) % (n_w + 1));
    }
    cls[p] = c;
    slot[p] = sl;
  }
  return PKV_OK;
}

int32_t pkv_factor_part_elems(int32_t kind, int32_t P, int32_t d, int32_t r, int64_t* elems) {
  if (!elems || (kind != PKV_KEYS && kind != PKV_VALUES && kind != PKV_KEYS_PRE_ROPE))
    return PKV_ERR_INVALID_ARG;
  if ((P != kP && P != kMinP) || d != kD) return PKV_ERR_UNSUPPORTED;
  if (r < 1 || r > P) return PKV_ERR_INVALID_ARG;
  *elems = part_elems(kind, r, P);
  return PKV_OK;
}

int32_t pkv_pack_factors(int32_t kind, int32_t P, int32_t d, int32_t r, int32_t dtype,
                         const float* Lf, const float* Rf, void* packed) {
  int64_t n;
  int32_t st = pkv_factor_part_elems(kind, P, d, r, &n);
  if (st != PKV_OK) return st;
  if ((dtype != PKV_BF16 && dtype != PKV_F32) || !Lf || !Rf || !packed)
    return PKV_ERR_INVALID_ARG;
  const PackDims pd = pack_dims(r, P);
  const int r8 = 8 * pd.n8;
  auto put = [&](int64_t idx, float v) {
    if (dtype == PKV_BF16) {
      uint16_t b;
      bf16_round_host(v, &b);
      ((uint16_t*)packed)[idx] = b;
    } else {
      ((float*)packed)[idx] = v;
    }
  };
  const int r_rf = kind == PKV_VALUES ? pd.r2 : r8;  // ranks the Rf operand stores
  for (int i = 0; i < r8; ++i) {
    for (int c = 0; c < kD && i < r_rf; ++c) {
      const float v = i < r ? Rf[(int64_t)i * kD + c] : 0.f;
      put(off_rf(kind, pd, i, c), v);
    }
    for (int j = 0; j < P; ++j) {
      const float v = i < r ? Lf[(int64_t)j * r + i] : 0.f;
      put(off_lf(kind, pd, j, i), v);
    }
  }
  return PKV_OK;
}

int32_t pkv_unpack_factors(int32_t kind, int32_t P, int32_t d, int32_t r, int32_t dtype,
                           const void* packed, float* Lf, float* Rf) {
  int64_t n;
  int32_t st = pkv_factor_part_elems(kind, P, d, r, &n);
  if (st != PKV_OK) return st;
  if ((dtype != PKV_BF16 && dtype != PKV_F32) || !Lf || !Rf || !packed)
    return PKV_ERR_INVALID_ARG;
  const PackDims pd = pack_dims(r, P);
  auto get = [&](int64_t idx) -> float {
    if (dtype == PKV_BF16) {
      uint32_t w = (uint32_t)((const uint16_t*)packed)[idx] << 16;
      float f;
      std::memcpy(&f, &w, 4);
      return f;
    }
    return ((const float*)packed)[idx];
  };
  for (int i = 0; i < r; ++i) {
    for (int c = 0; c < kD; ++c)
      Rf[(int64_t)i * kD + c] = get(off_rf(kind, pd, i, c));
    for (int j = 0; j < P; ++j)
      Lf[(int64_t)j * r + i] = get(off_lf(kind, pd, j, i));
  }
  return PKV_OK;
}

int32_t pkv_factor_part_bytes(int32_t kind, int32_t P, int32_t d, int32_t r, int32_t dtype,
                              int64_t* bytes) {
  if (!bytes || (kind != PKV_KEYS && kind != PKV_VALUES && kind != PKV_KEYS_PRE_ROPE))
    return PKV_ERR_INVALID_ARG;
  if ((P != kP && P != kMinP) || d != kD) return PKV_ERR_UNSUPPORTED;
  if (r < 1 || r > P) return PKV_ERR_INVALID_ARG;
  if (dtype == PKV_BF16 || dtype == PKV_F32) {
    *bytes = part_elems(kind, r, P) * (dtype == PKV_BF16 ? 2 : 4);
    return PKV_OK;
  }
  if (dtype != PKV_BF16_INT4) return PKV_ERR_INVALID_ARG;
  if (r > kQ4MaxRank || kind == PKV_KEYS_PRE_ROPE) return PKV_ERR_UNSUPPORTED;
  const Q4Dims q = q4_dims(r, P);
  *bytes = kind == PKV_KEYS ? q.k_bytes : q.v_bytes;
  return PKV_OK;
}

namespace {

int32_t check_q4_part(int32_t kind, int32_t P, int32_t d, int32_t r) {
  if ((P != kP && P != kMinP) || d != kD) return PKV_ERR_UNSUPPORTED;
  if (kind != PKV_KEYS && kind != PKV_VALUES) return PKV_ERR_INVALID_ARG;
  if (r < 1 || r > P) return PKV_ERR_INVALID_ARG;
  if (r > kQ4MaxRank) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

void put_nibble(uint8_t* part, const Q4Slot& s, int code) {
  const int byte = s.bit / 8, sh = s.bit % 8;
  uint8_t& b = part[s.byte + byte];
  b = (uint8_t)((b & ~(0xF << sh)) | ((code + 8) << sh));
}

int get_nibble(const uint8_t* part, const Q4Slot& s) {
  return ((part[s.byte + s.bit / 8] >> (s.bit % 8)) & 0xF) - 8;
}

void put_scale(uint8_t* part, int64_t byte, float v) {
  uint16_t b;
  bf16_round_host(v, &b);
  std::memcpy(part + byte, &b, 2);
}

float get_scale(const uint8_t* part, int64_t byte) {
  uint16_t b;
  std::memcpy(&b, part + byte, 2);
  const uint32_t w = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return f;
}

}  // namespace

int32_t pkv_pack_factors_int4(int32_t kind, int32_t P, int32_t d, int32_t r, const int8_t* Lq,
                              const float* Ls, const int8_t* Rq, const float* Rs, void* packed) {
  const int32_t st = check_q4_part(kind, P, d, r);
  if (st != PKV_OK) return st;
  if (!Lq || !Ls || !Rq || !Rs || !packed) return PKV_ERR_INVALID_ARG;
  for (int64_t n = 0; n < (int64_t)P * r; ++n)
    if (Lq[n] < -7 || Lq[n] > 7) return PKV_ERR_INVALID_ARG;
  for (int64_t n = 0; n < (int64_t)r * kD; ++n)
    if (Rq[n] < -7 || Rq[n] > 7) return PKV_ERR_INVALID_ARG;
  const Q4Dims q = q4_dims(r, P);
  const bool keys = kind == PKV_KEYS;
  uint8_t* part = (uint8_t*)packed;
  // every nibble starts as code 0 and every byte not holding a code or a
  // scale as 0x88
  std::memset(part, 0x88, (size_t)(keys ? q.k_bytes : q.v_bytes));
  const int r8 = 8 * q.pd.n8;
  for (int i = 0; i < r8; ++i) {
    for (int c = 0; c < kD; ++c) {
      const int code = i < r ? Rq[(int64_t)i * kD + c] : 0;
      put_nibble(part, keys ? q4_rt_k(q, i, c) : q4_rt_v(q, i, c), code);
    }
    for (int j = 0; j < P; ++j) {
      const int code = i < r ? Lq[(int64_t)j * r + i] : 0;
      put_nibble(part, keys ? q4_lt_k(q, j, i) : q4_lt_v(q, j, i), code);
    }
  }
  for (int c = 0; c < kD; ++c) put_scale(part, keys ? q4_sr_k(q, c) : q4_sr_v(q, c), Rs[c]);
  if (keys) {
    for (int i = 0; i < r8; ++i) put_scale(part, q4_sl_k(q, i), i < r ? Ls[i] : 0.f);
  } else {
    for (int j = 0; j < P; ++j) put_scale(part, q4_sl_v(q, j), Ls[j]);
  }
  return PKV_OK;
}

int32_t pkv_unpack_factors_int4(int32_t kind, int32_t P, int32_t d, int32_t r, const void* packed,
                                int8_t* Lq, float* Ls, int8_t* Rq, float* Rs) {
  const int32_t st = check_q4_part(kind, P, d, r);
  if (st != PKV_OK) return st;
  if (!Lq || !Ls || !Rq || !Rs || !packed) return PKV_ERR_INVALID_ARG;
  const Q4Dims q = q4_dims(r, P);
  const bool keys = kind == PKV_KEYS;
  const uint8_t* part = (const uint8_t*)packed;
  for (int i = 0; i < r; ++i) {
    for (int c = 0; c < kD; ++c)
      Rq[(int64_t)i * kD + c] = (int8_t)get_nibble(part, keys ? q4_rt_k(q, i, c) : q4_rt_v(q, i, c));
    for (int j = 0; j < P; ++j)
      Lq[(int64_t)j * r + i] = (int8_t)get_nibble(part, keys ? q4_lt_k(q, j, i) : q4_lt_v(q, j, i));
  }
  for (int c = 0; c < kD; ++c) Rs[c] = get_scale(part, keys ? q4_sr_k(q, c) : q4_sr_v(q, c));
  if (keys) {
    for (int i = 0; i < r; ++i) Ls[i] = get_scale(part, q4_sl_k(q, i));
  } else {
    for (int j = 0; j < P; ++j) Ls[j] = get_scale(part, q4_sl_v(q, j));
  }
  return PKV_OK;
}

int32_t pkv_cache_layout(const pkv_shape* shape, pkv_layout* out) {
  int32_t st = check_shape(shape);
  if (st != PKV_OK) return st;
  if (!out) return PKV_ERR_INVALID_ARG;
  make_layout(shape, out);
  return PKV_OK;
}

int32_t pkv_cache_create(const pkv_shape* shape, void* device_buffer, uint64_t device_bytes,
                         pkv_cache** out) {
  int32_t st = check_shape(shape);
  if (st != PKV_OK) return st;
  if (!out || !device_buffer || !aligned(device_buffer, kAlign)) return PKV_ERR_INVALID_ARG;
  pkv_layout lay;
  make_layout(shape, &lay);
  if (device_bytes < lay.total_bytes) return PKV_ERR_CAPACITY;
  pkv_cache* c = new (std::nothrow) pkv_cache;
  if (!c) return PKV_ERR_INVALID_ARG;
  c->shape = *shape;
  c->lay = lay;
  c->base = (uint8_t*)device_buffer;
  c->T = 0;
  c->n_fact = 0;
  c->pending = 0;
  *out = c;
  return PKV_OK;
}

void pkv_cache_destroy(pkv_cache* cache) {
  if (!cache) return;
  release_aux(cache);
  delete cache;
}

int32_t pkv_cache_set_aux_stream(pkv_cache* c, void* aux_stream) {
  if (!c) return PKV_ERR_INVALID_ARG;
  if (c->aux) {
    // work already queued there must finish before its events go away
    if (c->early_lo < c->early_hi || c->chunk_pending) return PKV_ERR_PROMOTION_PENDING;
    release_aux(c);
  }
  if (!aux_stream) return PKV_OK;
  const int ring = c->lay.n_ring_slots;
  if (ring > kMaxRing) return PKV_ERR_UNSUPPORTED;
  if (hipEventCreateWithFlags(&c->written, hipEventDisableTiming) != hipSuccess) return PKV_ERR_DEVICE;
  if (hipEventCreateWithFlags(&c->chunk_ready, hipEventDisableTiming) != hipSuccess) {
    release_aux(c);
    return PKV_ERR_DEVICE;
  }
  for (int i = 0; i < ring; ++i) {
    if (hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming) != hipSuccess) {
      release_aux(c);
      return PKV_ERR_DEVICE;
    }
    c->n_ready = i + 1;
  }
  c->aux = (hipStream_t)aux_stream;
  c->early_lo = c->early_hi = 0;
  return PKV_OK;
}

int32_t pkv_cache_set_key_rope(pkv_cache* c, const float* inv_freq, int32_t n_freq) {
  if (!c) return PKV_ERR_INVALID_ARG;
  if (c->shape.dtype == PKV_BF16_INT4) return PKV_ERR_UNSUPPORTED;
  if (c->T != 0) return PKV_ERR_INVALID_ARG;
  if (!inv_freq) {
    c->rope = 0;
    return PKV_OK;
  }
  if (n_freq != kD / 2) return PKV_ERR_INVALID_ARG;
  for (int m = 0; m < kD / 2; ++m)
    if (!std::isfinite(inv_freq[m])) return PKV_ERR_INVALID_ARG;
  std::memcpy(c->rope_freq, inv_freq, sizeof(c->rope_freq));
  c->rope = 1;
  return PKV_OK;
}

int32_t pkv_cache_state(const pkv_cache* c, int64_t* T, int64_t* n_fact, int32_t* pending) {
  if (!c) return PKV_ERR_INVALID_ARG;
  if (T) *T = c->T;
  if (n_fact) *n_fact = c->n_fact;
  if (pending) *pending = c->pending;
  return PKV_OK;
}

int32_t pkv_compress_pages(const void* X, int64_t n_pages, int32_t P, int32_t d, int32_t r,
                           int32_t in_dtype, int32_t out_dtype, void* Lf, void* Rf, float* sigma,
                           void* stream) {
  if ((P != kP && P != kMinP) || d != kD) return PKV_ERR_UNSUPPORTED;
  if (n_pages < 0 || r < 1 || r > P) return PKV_ERR_INVALID_ARG;
  if ((in_dtype != PKV_BF16 && in_dtype != PKV_F32) || (out_dtype != PKV_BF16 && out_dtype != PKV_F32))
    return PKV_ERR_INVALID_ARG;
  if (n_pages == 0) return PKV_OK;
  if (!X || !Lf || !Rf || !aligned(X, 16) || !aligned(Lf, 4) || !aligned(Rf, 4) ||
      (sigma && !aligned(sigma, 4)))
    return PKV_ERR_INVALID_ARG;
  CompressJob job;
  std::memset(&job, 0, sizeof(job));
  job.n_pages = n_pages;
  job.n_kind = 1;
  job.page_rows = P;
  job.n_f = n_pages;
  job.n_f_src0 = n_pages;
  job.src[0].base[0] = job.src[0].base[1] = X;
  job.src[0].f_stride = (int64_t)P * kD;
  job.in_dtype = in_dtype;
  job.rank[0] = job.rank[1] = r;
  job.out_dtype = out_dtype;
  job.fac = nullptr;
  job.lf = Lf;
  job.rf = Rf;
  job.sigma = sigma;
  return dev_status(launch_compress(job, (hipStream_t)stream));
}

int32_t pkv_prefill(pkv_cache* c, const void* K, const void* V, int64_t T, void* stream) {
  if (!c || T < 0) return PKV_ERR_INVALID_ARG;
  if (T > 0 && (!K || !V || !aligned(K, 16) || !aligned(V, 16))) return PKV_ERR_INVALID_ARG;
  if (T > c->shape.max_tokens) return PKV_ERR_CAPACITY;
  const CacheGeom g = geom_of(c);
  const int64_t n_fact = steady_fact(T, g.P, g.n_s, g.n_w);
  hipStream_t s = (hipStream_t)stream;
  // early factorizations and chunk decompositions still in flight read the
  // ring slots and write the factor slots this prefill overwrites
  if (wait_early(c, s) != hipSuccess || wait_chunk(c, s) != hipSuccess) return PKV_ERR_DEVICE;
  hipError_t e = launch_prefill_dense(g, K, V, T, n_fact, s);
  if (e == hipSuccess) {
    const CompressSrc src = dense_src(c, K, V, T, (int64_t)g.n_s * g.P, 0);
    e = factorize(c, src, n_fact, src, 0, s);
  }
  if (e == hipSuccess) e = launch_table_fill(g, T, n_fact, s);
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  c->T = T;
  c->n_fact = n_fact;
  c->pending = 0;
  c->early_lo = c->early_hi = 0;
  return PKV_OK;
}

int32_t pkv_prefill_chunk(pkv_cache* c, const void* K, const void* V, int64_t C, void* stream) {
  if (!c || C < 0) return PKV_ERR_INVALID_ARG;
  if (C == 0) return PKV_OK;
  if (!K || !V || !aligned(K, 16) || !aligned(V, 16)) return PKV_ERR_INVALID_ARG;
  if (c->pending) return PKV_ERR_PROMOTION_PENDING;
  const int64_t T0 = c->T, T1 = T0 + C;
  if (T1 > c->shape.max_tokens) return PKV_ERR_CAPACITY;
  const CacheGeom g = geom_of(c);
  const int64_t nf0 = c->n_fact, nf1 = steady_fact(T1, g.P, g.n_s, g.n_w);
  if (nf1 > g.F_max) return PKV_ERR_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  // early factorizations read ring slots that this chunk may overwrite
  hipError_t e = wait_early(c, s);
  const int64_t p0 = T0 / g.P;               // page of token T0
  const int64_t pc = (T0 + g.P - 1) / g.P;   // first page that starts inside the chunk
  const int64_t np1 = (T1 + g.P - 1) / g.P;  // pages at T1
  const int64_t leave_lo = g.n_s + nf0, fact_hi = g.n_s + nf1;  // pages that leave the window
  // ... of them, those in the ring at T0 (none when T0 is inside the sink)
  const int64_t ring_hi = std::max(leave_lo, std::min(fact_hi, pc));
  const int64_t chunk_lo = std::max(leave_lo, pc);               // ... and those never in it
  const int64_t n_chunk = fact_hi > chunk_lo ? fact_hi - chunk_lo : 0;
  const CompressSrc chunk = dense_src(c, K, V, C, chunk_lo * g.P - T0, chunk_lo - g.n_s);
  // ring pages already factorized on the aux stream (their factor slots are
  // written; the wait above ordered this stream after that work)
  auto clamp = [](int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); };
  const bool early = c->early_lo < c->early_hi;
  const int64_t a_hi = early ? clamp(c->early_lo, leave_lo, ring_hi) : ring_hi;
  const int64_t b_lo = early ? clamp(c->early_hi, leave_lo, ring_hi) : ring_hi;
  // 1. the page filling at T0, when it leaves the window in this chunk: its
  //    rows from the chunk first, in its ring slot
  if (e == hipSuccess && T0 % g.P != 0 && p0 >= g.n_s && p0 < fact_hi)
    e = launch_chunk_dense(g, K, V, T0, T1, p0, p0 + 1, s);
  // 2. decomposition of the pages leaving the window, as one launch: ring
  //    pages [leave_lo, a_hi) and [b_lo, ring_hi), and -- without an aux
  //    stream -- the chunk's own pages [chunk_lo, fact_hi)
  if (e == hipSuccess) {
    if (c->aux)
      e = factorize(c, ring_src(c, leave_lo), a_hi - leave_lo, ring_src(c, b_lo), ring_hi - b_lo, s);
    else
      e = factorize(c, ring_src(c, leave_lo), a_hi - leave_lo, chunk, n_chunk, s);
  }
  // 3. rows of the pages that stay dense: sink pages, then the window and
  //    the partial page (after step 2, which read the ring slots they reuse)
  if (e == hipSuccess) e = launch_chunk_dense(g, K, V, T0, T1, p0, np1 < g.n_s ? np1 : g.n_s, s);
  if (e == hipSuccess) e = launch_chunk_dense(g, K, V, T0, T1, p0 > fact_hi ? p0 : fact_hi, np1, s);
  if (e == hipSuccess) e = launch_table_fill(g, T1, nf1, s);
  // 4. with an aux stream, one launch there after the copies: the chunk's own
  //    pages, and the window's complete pages not yet factorized (early
  //    factorization: they leave the window later, and only wait for it)
  int64_t x_lo = fact_hi, x_hi = fact_hi;
  if (e == hipSuccess && c->aux) {
    x_lo = early && c->early_hi > fact_hi ? c->early_hi : fact_hi;
    x_hi = T1 / g.P < g.n_s + g.F_max ? T1 / g.P : g.n_s + g.F_max;
    if (g.n_w == 0 || x_hi < x_lo) x_hi = x_lo;
    if (x_hi > x_lo || n_chunk > 0) {
      e = hipEventRecord(c->written, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(c->aux, c->written, 0);
      if (e == hipSuccess) e = factorize(c, ring_src(c, x_lo), x_hi - x_lo, chunk, n_chunk, c->aux);
      for (int64_t p = x_lo; e == hipSuccess && p < x_hi; ++p)
        e = hipEventRecord(c->ready[(p - g.n_s) % (g.n_w + 1)], c->aux);
      if (e == hipSuccess && n_chunk > 0) {
        e = hipEventRecord(c->chunk_ready, c->aux);
        if (e == hipSuccess) c->chunk_pending = true;
      }
    }
  }
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  // early pages still in the window: the older ones that stay, then the new
  const int64_t keep_lo = early && c->early_hi > fact_hi ? (c->early_lo > fact_hi ? c->early_lo : fact_hi)
                                                        : x_lo;
  c->early_lo = keep_lo;
  c->early_hi = x_hi > keep_lo ? x_hi : keep_lo;
  if (c->early_lo >= c->early_hi) c->early_lo = c->early_hi = 0;
  c->T = T1;
  c->n_fact = nf1;
  return PKV_OK;
}

int32_t pkv_append(pkv_cache* c, const void* k_new, const void* v_new, int32_t* promotion_pending,
                   void* stream) {
  if (!c || !k_new || !v_new) return PKV_ERR_INVALID_ARG;
  if (c->pending) return PKV_ERR_PROMOTION_PENDING;
  if (c->T >= c->shape.max_tokens) return PKV_ERR_CAPACITY;
  const CacheGeom g = geom_of(c);
  hipError_t e = launch_append(g, k_new, v_new, c->T, (hipStream_t)stream);
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  c->T += 1;
  // a completed page enters the window; the oldest window page leaves it
  const int64_t n_old_ok = steady_fact(c->T, g.P, g.n_s, g.n_w);
  c->pending = n_old_ok > c->n_fact ? 1 : 0;
  if (promotion_pending) *promotion_pending = c->pending;
  return PKV_OK;
}

int32_t pkv_promote_page(pkv_cache* c, void* stream) {
  if (!c) return PKV_ERR_INVALID_ARG;
  if (!c->pending) return PKV_ERR_NOT_ELIGIBLE;
  const int32_t st = promote_now(c, stream);
  if (st == PKV_OK) c->pending = 0;
  return st;
}

int32_t pkv_decode_workspace_bytes(const pkv_cache* c, int32_t n_split, uint64_t* bytes) {
  if (!c || !bytes || n_split < 0 || n_split > kMaxDecodeSplits) return PKV_ERR_INVALID_ARG;
  const CacheGeom g = geom_of(c);
  const int ns = n_split > 0 ? n_split : decode_default_splits(g, c->T, c->n_fact);
  const uint64_t rows = (uint64_t)g.B * g.Hq * ns;
  *bytes = align_up(rows * kD * 4) + align_up(rows * 2 * 4);
  return PKV_OK;
}

namespace {

// Shared argument checks of the decode calls for a cache of length T with
// n_fact factorized pages; fills job (without out).
int32_t decode_job_at(const pkv_cache* c, int64_t T, int64_t n_fact, const void* q, void* workspace,
                      uint64_t workspace_bytes, int32_t n_split, AttnJob* job, bool allow_empty = false) {
  if (!c || !workspace || n_split < 0 || n_split > kMaxDecodeSplits) return PKV_ERR_INVALID_ARG;
  if (T < (allow_empty ? 0 : 1)) return PKV_ERR_INVALID_ARG;
  if ((q && !aligned(q, 16)) || !aligned(workspace, kAlign)) return PKV_ERR_INVALID_ARG;
  const CacheGeom g = geom_of(c);
  const int ns = n_split > 0 ? n_split : decode_default_splits(g, T, n_fact);
  const uint64_t rows = (uint64_t)g.B * g.Hq * ns;
  const uint64_t need = align_up(rows * kD * 4) + align_up(rows * 2 * 4);
  if (workspace_bytes < need) return PKV_ERR_CAPACITY;
  job->q = q;
  job->out = nullptr;
  job->ws_o = (float*)workspace;
  job->ws_ml = (float*)((uint8_t*)workspace + align_up(rows * kD * 4));
  job->n_split = ns;
  job->T = T;
  job->n_fact = n_fact;
  return PKV_OK;
}

int32_t decode_job(const pkv_cache* c, const void* q, void* workspace, uint64_t workspace_bytes,
                   int32_t n_split, AttnJob* job) {
  if (!c) return PKV_ERR_INVALID_ARG;
  return decode_job_at(c, c->T, c->n_fact, q, workspace, workspace_bytes, n_split, job);
}

}  // namespace

namespace {

// Caches a batched attention may cover together: batch 1 each, equal shape
// except max_tokens, the same pre-RoPE setting.
bool batchable(const pkv_cache* a, const pkv_cache* b) {
  const pkv_shape &x = a->shape, &y = b->shape;
  return x.batch == 1 && y.batch == 1 && x.n_q_heads == y.n_q_heads && x.n_kv_heads == y.n_kv_heads &&
         x.head_dim == y.head_dim && x.page_len == y.page_len && x.rank_k == y.rank_k &&
         x.rank_v == y.rank_v && x.sink == y.sink && x.window == y.window && x.dtype == y.dtype &&
         a->rope == b->rope && (!a->rope || std::memcmp(a->rope_freq, b->rope_freq, sizeof(a->rope_freq)) == 0);
}

// Validates a batch; split counts (the grid's in *ns, each cache's in
// ns_seq) and the workspace its attention needs.
int32_t batch_plan(const pkv_cache* const* caches, int32_t n, int32_t n_split, int* ns, int* ns_seq,
                   uint64_t* need, bool allow_empty) {
  if (!caches || n < 1 || n > kMaxBatchCaches || n_split < 0 || n_split > kMaxDecodeSplits)
    return PKV_ERR_INVALID_ARG;
  int64_t T_max = 0, nf_max = 0;
  for (int i = 0; i < n; ++i) {
    if (!caches[i] || !batchable(caches[0], caches[i]) || caches[i]->T < (allow_empty ? 0 : 1))
      return PKV_ERR_INVALID_ARG;
    if (caches[i]->T > T_max) {
      T_max = caches[i]->T;
      nf_max = caches[i]->n_fact;
    }
  }
  CacheGeom g = geom_of(caches[0]);
  g.B = n;  // the batch's (sequence, KV head) pairs
  if (n_split == 0 && batched_kernel(g)) {
    // the library's count: splits in proportion to each cache's pages
    int64_t T[kMaxBatchCaches];
    for (int i = 0; i < n; ++i) T[i] = caches[i]->T;
    *ns = decode_batch_splits(g, T, n, ns_seq);
  } else {
    // every cache's range in n_split parts (the per-cache launches of formats
    // without a batched kernel share one split count too)
    *ns = n_split > 0 ? n_split : decode_default_splits(g, T_max, nf_max);
    for (int i = 0; i < n; ++i) ns_seq[i] = *ns;
  }
  const uint64_t rows = (uint64_t)n * g.Hq * *ns;
  *need = align_up(rows * kD * 4) + align_up(rows * 2 * 4);
  return PKV_OK;
}

}  // namespace

int32_t pkv_decode_batch_workspace_bytes(const pkv_cache* const* caches, int32_t n, int32_t n_split,
                                         uint64_t* bytes) {
  if (!bytes) return PKV_ERR_INVALID_ARG;
  int ns, ns_seq[kMaxBatchCaches];
  return batch_plan(caches, n, n_split, &ns, ns_seq, bytes, true);
}

int32_t pkv_decode_attn_batch(const pkv_cache* const* caches, int32_t n, const void* q, float* out,
                              void* workspace, uint64_t workspace_bytes, int32_t n_split, void* stream) {
  int ns, ns_seq[kMaxBatchCaches];
  uint64_t need;
  const int32_t st = batch_plan(caches, n, n_split, &ns, ns_seq, &need, false);
  if (st != PKV_OK) return st;
  if (!q || !out || !workspace || !aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, kAlign))
    return PKV_ERR_INVALID_ARG;
  if (workspace_bytes < need) return PKV_ERR_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  CacheGeom gs[kMaxBatchCaches];
  int64_t T[kMaxBatchCaches], nf[kMaxBatchCaches];
  hipError_t e = hipSuccess;
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    gs[i] = geom_of(caches[i]);
    T[i] = caches[i]->T;
    nf[i] = caches[i]->n_fact;
    e = wait_chunk(caches[i], s);
  }
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  const int Hq = gs[0].Hq;
  const uint64_t rows = (uint64_t)n * Hq * ns;
  AttnJob job;
  job.q = q;
  job.out = out;
  job.ws_o = (float*)workspace;
  job.ws_ml = (float*)((uint8_t*)workspace + align_up(rows * kD * 4));
  job.n_split = ns;
  job.T = T[0];
  job.n_fact = nf[0];
  e = launch_partial_batch(gs, T, nf, ns_seq, n, job, s);
  if (e == hipErrorNotSupported) {  // no batched kernel for this format: one launch per cache
    (void)hipGetLastError();
    const int64_t esz = caches[0]->lay.elem_bytes;
    e = hipSuccess;
    for (int i = 0; i < n && e == hipSuccess; ++i) {
      AttnJob ji = job;
      ji.q = (const uint8_t*)q + (int64_t)i * Hq * kD * esz;
      ji.ws_o = job.ws_o + (int64_t)i * Hq * ns * kD;
      ji.ws_ml = job.ws_ml + (int64_t)i * Hq * ns * 2;
      ji.T = T[i];
      ji.n_fact = nf[i];
      e = launch_partial(gs[i], ji, s);
    }
  }
  if (e == hipSuccess) e = launch_merge_batch(gs, n, job, nullptr, ns_seq, s);
  return dev_status(e);
}

int32_t pkv_decode_partial(const pkv_cache* c, const void* q, void* workspace,
                           uint64_t workspace_bytes, int32_t n_split, void* stream) {
  if (!q) return PKV_ERR_INVALID_ARG;
  AttnJob job;
  int32_t st = decode_job(c, q, workspace, workspace_bytes, n_split, &job);
  if (st != PKV_OK) return st;
  if (wait_chunk(c, (hipStream_t)stream) != hipSuccess) return PKV_ERR_DEVICE;
  return dev_status(launch_partial(geom_of(c), job, (hipStream_t)stream));
}

int32_t pkv_decode_merge(const pkv_cache* c, const void* workspace, uint64_t workspace_bytes,
                         int32_t n_split, float* out, void* stream) {
  if (!out || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  AttnJob job;
  int32_t st = decode_job(c, nullptr, (void*)workspace, workspace_bytes, n_split, &job);
  if (st != PKV_OK) return st;
  job.out = out;
  return dev_status(launch_merge(geom_of(c), job, (hipStream_t)stream));
}

int32_t pkv_decode_attn(const pkv_cache* c, const void* q, float* out, void* workspace,
                        uint64_t workspace_bytes, int32_t n_split, void* stream) {
  if (!q || !out || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  AttnJob job;
  int32_t st = decode_job(c, q, workspace, workspace_bytes, n_split, &job);
  if (st != PKV_OK) return st;
  job.out = out;
  const CacheGeom g = geom_of(c);
  hipError_t e = wait_chunk(c, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_partial(g, job, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_merge(g, job, (hipStream_t)stream);
  return dev_status(e);
}

int32_t pkv_decode_attn_noalloc(const pkv_cache* c, const void* q, float* out, int32_t n_split,
                                void* stream) {
  if (!c || !q || !out || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  if (n_split < 0 || n_split > kMaxDecodeSplits) return PKV_ERR_INVALID_ARG;
  uint64_t need = 0;
  int32_t st = pkv_decode_workspace_bytes(c, n_split, &need);
  if (st != PKV_OK) return st;
  if (need > kNoAllocScratchBytes) return PKV_ERR_CAPACITY;  // before any device call
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return PKV_ERR_DEVICE;
  return pkv_decode_attn(c, q, out, ws, kNoAllocScratchBytes, n_split, stream);
}

int32_t pkv_decode_step(pkv_cache* c, const void* k_new, const void* v_new, const void* q,
                        float* out, void* workspace, uint64_t workspace_bytes, int32_t n_split,
                        void* stream) {
  if (!c || !k_new || !v_new || !q || !out) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  if (c->pending) return PKV_ERR_PROMOTION_PENDING;
  if (c->T >= c->shape.max_tokens) return PKV_ERR_CAPACITY;
  const CacheGeom g = geom_of(c);
  const int64_t T0 = c->T, T1 = T0 + 1;
  const int64_t p = T0 / g.P;               // page of the new token
  const int row = (int)(T0 % g.P);
  const bool promote = steady_fact(T1, g.P, g.n_s, g.n_w) > c->n_fact;
  const int64_t p_old = g.n_s + c->n_fact;  // page leaving the window when promote
  if (promote && c->n_fact >= g.F_max) return PKV_ERR_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  if (wait_chunk(c, s) != hipSuccess) return PKV_ERR_DEVICE;
  if (promote && p_old == p) {
    // no window (w = 0): the page the token completes is factorized at once,
    // so the token must be in place first; separate launches
    AttnJob job;
    int32_t st = decode_job_at(c, T1, c->n_fact + 1, q, workspace, workspace_bytes, n_split, &job);
    if (st != PKV_OK) return st;
    job.out = out;
    st = pkv_append(c, k_new, v_new, nullptr, stream);
    if (st == PKV_OK) st = pkv_promote_page(c, stream);
    if (st != PKV_OK) return st;
    hipError_t e = launch_partial(g, job, s);
    if (e == hipSuccess) e = launch_merge(g, job, s);
    return dev_status(e);
  }
  // Attend over the T0 cached tokens (after the promotion, which does not
  // touch the page of the new token); the merge adds the new token's state
  // and writes the token into its page.
  AttnJob job;
  int32_t st = decode_job_at(c, T0, c->n_fact + (promote ? 1 : 0), q, workspace, workspace_bytes,
                             n_split, &job, true);
  if (st != PKV_OK) return st;
  job.out = out;
  if (promote) {
    st = promote_now(c, stream);
    if (st != PKV_OK) return st;
  }
  job.k_new = k_new;
  job.v_new = v_new;
  job.app_page = p;
  job.app_row = row;
  job.app_entry = p < g.n_s ? table_entry(PKV_PAGE_SINK, (int)p)
                            : table_entry(row == g.P - 1 ? PKV_PAGE_WIN : PKV_PAGE_PART,
                                          (int)((p - g.n_s) % (g.n_w + 1)));
  hipError_t e = hipSuccess;
  if (T0 > 0) e = launch_partial(g, job, s);
  if (T0 == 0) job.n_split = 0;  // nothing cached yet: the new token alone
  if (e == hipSuccess) e = launch_merge(g, job, s);
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  c->T = T1;
  // the token completed window page p: factorize it ahead of the step at
  // which it leaves the window
  if (c->aux && row == g.P - 1 && p >= g.n_s && g.n_w > 0) return factorize_early(c, p, s);
  return PKV_OK;
}

int32_t pkv_decode_step_batch(pkv_cache* const* caches, int32_t n, const void* k_new, const void* v_new,
                              const void* q, float* out, void* workspace, uint64_t workspace_bytes,
                              int32_t n_split, void* stream) {
  int ns, ns_seq[kMaxBatchCaches];
  uint64_t need;
  int32_t st = batch_plan(caches, n, n_split, &ns, ns_seq, &need, true);
  if (st != PKV_OK) return st;
  if (!k_new || !v_new || !q || !out || !workspace || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, kAlign))
    return PKV_ERR_INVALID_ARG;
  if (workspace_bytes < need) return PKV_ERR_CAPACITY;
  // every check before anything changes
  bool one_by_one = false;
  for (int i = 0; i < n; ++i) {
    const pkv_cache* c = caches[i];
    if (c->pending) return PKV_ERR_PROMOTION_PENDING;
    if (c->T >= c->shape.max_tokens) return PKV_ERR_CAPACITY;
    const CacheGeom g = geom_of(c);
    const bool promote = steady_fact(c->T + 1, g.P, g.n_s, g.n_w) > c->n_fact;
    if (promote && c->n_fact >= g.F_max) return PKV_ERR_CAPACITY;
    // no window: the page a token completes is factorized at once, after the
    // token is in place (pkv_decode_step's separate launches)
    if (promote && g.n_s + c->n_fact == c->T / g.P) one_by_one = true;
  }
  hipStream_t s = (hipStream_t)stream;
  const CacheGeom g0 = geom_of(caches[0]);
  const int64_t esz = caches[0]->lay.elem_bytes;
  if (one_by_one) {  // the caches step in turn, reusing the workspace (one stream)
    for (int i = 0; i < n; ++i) {
      st = pkv_decode_step(caches[i], (const uint8_t*)k_new + (int64_t)i * g0.Hkv * kD * esz,
                           (const uint8_t*)v_new + (int64_t)i * g0.Hkv * kD * esz,
                           (const uint8_t*)q + (int64_t)i * g0.Hq * kD * esz, out + (int64_t)i * g0.Hq * kD,
                           workspace, workspace_bytes, ns, stream);
      if (st != PKV_OK) return st;
    }
    return PKV_OK;
  }
  for (int i = 0; i < n; ++i)
    if (wait_chunk(caches[i], s) != hipSuccess) return PKV_ERR_DEVICE;
  // promotions of the pages leaving the windows (at most one per cache):
  // pages factorized early only wait for their event; the others are
  // decomposed in one launch that also sets their table entries
  int due[kMaxBatchCaches];
  int n_due = 0;
  for (int i = 0; i < n; ++i) {
    pkv_cache* c = caches[i];
    const CacheGeom g = geom_of(c);
    if (steady_fact(c->T + 1, g.P, g.n_s, g.n_w) <= c->n_fact) continue;
    const int64_t p_old = g.n_s + c->n_fact;
    if (c->early_lo <= p_old && p_old < c->early_hi) {
      st = promote_now(c, stream);
      if (st != PKV_OK) return st;
    } else {
      due[n_due++] = i;
    }
  }
  if (n_due == 1) {
    st = promote_now(caches[due[0]], stream);
    if (st != PKV_OK) return st;
  } else if (n_due > 1) {
    CompressBatch jb;
    std::memset(&jb, 0, sizeof(jb));
    const pkv_cache* c0 = caches[due[0]];
    jb.base = factor_job(c0, ring_src(c0, g0.n_s), 1, ring_src(c0, g0.n_s), 0);
    jb.n = n_due;
    for (int k = 0; k < n_due; ++k) {
      pkv_cache* c = caches[due[k]];
      const int64_t f = c->n_fact;
      CompressMember& m = jb.m[k];
      m.src_k = c->base + c->lay.win_k;
      m.src_v = c->base + c->lay.win_v;
      m.fac = c->base + c->lay.factors;
      m.fac_bh_pages = c->lay.max_fact_pages;
      m.in_f0 = f;  // window page n_s + f sits in ring slot f mod (n_w + 1)
      m.out_f0 = f;
      m.table = (int32_t*)(c->base + c->lay.page_table);
      m.table_page = g0.n_s + f;
      m.table_entry = table_entry(PKV_PAGE_FACT, (int)f);
    }
    hipError_t e = launch_compress_batch(jb, s);
    if (e == hipErrorNotSupported) {  // ranks above 32: one launch per cache
      (void)hipGetLastError();
      for (int k = 0; k < n_due; ++k) {
        st = promote_now(caches[due[k]], stream);
        if (st != PKV_OK) return st;
      }
    } else if (e != hipSuccess) {
      return PKV_ERR_DEVICE;
    } else {
      for (int k = 0; k < n_due; ++k) caches[due[k]]->n_fact += 1;
    }
  }
  // attention over each cache's T_i tokens, then the merge with the new tokens
  CacheGeom gs[kMaxBatchCaches];
  int64_t T[kMaxBatchCaches], nf[kMaxBatchCaches];
  AttnJob apps[kMaxBatchCaches];
  for (int i = 0; i < n; ++i) {
    const pkv_cache* c = caches[i];
    gs[i] = geom_of(c);
    T[i] = c->T;
    nf[i] = c->n_fact;
    const int64_t p = c->T / gs[i].P;
    const int row = (int)(c->T % gs[i].P);
    apps[i].app_page = p;
    apps[i].app_row = row;
    apps[i].app_entry = p < gs[i].n_s ? table_entry(PKV_PAGE_SINK, (int)p)
                                      : table_entry(row == gs[i].P - 1 ? PKV_PAGE_WIN : PKV_PAGE_PART,
                                                    (int)((p - gs[i].n_s) % (gs[i].n_w + 1)));
  }
  const uint64_t rows = (uint64_t)n * g0.Hq * ns;
  AttnJob job;
  job.q = q;
  job.out = out;
  job.ws_o = (float*)workspace;
  job.ws_ml = (float*)((uint8_t*)workspace + align_up(rows * kD * 4));
  job.n_split = ns;
  job.T = T[0];
  job.n_fact = nf[0];
  hipError_t e = launch_partial_batch(gs, T, nf, ns_seq, n, job, s);
  if (e == hipErrorNotSupported) {  // no batched kernel for this format: one launch per cache
    (void)hipGetLastError();
    e = hipSuccess;
    for (int i = 0; i < n && e == hipSuccess; ++i) {
      AttnJob ji = job;
      ji.q = (const uint8_t*)q + (int64_t)i * g0.Hq * kD * esz;
      ji.ws_o = job.ws_o + (int64_t)i * g0.Hq * ns * kD;
      ji.ws_ml = job.ws_ml + (int64_t)i * g0.Hq * ns * 2;
      ji.T = T[i];
      ji.n_fact = nf[i];
      e = launch_partial(gs[i], ji, s);
    }
  }
  job.k_new = k_new;
  job.v_new = v_new;
  if (e == hipSuccess) e = launch_merge_batch(gs, n, job, apps, ns_seq, s);
  if (e != hipSuccess) return PKV_ERR_DEVICE;
  // tokens that completed a window page: factorize those pages early on the
  // caches' aux streams -- one launch when the caches share one aux stream
  int early[kMaxBatchCaches];
  int64_t early_page[kMaxBatchCaches];
  int n_early = 0;
  bool shared_aux = true;
  for (int i = 0; i < n; ++i) {
    pkv_cache* c = caches[i];
    const int64_t p = c->T / gs[i].P;
    const int row = (int)(c->T % gs[i].P);
    c->T += 1;
    if (c->aux && row == gs[i].P - 1 && p >= gs[i].n_s && gs[i].n_w > 0 && p - gs[i].n_s < gs[i].F_max) {
      shared_aux = shared_aux && (n_early == 0 || c->aux == caches[early[0]]->aux);
      early_page[n_early] = p;
      early[n_early++] = i;
    }
  }
  if (n_early > 1 && shared_aux) {
    pkv_cache* c0 = caches[early[0]];
    hipStream_t aux = c0->aux;
    CompressBatch jb;
    std::memset(&jb, 0, sizeof(jb));
    jb.base = factor_job(c0, ring_src(c0, early_page[0]), 1, ring_src(c0, early_page[0]), 0);
    jb.n = n_early;
    for (int k = 0; k < n_early; ++k) {
      pkv_cache* c = caches[early[k]];
      const int64_t f = early_page[k] - g0.n_s;  // the page keeps its WIN entry until it leaves
      jb.m[k] = CompressMember{c->base + c->lay.win_k, c->base + c->lay.win_v, c->base + c->lay.factors,
                               c->lay.max_fact_pages, f, f, nullptr, 0, 0};
    }
    hipError_t e = hipEventRecord(c0->written, s);  // after this step's launches on s
    if (e == hipSuccess) e = hipStreamWaitEvent(aux, c0->written, 0);
    if (e == hipSuccess) e = launch_compress_batch(jb, aux);
    if (e == hipErrorNotSupported) {  // ranks above 32: one launch per cache
      (void)hipGetLastError();
    } else {
      for (int k = 0; k < n_early && e == hipSuccess; ++k) {
        pkv_cache* c = caches[early[k]];
        const int64_t p = early_page[k];
        e = hipEventRecord(c->ready[(p - g0.n_s) % (g0.n_w + 1)], aux);
        if (c->early_lo == c->early_hi) c->early_lo = p;
        c->early_hi = p + 1;
      }
      return dev_status(e);
    }
  }
  for (int k = 0; k < n_early; ++k) {
    st = factorize_early(caches[early[k]], early_page[k], s);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

int32_t pkv_read_page_table(const pkv_cache* c, int32_t* cls, int32_t* slot, int64_t n,
                            void* stream) {
  if (!c || n < 0 || n > c->lay.max_pages) return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (!cls || !slot) return PKV_ERR_INVALID_ARG;
  int32_t* tmp = new (std::nothrow) int32_t[n];
  if (!tmp) return PKV_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(tmp, c->base + c->lay.page_table, n * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete[] tmp;
    return PKV_ERR_DEVICE;
  }
  for (int64_t p = 0; p < n; ++p) {
    cls[p] = table_class(tmp[p]);
    slot[p] = table_slot(tmp[p]);
  }
  delete[] tmp;
  return PKV_OK;
}

int32_t pkv_time_next_kernel(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return PKV_ERR_INVALID_ARG;
  t_kernel_events.start = (hipEvent_t)start_event;
  t_kernel_events.stop = (hipEvent_t)stop_event;
  return PKV_OK;
}

}  // extern "C"
