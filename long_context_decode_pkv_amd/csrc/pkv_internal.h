// Internal declarations shared by the HIP sources of libpkv (not part of the
// C-ABI).  Host and device code both include this header.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kP = 64;    // page length of the matrix-core layouts and kernels
constexpr int kMinP = 32;  // the other page length: 32-row pages in the 64-row frame
constexpr int kD = 128;   // head dim supported by the kernels
constexpr int kMaxG = 8;  // query heads per KV head handled by one wave
constexpr int kMaxBatchCaches = 32;    // caches of one batched attention launch
constexpr int kMaxDecodeSplits = 512;  // workgroups per (sequence, KV head) in one decode

// --------------------------------------------------------------------------
// Packed factor part layout (P = 64, d = 128).
//
// The attention kernel contracts every factor on the gfx950 matrix cores
// (v_mfma_f32_16x16x32_bf16): lane l of a wave supplies row (l % 16) of the
// A operand and the 8 reduction-index slots 8*(l/16)..+7.  The pool stores
// each operand tile in exactly that lane order, so one 64-lane load
// instruction reads a contiguous run and lands in operand registers with no
// shuffling.  Rank r is padded to r8 = 8*n8; A = 2*n8 ranks belong to each
// lane quad q = l/16 (ranks 2*n8*q .. 2*n8*q + A - 1).
//
// K part: [K1: Rf_K as the A operand of t = Rf_K q]  (r8 x d)
//         [K2: Lf_K as the A operand of s = Lf_K t]  (P x r8)
// V part: [V1: Lf_V^T as the A operand of u = Lf_V^T p] (r8 x P)
//         [V2: Rf_V^T as the A operand of o += Rf_V^T u] (d x r8)
//
// Rank tiles (K1, V1): tile mt holds a = 4mt + v (v < 4) of every lane quad;
// MFMA row rho = 4b + v carries rank 2*n8*b + 4mt + v.  When n8 is odd the
// last tile holds only v < 2 and is stored compacted (32 lanes).
// Page-row tiles (K2): MFMA row rho = 4b + v of tile mt is page row
// 16b + 4mt + v, so the score tile of lane quad q covers rows 16q..16q+15.
// --------------------------------------------------------------------------

struct PackDims {
  int P;    // page length
  int n8;   // ceil(r / 8)
  int A;    // ranks per lane quad = 2 * n8
  int RT;   // rank tiles = ceil(A / 4)
  int KS2;  // 32-wide reduction steps over the rank = ceil(A / 8)
  int r2;   // ranks V2 stores: r rounded up to even (KS2 = 1), else r8
  int nf;   // V2 (KS2 = 1): lane quads holding A ranks ...
  int ap;   // ... and the ranks of the partial quad after them (0 or even)
  int64_t k1, k2, v1, v2;  // element counts of the four operands
};

__host__ __device__ constexpr PackDims pack_dims(int r, int P = kP) {
  PackDims p{};
  p.P = P;
  p.n8 = (r + 7) / 8;
  p.A = 2 * p.n8;
  p.RT = (p.A + 3) / 4;
  p.KS2 = (p.A + 7) / 8;
  p.r2 = p.KS2 == 1 ? r + (r & 1) : 8 * p.n8;
  p.nf = p.r2 / p.A;
  p.ap = p.r2 % p.A;
  p.k1 = (int64_t)8 * p.n8 * kD;
  p.k2 = (int64_t)P * 8 * p.n8;
  p.v1 = (int64_t)8 * p.n8 * P;
  p.v2 = (int64_t)kD * p.r2;
  return p;
}

// Elements of a factor part: r8 (P + d) for key parts, r8 P + r2 d for
// value parts (V2 at the exact, even-rounded rank; the same as keys when 8
// divides r).
__host__ __device__ inline int64_t part_elems(int kind, int r, int P = kP) {
  PackDims p = pack_dims(r, P);
  return kind == PKV_VALUES ? p.v1 + p.v2 : p.k1 + p.k2;
}

// --------------------------------------------------------------------------
// Pages of P = 32 tokens keep the 64-row layout with page rows 32..63
// absent: K1 and V2 (rank x channel operands) are unchanged; K2 and V1 drop
// the lanes whose rows those are and store the rest compacted -- K2 lane
// lam = 8 qk + rho (rho < 8), 32 A elements per row tile; V1 lanes 0..31,
// 512 elements per full rank tile (a compacted last tile: lanes
// lam = 8 qk + 2 b + v with qk < 2, 256).  A part holds r8 (32 + d)
// elements.
// --------------------------------------------------------------------------

// Rank i -> (tile mt, row-in-tile rho, compact index pieces).
struct RankSlot {
  int mt, rho, b, v;
  bool partial;
};

__host__ __device__ inline RankSlot rank_slot(const PackDims& p, int i) {
  RankSlot s;
  s.b = i / p.A;
  int a = i % p.A;
  s.mt = a / 4;
  s.v = a % 4;
  s.rho = 4 * s.b + s.v;
  s.partial = (4 * s.mt + 4 > p.A);
  return s;
}

// K1: Rf_K[i][c]
__host__ __device__ inline int64_t off_rf_k(const PackDims& p, int i, int c) {
  RankSlot s = rank_slot(p, i);
  int ks = c / 32, qk = (c % 32) / 8, e = c % 8;
  int64_t base = (int64_t)s.mt * 2048;
  if (!s.partial) return base + ks * 512 + (16 * qk + s.rho) * 8 + e;
  int lam = qk * 8 + s.b * 2 + s.v;
  return base + ks * 256 + lam * 8 + e;
}

// K2: Lf_K[j][i]
__host__ __device__ inline int64_t off_lf_k(const PackDims& p, int j, int i) {
  int bq = j / 16, mt = (j % 16) / 4, vj = j % 4;
  int rho = 4 * bq + vj;
  int qk = i / p.A, a = i % p.A, ks = a / 8, e = a % 8;
  int w = (p.A - 8 * ks) < 8 ? (p.A - 8 * ks) : 8;
  if (p.P != kP) return p.k1 + (int64_t)mt * 32 * p.A + 256 * ks + (8 * qk + rho) * w + e;  // rho < 8
  int lane = 16 * qk + rho;
  return p.k1 + (int64_t)mt * 64 * p.A + 512 * ks + lane * w + e;
}

// V1: Lf_V[j][i] (stored as Lf_V^T)
__host__ __device__ inline int64_t off_lf_v(const PackDims& p, int j, int i) {
  RankSlot s = rank_slot(p, i);
  int qk = j / 16, ks = (j % 16) / 8, e = j % 8;
  const int64_t tile = p.P == kP ? 1024 : 512;  // P = 32: lanes 0..31 (qk < 2)
  int64_t base = (int64_t)s.mt * tile;
  if (!s.partial) return base + ks * (tile / 2) + (16 * qk + s.rho) * 8 + e;
  int lam = qk * 8 + s.b * 2 + s.v;
  return base + ks * (tile / 4) + lam * 8 + e;
}

// Channel-major Rf (d x r8) in the A-operand order of o += Rf^T u: channel
// tile mt, lane 16 qk + rho holds ranks A qk .. A qk + A - 1 of channel
// 16 mt + rho (offset within the operand).
__host__ __device__ inline int64_t off_rf_cm_padded(const PackDims& p, int i, int c) {
  int mt = c / 16, rho = c % 16;
  int qk = i / p.A, a = i % p.A, ks = a / 8, e = a % 8;
  int w = (p.A - 8 * ks) < 8 ? (p.A - 8 * ks) : 8;
  int lane = 16 * qk + rho;
  return (int64_t)mt * 64 * p.A + 512 * ks + lane * w + e;
}

// V2: Rf_V[i][c] (stored as Rf_V^T, i < r2).  For r8 <= 32 (KS2 = 1) the
// ranks are kept exactly, rounded up to even: channel tile mt holds 16 r2
// elements, first the partial lane quad nf (16 lanes x ap ranks), then the
// full quads 0 .. nf - 1 (16 lanes x A ranks each, lane 16 qk + rho).  When
// 8 divides r (nf = 4, ap = 0) that is the padded order.
__host__ __device__ inline int64_t off_rf_v(const PackDims& p, int i, int c) {
  if (p.KS2 > 1) return p.v1 + off_rf_cm_padded(p, i, c);
  int mt = c / 16, rho = c % 16;
  int qk = i / p.A, a = i % p.A;
  int64_t tile = p.v1 + (int64_t)mt * 16 * p.r2;
  if (qk < p.nf) return tile + 16 * p.ap + (16 * qk + rho) * p.A + a;
  return tile + rho * p.ap + a;  // the partial quad (a < ap)
}

// Rf_K of a pre-RoPE cache's key part (PKV_KEYS_PRE_ROPE): channel-major in
// the padded order (r8 ranks), at the start of the part (Lf_K follows at
// K2's offset).
__host__ __device__ inline int64_t off_rf_k_cm(const PackDims& p, int i, int c) {
  return off_rf_cm_padded(p, i, c);
}

// The offsets of a part of kind PKV_KEYS / PKV_VALUES / PKV_KEYS_PRE_ROPE.
__host__ __device__ inline int64_t off_rf(int kind, const PackDims& p, int i, int c) {
  return kind == PKV_KEYS ? off_rf_k(p, i, c) : (kind == PKV_VALUES ? off_rf_v(p, i, c) : off_rf_k_cm(p, i, c));
}
__host__ __device__ inline int64_t off_lf(int kind, const PackDims& p, int j, int i) {
  return kind == PKV_VALUES ? off_lf_v(p, j, i) : off_lf_k(p, j, i);
}

// --------------------------------------------------------------------------
// INT4 factor part layout (PuzzleKV Sec. 4.3): Lt = U_r Sigma_r^(1/2) and
// Rt = Sigma_r^(1/2) W_r^T, each held as symmetric 4-bit codes c in -7..7
// with one bf16 scale per group -- per column of Lt_K (rank), Rt_K and Rt_V
// (channel), per row of Lt_V (token).  Ranks up to 32 (one 32-wide
// reduction step over the rank, KS2 = 1).
//
// A code is stored as the nibble c + 8.  The operands keep the matrix-core
// roles and lane order of the bf16 layout above; a lane's 8 reduction slots
// of one MFMA step form one unit.  K1 / V1 units (8 channels / tokens) are
// dwords; K2 / V2 units hold the lane quad's A ranks in UB = A / 2 bytes
// (A = 2, 4, 6, 8 -> 1, 2, 3, 4 bytes; a 3-byte unit starts at any byte).
// Within a unit of W = 2 UB nibbles, element e sits at bit
// 4 ((e % 2) W / 2 + e / 2): for a dword, ((u >> 4k) & 0x000F000F) are the
// nibbles of elements 2k and 2k + 1 in the two 16-bit halves; a 3-byte unit
// holds elements 0, 2, 4 in its low 12 bits and 1, 3, 5 in its high 12.
// Padding ranks (r < 8 ceil(r / 8)) hold the nibble 8, i.e. c = 0.
//
// K part (byte offsets):  K1 codes  [tile][lane][ks 0..3] dwords; 1024 per
//                                   full tile, 512 for a compacted last tile
//                         K2 codes  [lane][mt 0..3] units
//                         sR_K      [c] bf16, c < d
//                         sL_K      [i] bf16, i < r8 (0 for padding ranks)
// V part:                 V1 codes  [tile][lane][ks 0..1] dwords; 512 / 256
//                         V2 codes  [lane][mt 0..7] units
//                         sL_V      [j] bf16, j < P
//                         sR_V      [q4][mt][v] bf16: channel 16 mt + 4 q4 + v
// Each part is padded to a multiple of 64 bytes.
// --------------------------------------------------------------------------

constexpr int kQ4MaxRank = 32;

// A rank unit holds the A codes of a lane quad (A = 2, 4, 6 or 8: one nibble
// each) in A / 2 bytes.
__host__ __device__ constexpr int q4_unit_bytes(int A) { return A / 2; }

struct Q4Dims {
  PackDims pd;
  int ub;                     // bytes of a K2 / V2 unit
  int64_t k2, sr_k, sl_k, k_bytes;
  int64_t v2, sl_v, sr_v, v_bytes;
};

// 32-token pages (P = 32) drop the lanes of page rows 32..63 from K2 and
// V1 as in the bf16 layout: K2 keeps the units of lanes l % 16 < 8 at
// lam = 8 (l / 16) + l % 16, V1 the rows of lanes 0..31 (a compacted last
// tile: rows qk * 8 + 2 b + v with qk < 2); sL_V holds P scales.
__host__ __device__ constexpr Q4Dims q4_dims(int r, int P = kP) {
  Q4Dims q{};
  q.pd = pack_dims(r, P);
  const int A = q.pd.A, full = A / 4, part = (A % 4) ? 1 : 0;
  const int64_t h = P == kP ? 1 : 2;  // lanes kept of K2 and V1: 1 / h
  q.ub = q4_unit_bytes(A);
  q.k2 = (int64_t)full * 1024 + part * 512;
  q.sr_k = q.k2 + 256LL / h * q.ub;
  q.sl_k = q.sr_k + 2LL * kD;
  q.k_bytes = (q.sl_k + 2LL * 4 * A + 63) / 64 * 64;
  q.v2 = ((int64_t)full * 512 + part * 256) / h;
  q.sl_v = q.v2 + 512LL * q.ub;
  q.sr_v = q.sl_v + 2LL * P;
  q.v_bytes = (q.sr_v + 2LL * kD + 63) / 64 * 64;
  return q;
}

__host__ __device__ inline int q4_nibble_bit(int W, int e) { return 4 * ((e % 2) * (W / 2) + e / 2); }

// Location of one code: the unit's byte offset in the part, its width in
// nibbles and the code's bit position in it.
struct Q4Slot {
  int64_t byte;
  int W;
  int bit;
};

// Row of rank i in its rank tile (full tile: lane 16 qk + rho; compacted
// tile: qk * 8 + b * 2 + v).
__host__ __device__ inline int q4_tile_row(const RankSlot& s, int qk) {
  return s.partial ? qk * 8 + s.b * 2 + s.v : 16 * qk + s.rho;
}

// K1: Rt_K[i][c]
__host__ __device__ inline Q4Slot q4_rt_k(const Q4Dims& q, int i, int c) {
  const RankSlot s = rank_slot(q.pd, i);
  const int ks = c / 32, qk = (c % 32) / 8, e = c % 8;
  return Q4Slot{(int64_t)s.mt * 1024 + (q4_tile_row(s, qk) * 4 + ks) * 4, 8, q4_nibble_bit(8, e)};
}

// K2: Lt_K[j][i]
__host__ __device__ inline Q4Slot q4_lt_k(const Q4Dims& q, int j, int i) {
  const int mt = (j % 16) / 4, rho = 4 * (j / 16) + j % 4;
  const int lane = q.pd.P == kP ? 16 * (i / q.pd.A) + rho : 8 * (i / q.pd.A) + rho;  // P = 32: rho < 8
  return Q4Slot{q.k2 + ((int64_t)lane * 4 + mt) * q.ub, 2 * q.ub, q4_nibble_bit(2 * q.ub, i % q.pd.A)};
}

// V1: Lt_V[j][i] (as Lt_V^T)
__host__ __device__ inline Q4Slot q4_lt_v(const Q4Dims& q, int j, int i) {
  const RankSlot s = rank_slot(q.pd, i);
  const int qk = j / 16, ks = (j % 16) / 8, e = j % 8;
  const int64_t tile = q.pd.P == kP ? 512 : 256;  // P = 32: rows of lanes 0..31
  return Q4Slot{(int64_t)s.mt * tile + (q4_tile_row(s, qk) * 2 + ks) * 4, 8, q4_nibble_bit(8, e)};
}

// V2: Rt_V[i][c] (as Rt_V^T)
__host__ __device__ inline Q4Slot q4_rt_v(const Q4Dims& q, int i, int c) {
  const int mt = c / 16, lane = 16 * (i / q.pd.A) + c % 16;
  return Q4Slot{q.v2 + ((int64_t)lane * 8 + mt) * q.ub, 2 * q.ub, q4_nibble_bit(2 * q.ub, i % q.pd.A)};
}

// Byte offsets of the scales.
__host__ __device__ inline int64_t q4_sr_k(const Q4Dims& q, int c) { return q.sr_k + 2LL * c; }
__host__ __device__ inline int64_t q4_sl_k(const Q4Dims& q, int i) { return q.sl_k + 2LL * i; }
__host__ __device__ inline int64_t q4_sl_v(const Q4Dims& q, int j) { return q.sl_v + 2LL * j; }
__host__ __device__ inline int64_t q4_sr_v(const Q4Dims& q, int c) {
  return q.sr_v + 2LL * (((c % 16) / 4) * 32 + (c / 16) * 4 + c % 4);
}

// Dense pages of an INT4-factor cache are bf16.
__host__ __device__ inline int dense_dtype(int dtype) { return dtype == PKV_F32 ? PKV_F32 : PKV_BF16; }

// Page-table entry encoding.
__host__ __device__ inline int32_t table_entry(int cls, int slot) { return (cls << 24) | slot; }
__host__ __device__ inline int table_class(int32_t e) { return (e >> 24) & 0xff; }
__host__ __device__ inline int table_slot(int32_t e) { return e & 0xffffff; }

// --------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files; return hipError_t of launch).
// --------------------------------------------------------------------------

// Where the pages to decompose come from and where their factors go.
// One source of a job's pages.  Its page f (0 <= f < its count) is read
// from input slot in_f0 + f -- taken modulo f_mod when f_mod > 0, for the
// recent-window ring -- at base[kind] + bh * bh_stride + slot * f_stride
// elements, and (cache jobs) its factors go to factor slot out_f0 + f.
struct CompressSrc {
  const void* base[2];          // per kind
  int trans[2];                 // 0: page is [P][d]; 1: page stored as [d][P]
  int64_t bh_stride;            // elements
  int64_t f_stride;             // elements
  int64_t in_f0, f_mod, out_f0;
};

struct CompressJob {
  // page n -> kind = n % n_kind, f = (n / n_kind) % n_f, bh = n / (n_kind * n_f);
  // f < n_f_src0 is page f of src[0], the others page f - n_f_src0 of src[1]
  int64_t n_pages;
  int n_kind;                   // 1 (standalone) or 2 (K and V of a cache)
  int page_rows;                // P: 64, or 32 (decomposed as 64 rows, the rest zero)
  int64_t n_f;
  int64_t n_f_src0;
  CompressSrc src[2];
  int in_dtype;                 // pkv_dtype
  int rank[2];                  // per kind
  int out_dtype;
  int key_part_kind;            // layout of kind-0 parts: PKV_KEYS or PKV_KEYS_PRE_ROPE
  // packed output (cache): fac + (bh * fac_bh_pages + slot) * page_bytes + kind * k_part_bytes
  uint8_t* fac;
  int64_t fac_bh_pages;
  int64_t page_bytes;
  int64_t k_part_bytes;
  // row-major output (standalone) when fac == nullptr
  void* lf;
  void* rf;
  float* sigma;
};

// Pages of several caches of one shape in one launch (the promotions of a
// batched decode step).  Page n belongs to member n / base.n_pages and is
// page n % base.n_pages of `base` (one source, src[0]) with the member's
// window ring (src_k, src_v), input and factor slots and factor pool (whose
// per-(sequence, KV head) stride is the member's own F_max); the first page
// of a member also writes its page-table entry.
struct CompressMember {
  const void* src_k;
  const void* src_v;
  uint8_t* fac;
  int64_t fac_bh_pages;  // the member's F_max (its own capacity)
  int64_t in_f0, out_f0;
  int32_t* table;
  int64_t table_page;
  int32_t table_entry;
};

struct CompressBatch {
  CompressJob base;
  int n;
  CompressMember m[kMaxBatchCaches];
};

// Events the caller asked to bracket the next decode-partial or page
// decomposition kernel with (pkv_time_next_kernel).  Taking them clears the
// request; both are null when none is pending.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
KernelEvents take_kernel_events();

hipError_t launch_compress(const CompressJob& job, hipStream_t stream);
// Tridiagonal-route decomposition for ranks up to kTriMaxRank (launch_compress
// dispatches to it).
constexpr int kTriMaxRank = 32;
hipError_t launch_compress_tri(const CompressJob& job, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop);
// One launch over a batch of cache jobs; ranks up to kTriMaxRank only
// (hipErrorNotSupported above).
hipError_t launch_compress_batch(const CompressBatch& jb, hipStream_t stream);

struct CacheGeom {
  int B, Hkv, Hq, G;
  int P;                        // page length: 64 or 32
  int n_s, n_w;
  int64_t F_max, max_pages;
  int dtype;
  int r_k, r_v;
  uint8_t* base;
  pkv_layout lay;
  int rope;                     // keys are pre-RoPE (pkv_cache_set_key_rope)
  float rope_freq[kD / 2];
};

hipError_t launch_prefill_dense(const CacheGeom& g, const void* K, const void* V, int64_t T,
                                int64_t n_fact, hipStream_t stream);
hipError_t launch_chunk_dense(const CacheGeom& g, const void* K, const void* V, int64_t T0, int64_t T1,
                              int64_t p_lo, int64_t p_hi, hipStream_t stream);
hipError_t launch_table_fill(const CacheGeom& g, int64_t T, int64_t n_fact, hipStream_t stream);
hipError_t launch_table_set(const CacheGeom& g, int64_t page, int32_t entry, hipStream_t stream);
hipError_t launch_append(const CacheGeom& g, const void* k, const void* v, int64_t T,
                         hipStream_t stream);

struct AttnJob {
  const void* q;
  float* out;
  float* ws_o;   // [B*Hq][n_split][d]
  float* ws_ml;  // [B*Hq][n_split][2]
  int n_split;
  int64_t T, n_fact;
  // Optional append folded into the merge (launch_merge): the new token
  // (k_new / v_new [B][H_kv][d]) joins the Eq. 5 merge as one more state
  // beside the splits (which cover tokens 0 .. T - 1), and is written to
  // row app_row of page app_page (table entry app_entry after the append).
  // k_new == nullptr: no append.
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int64_t app_page = -1;
  int app_row = -1;
  int32_t app_entry = 0;
};

hipError_t launch_partial(const CacheGeom& g, const AttnJob& job, hipStream_t stream);
// One launch over n <= kMaxBatchCaches caches of batch 1 and equal shape
// (gs[i], lengths T[i], factor counts n_fact[i]); cache i's range is shared
// by ns[i] <= job.n_split splits, its workspace rows job.n_split apart.
// hipErrorNotSupported for formats without a batched kernel.
hipError_t launch_partial_batch(const CacheGeom* gs, const int64_t* T, const int64_t* n_fact, const int* ns,
                                int n, const AttnJob& job, hipStream_t stream);

hipError_t launch_merge(const CacheGeom& g, const AttnJob& job, hipStream_t stream);
// The merge of a batch of n caches of batch 1 (rows of cache i after those of
// cache i - 1, each with ns[i] states, job.n_split apart); with job.k_new set
// ([n][H_kv][d]), cache i's token goes to the page, row and entry of apps[i]
// in cache gs[i].
hipError_t launch_merge_batch(const CacheGeom* gs, int n, const AttnJob& job, const AttnJob* apps, const int* ns,
                              hipStream_t stream);
// Whether a batch of caches of this shape has a batched partial kernel.
bool batched_kernel(const CacheGeom& g);
// Splits per cache of a batched launch with caller-chosen count 0 (ns[i]),
// in proportion to the caches' pages; returns the largest.
int decode_batch_splits(const CacheGeom& g, const int64_t* T, int n, int* ns);
int decode_default_splits(const CacheGeom& g, int64_t T, int64_t n_fact);

// Size of the library-held decode workspace of pkv_decode_attn_noalloc
// (one copy per device, held until the process ends).
constexpr uint64_t kNoAllocScratchBytes = PKV_NOALLOC_WORKSPACE_BYTES;
// That workspace's device address on the current device (looked up once per
// device by hipGetSymbolAddress).
hipError_t noalloc_scratch(void** ptr);

}  // namespace pkv
