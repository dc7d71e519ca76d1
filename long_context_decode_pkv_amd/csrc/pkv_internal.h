// Internal declarations shared by the HIP sources of libpkv (not part of the
// C-ABI).  Host and device code both include this header.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kP = 64;    // page length supported by the kernels
constexpr int kD = 128;   // head dim supported by the kernels
constexpr int kMaxG = 8;  // query heads per KV head handled by one wave
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
  int n8;   // ceil(r / 8)
  int A;    // ranks per lane quad = 2 * n8
  int RT;   // rank tiles = ceil(A / 4)
  int KS2;  // 32-wide reduction steps over the rank = ceil(A / 8)
  int64_t k1, k2, v1, v2;  // element counts of the four operands
};

__host__ __device__ inline PackDims pack_dims(int r) {
  PackDims p;
  p.n8 = (r + 7) / 8;
  p.A = 2 * p.n8;
  p.RT = (p.A + 3) / 4;
  p.KS2 = (p.A + 7) / 8;
  p.k1 = (int64_t)8 * p.n8 * kD;
  p.k2 = (int64_t)kP * 8 * p.n8;
  p.v1 = (int64_t)8 * p.n8 * kP;
  p.v2 = (int64_t)kD * 8 * p.n8;
  return p;
}

__host__ __device__ inline int64_t part_elems(int r) {
  PackDims p = pack_dims(r);
  return p.k1 + p.k2;  // == p.v1 + p.v2 == r8 (P + d)
}

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
  int lane = 16 * qk + rho;
  return p.k1 + (int64_t)mt * 64 * p.A + 512 * ks + lane * w + e;
}

// V1: Lf_V[j][i] (stored as Lf_V^T)
__host__ __device__ inline int64_t off_lf_v(const PackDims& p, int j, int i) {
  RankSlot s = rank_slot(p, i);
  int qk = j / 16, ks = (j % 16) / 8, e = j % 8;
  int64_t base = (int64_t)s.mt * 1024;
  if (!s.partial) return base + ks * 512 + (16 * qk + s.rho) * 8 + e;
  int lam = qk * 8 + s.b * 2 + s.v;
  return base + ks * 256 + lam * 8 + e;
}

// V2: Rf_V[i][c] (stored as Rf_V^T)
__host__ __device__ inline int64_t off_rf_v(const PackDims& p, int i, int c) {
  int mt = c / 16, rho = c % 16;
  int qk = i / p.A, a = i % p.A, ks = a / 8, e = a % 8;
  int w = (p.A - 8 * ks) < 8 ? (p.A - 8 * ks) : 8;
  int lane = 16 * qk + rho;
  return p.v1 + (int64_t)mt * 64 * p.A + 512 * ks + lane * w + e;
}

// Page-table entry encoding.
__host__ __device__ inline int32_t table_entry(int cls, int slot) { return (cls << 24) | slot; }
__host__ __device__ inline int table_class(int32_t e) { return (e >> 24) & 0xff; }
__host__ __device__ inline int table_slot(int32_t e) { return e & 0xffffff; }

// --------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files; return hipError_t of launch).
// --------------------------------------------------------------------------

// Where the pages to decompose come from and where their factors go.
struct CompressJob {
  // page n -> kind = n % n_kind, f = (n / n_kind) % n_f, bh = n / (n_kind * n_f)
  int64_t n_pages;
  int n_kind;                   // 1 (standalone) or 2 (K and V of a cache)
  int64_t n_f;
  const void* in_base[2];       // per kind
  int in_trans[2];              // 0: page is [P][d]; 1: page stored as [d][P]
  int64_t in_bh_stride;         // elements
  int64_t in_f_stride;          // elements
  int in_dtype;                 // pkv_dtype
  int rank[2];                  // per kind
  int out_dtype;
  // packed output (cache): fac + ((bh * fac_bh_pages) + f0 + f) * page_bytes + kind * k_part_bytes
  uint8_t* fac;
  int64_t fac_bh_pages;
  int64_t f0;
  int64_t page_bytes;
  int64_t k_part_bytes;
  // row-major output (standalone) when fac == nullptr
  void* lf;
  void* rf;
  float* sigma;
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

struct CacheGeom {
  int B, Hkv, Hq, G;
  int n_s, n_w;
  int64_t F_max, max_pages;
  int dtype;
  int r_k, r_v;
  uint8_t* base;
  pkv_layout lay;
};

hipError_t launch_prefill_dense(const CacheGeom& g, const void* K, const void* V, int64_t T,
                                int64_t n_fact, hipStream_t stream);
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
hipError_t launch_merge(const CacheGeom& g, const AttnJob& job, hipStream_t stream);
int decode_default_splits(const CacheGeom& g, int64_t T, int64_t n_fact);

}  // namespace pkv
