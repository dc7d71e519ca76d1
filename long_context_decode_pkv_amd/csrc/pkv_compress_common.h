// Device helpers shared by the two page-decomposition kernels
// (pkv_compress.hip: Jacobi, any rank; pkv_compress_tri.hip: tridiagonal
// route, ranks up to 32).
#pragma once

#include "pkv_internal.h"

namespace pkv {
namespace cmp {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kLd = 65;  // LDS row stride in floats: row/column walks hit distinct banks

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element (j, c) of a page of P rows, j < P (token), c < d (channel).
// A page of P = 32 rows sits in the kernels' 64-row frame with zero rows
// below it (its Gram matrix has a zero block; the eigen-solve then runs on
// the leading 32 x 32 block).  P is a multiple of 16, so a 16-row tile or a
// 4-row reduction step lies wholly inside the page or wholly in the zero
// rows, and the callers skip those as a whole instead of reading them.
template <typename Elem>
__device__ inline float page_elem(const Elem* X, int trans, int P, int j, int c) {
  Elem v = trans ? X[c * P + j] : X[j * kD + c];
  if constexpr (sizeof(Elem) == 2) return bf16_bits_to_f32(v);
  else return v;
}

__device__ inline void store_elem(void* base, int64_t idx, int dtype, float v) {
  if (dtype == PKV_BF16) ((uint16_t*)base)[idx] = f32_to_bf16_bits(v);
  else ((float*)base)[idx] = v;
}

// 8 consecutive channels c0.. of page row `row` < P as a bf16 MFMA operand.
__device__ inline bf16x8 row8(const uint16_t* X, int trans, int P, int row, int c0) {
  if (!trans) return __builtin_bit_cast(bf16x8, *(const uint4*)(X + row * kD + c0));
  // the column stride as a constant keeps the 8 loads on one address
  bf16x8 v;
  if (P == kP) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(__bf16, X[(c0 + e) * kP + row]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(__bf16, X[(c0 + e) * kMinP + row]);
  }
  return v;
}

// One 16x16 tile (rows 16 ta.., columns 16 tb..) of G = X X^T on the matrix
// cores: lane l holds G[16 ta + 4 (l / 16) + v][16 tb + l % 16], v < 4.
// Tiles in the padding rows of a short page are zero.
template <typename Elem>
__device__ inline floatx4 gram_tile(const Elem* X, int trans, int P, int ta, int tb, int lane) {
  const int i = lane & 15, q = lane >> 4;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  if (16 * ta >= P || 16 * tb >= P) return acc;  // uniform
  if constexpr (sizeof(Elem) == 2) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 av = row8(X, trans, P, 16 * ta + i, 32 * ks + 8 * q);
      const bf16x8 bv = row8(X, trans, P, 16 * tb + i, 32 * ks + 8 * q);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
  } else {
#pragma unroll 4
    for (int kc = 0; kc < kD / 4; ++kc) {
      if ((kc & 3) == 0) __builtin_amdgcn_sched_barrier(0);
      const float av = page_elem(X, trans, P, 16 * ta + i, 4 * kc + q);
      const float bv = page_elem(X, trans, P, 16 * tb + i, 4 * kc + q);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
    }
  }
  return acc;
}

// Where page n of a job comes from and goes to.
struct PageRef {
  int kind;
  int64_t bh;
  int64_t slot;  // factor slot (cache jobs)
  int trans, r;
  int P;         // page rows
  const void* X;
  uint8_t* part; // its packed factor part (cache jobs), else nullptr
};

__device__ inline PageRef page_ref(const CompressJob& job, int64_t n, int elem_bytes) {
  PageRef p;
  p.kind = (int)(n % job.n_kind);
  const int64_t fj = (n / job.n_kind) % job.n_f;
  p.bh = n / ((int64_t)job.n_kind * job.n_f);
  const bool second = fj >= job.n_f_src0;
  const CompressSrc& src = second ? job.src[1] : job.src[0];
  const int64_t f = second ? fj - job.n_f_src0 : fj;
  int64_t in = src.in_f0 + f;
  if (src.f_mod > 0) in %= src.f_mod;
  p.slot = src.out_f0 + f;
  p.trans = src.trans[p.kind];
  p.r = job.rank[p.kind];
  p.P = job.page_rows;
  p.X = (const uint8_t*)src.base[p.kind] + (p.bh * src.bh_stride + in * src.f_stride) * elem_bytes;
  p.part = job.fac ? job.fac + (p.bh * job.fac_bh_pages + p.slot) * job.page_bytes +
                         (int64_t)p.kind * job.k_part_bytes
                   : nullptr;
  return p;
}

// Page n of a batch of cache jobs: member n / per (per = jb.base.n_pages),
// page n % per of its job -- jb.base with the member's pools.
__device__ inline PageRef page_ref(const CompressBatch& jb, int64_t n, int elem_bytes) {
  const CompressJob& job = jb.base;
  const int64_t per = job.n_pages;
  const CompressMember& m = jb.m[n / per];
  const int64_t local = n % per;
  PageRef p;
  p.kind = (int)(local % job.n_kind);
  const int64_t f = (local / job.n_kind) % job.n_f;
  p.bh = local / ((int64_t)job.n_kind * job.n_f);
  const CompressSrc& src = job.src[0];
  int64_t in = m.in_f0 + f;
  if (src.f_mod > 0) in %= src.f_mod;
  p.slot = m.out_f0 + f;
  p.trans = src.trans[p.kind];
  p.r = job.rank[p.kind];
  p.P = job.page_rows;
  p.X = (const uint8_t*)(p.kind ? m.src_v : m.src_k) + (p.bh * src.bh_stride + in * src.f_stride) * elem_bytes;
  p.part = m.fac + (p.bh * m.fac_bh_pages + p.slot) * job.page_bytes + (int64_t)p.kind * job.k_part_bytes;
  return p;
}

// Packed factor part of a cache job's page.
__device__ inline uint8_t* factor_part(const CompressJob&, const PageRef& p) { return p.part; }

// Destination of factor element Rf[i][c] (i < rf_store) and Lf[j][i]
// (i < r_store): a packed part stores Lf at r8 ranks, zero-padded, and Rf at
// r8 (key parts) or at its even-rounded rank r2 (value parts).
struct FactorDst {
  bool packed;
  PackDims pd;
  int r, r_store, rf_store, kind;
  int P;
  int64_t n;
  void* rf;
  void* lf;
  __device__ FactorDst(const CompressJob& job, const PageRef& p, int64_t n_) {
    packed = p.part != nullptr;
    pd = pack_dims(p.r, p.P);
    r = p.r;
    P = p.P;
    r_store = packed ? 8 * pd.n8 : p.r;
    kind = p.kind == 0 ? job.key_part_kind : PKV_VALUES;  // part layout
    rf_store = packed && kind == PKV_VALUES ? pd.r2 : r_store;
    n = n_;
    if (packed) {
      rf = lf = factor_part(job, p);
    } else {
      rf = job.rf;
      lf = job.lf;
    }
  }
  __device__ __forceinline__ int64_t rf_idx(int i, int c) const {
    if (!packed) return n * (int64_t)r * kD + (int64_t)i * kD + c;
    return off_rf(kind, pd, i, c);
  }
  __device__ __forceinline__ int64_t lf_idx(int j, int i) const {
    if (!packed) return n * (int64_t)P * r + (int64_t)j * r + i;
    return off_lf(kind, pd, j, i);
  }
};

}  // namespace cmp
}  // namespace pkv
