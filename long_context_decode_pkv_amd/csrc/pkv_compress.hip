// Batched page decomposition on gfx950.
//
// PuzzleKV (Sec. 3.3, text after Eq. 3) obtains each page's factors from the
// page's P x P Gram matrix G = X X^T: its top-r eigenvectors Q are the leading
// left singular vectors, L = Q and R = Q^T X.  This kernel follows that route
// with one 64-lane wavefront per page:
//
//   1. G = X X^T on the matrix cores (bf16 inputs: v_mfma_f32_16x16x32_bf16,
//      whose bf16 products are exact and accumulate in fp32; fp32 inputs:
//      v_mfma_f32_16x16x4_f32).  Only the 10 upper tiles are formed, the
//      lower ones are mirrored.
//   2. Eigen-decomposition of G in fp32 by cyclic two-sided Jacobi rotations
//      in LDS.  Each round rotates 32 disjoint index pairs at once (the
//      circle-method round-robin order, so a sweep of 63 rounds meets every
//      pair once).  A rotation is skipped when the off-diagonal is below
//      2^-23 sqrt(|G_pp G_qq|) (relative to the pair's own diagonal, so the
//      near-degenerate small eigenvalues at the rank cut are still resolved)
//      or below 2^-30 trace(G) (a floor for exactly null directions); sweeps
//      stop when a whole sweep rotates nothing.
//   3. The r largest eigenvalues pick Q_r; R = Q_r^T X on the matrix cores in
//      fp32; sigma_i = ||R_i|| (from R, which is more accurate than sqrt of
//      the eigenvalue for small sigma).
//   4. Lf = Q_r diag(sigma), Rf = diag(1/sigma) R (zero when sigma = 0),
//      rounded nearest-even to the output dtype, stored row-major or into a
//      cache's packed factor part.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kLd = 65;  // LDS row stride in floats: row/column walks hit distinct banks
constexpr int kMaxSweeps = 24;

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element (j, c) of a page, j < P (token), c < d (channel).
template <typename Elem>
__device__ inline float page_elem(const Elem* X, int trans, int j, int c) {
  Elem v = trans ? X[c * kP + j] : X[j * kD + c];
  if constexpr (sizeof(Elem) == 2) return bf16_bits_to_f32(v);
  else return v;
}

__device__ inline float lane_value(float x, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
}

__device__ inline void store_elem(void* base, int64_t idx, int dtype, float v) {
  if (dtype == PKV_BF16) ((uint16_t*)base)[idx] = f32_to_bf16_bits(v);
  else ((float*)base)[idx] = v;
}

// G tile (16ta.., 16tb..) into LDS (and its mirror).
__device__ inline void store_gram_tile(float* Gs, int ta, int tb, floatx4 acc, int lane) {
  const int j = lane & 15, q = lane >> 4;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 16 * ta + 4 * q + v, col = 16 * tb + j;
    Gs[row * kLd + col] = acc[v];
    Gs[col * kLd + row] = acc[v];
  }
}

template <typename Elem>
__device__ void gram(const Elem* X, int trans, float* Gs, int lane) {
  const int i = lane & 15, q = lane >> 4;
  if constexpr (sizeof(Elem) == 2) {
    for (int ta = 0; ta < 4; ++ta) {
      bf16x8 a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int row = 16 * ta + i, c0 = 32 * ks + 8 * q;
        if (!trans) {
          uint4 raw = *(const uint4*)(X + row * kD + c0);
          a[ks] = __builtin_bit_cast(bf16x8, raw);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[ks][e] = __builtin_bit_cast(__bf16, X[(c0 + e) * kP + row]);
        }
      }
      for (int tb = ta; tb < 4; ++tb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 bop;
          const int row = 16 * tb + i, c0 = 32 * ks + 8 * q;
          if (tb == ta) {
            bop = a[ks];
          } else if (!trans) {
            uint4 raw = *(const uint4*)(X + row * kD + c0);
            bop = __builtin_bit_cast(bf16x8, raw);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bop[e] = __builtin_bit_cast(__bf16, X[(c0 + e) * kP + row]);
          }
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bop, acc, 0, 0, 0);
        }
        store_gram_tile(Gs, ta, tb, acc, lane);
      }
    }
  } else {
    for (int ta = 0; ta < 4; ++ta) {
      for (int tb = ta; tb < 4; ++tb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kc = 0; kc < kD / 4; ++kc) {
          const float av = page_elem(X, trans, 16 * ta + i, 4 * kc + q);
          const float bv = page_elem(X, trans, 16 * tb + i, 4 * kc + q);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
        }
        store_gram_tile(Gs, ta, tb, acc, lane);
      }
    }
  }
}

// Round-robin (circle method) pair k of round t over 64 indices.
__device__ inline void rr_pair(int t, int k, int& p, int& qq) {
  if (k == 0) {
    p = t;
    qq = 63;
  } else {
    p = (t + k) % 63;
    qq = (t - k + 63) % 63;
  }
}

__device__ void jacobi(float* Gs, float* Vs, int lane) {
  // trace -> absolute floor for off-diagonal entries
  float tr = Gs[lane * kLd + lane];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tr += __shfl_xor(tr, o);
  const float tol_abs = tr * 0x1p-30f;
  const float tol_rel = 0x1p-23f;

  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    int rotated_any = 0;
    for (int t = 0; t < 63; ++t) {
      // phase A: lane k < 32 owns pair k
      float c = 1.f, s = 0.f;
      int p = 0, qq = 0;
      bool rot = false;
      if (lane < 32) {
        rr_pair(t, lane, p, qq);
        const float app = Gs[p * kLd + p], aqq = Gs[qq * kLd + qq], apq = Gs[p * kLd + qq];
        const float thr = fmaxf(tol_rel * sqrtf(fabsf(app * aqq)), tol_abs);
        if (fabsf(apq) > thr) {
          const float tau = (aqq - app) / (2.f * apq);
          const float tt = copysignf(1.f, tau) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + tt * tt);
          s = tt * c;
          rot = true;
        }
      }
      const unsigned long long mask = __ballot(rot);
      if (mask == 0ull) continue;  // uniform: nothing to rotate this round
      rotated_any = 1;
      __syncthreads();
      // phase B: G <- G J and V <- V J (columns p, q); lane = row
#pragma unroll 4
      for (int k = 0; k < 32; ++k) {
        const float ck = lane_value(c, k), sk = lane_value(s, k);
        int pk, qk;
        rr_pair(t, k, pk, qk);
        const float gp = Gs[lane * kLd + pk], gq = Gs[lane * kLd + qk];
        Gs[lane * kLd + pk] = ck * gp - sk * gq;
        Gs[lane * kLd + qk] = sk * gp + ck * gq;
        const float vp = Vs[lane * kLd + pk], vq = Vs[lane * kLd + qk];
        Vs[lane * kLd + pk] = ck * vp - sk * vq;
        Vs[lane * kLd + qk] = sk * vp + ck * vq;
      }
      __syncthreads();
      // phase C: G <- J^T G (rows p, q); lane = column
#pragma unroll 4
      for (int k = 0; k < 32; ++k) {
        const float ck = lane_value(c, k), sk = lane_value(s, k);
        int pk, qk;
        rr_pair(t, k, pk, qk);
        const float gp = Gs[pk * kLd + lane], gq = Gs[qk * kLd + lane];
        Gs[pk * kLd + lane] = ck * gp - sk * gq;
        Gs[qk * kLd + lane] = sk * gp + ck * gq;
      }
      __syncthreads();
      if (rot) {  // the rotation annihilates the pair's off-diagonal exactly
        Gs[p * kLd + qq] = 0.f;
        Gs[qq * kLd + p] = 0.f;
      }
      __syncthreads();
    }
    if (!rotated_any) break;
  }
}

template <typename Elem>
__device__ void compress_one(const CompressJob& job, int64_t n, float* Gs, float* Vs, int* sel,
                             float* sig, int lane) {
  const int kind = (int)(n % job.n_kind);
  const int64_t f = (n / job.n_kind) % job.n_f;
  const int64_t bh = n / ((int64_t)job.n_kind * job.n_f);
  const Elem* X = (const Elem*)job.in_base[kind] + bh * job.in_bh_stride + f * job.in_f_stride;
  const int trans = job.in_trans[kind];
  const int r = job.rank[kind];

  // 1. Gram matrix, eigenvector accumulator = I
  gram<Elem>(X, trans, Gs, lane);
  for (int j = 0; j < kP; ++j) Vs[j * kLd + lane] = (j == lane) ? 1.f : 0.f;
  __syncthreads();

  // 2. Jacobi eigen-solve
  jacobi(Gs, Vs, lane);
  __syncthreads();

  // 3. top-r selection: rank of lane's eigenvalue (descending, ties by index)
  {
    const float lam = Gs[lane * kLd + lane];
    int rank = 0;
    for (int y = 0; y < kP; ++y) {
      const float ly = Gs[y * kLd + y];
      rank += (ly > lam || (ly == lam && y < lane)) ? 1 : 0;
    }
    sel[rank] = lane;
  }
  __syncthreads();

  // R = Q_r^T X in fp32 on the matrix cores, 16 ranks x 16 channels per tile.
  const int ci = lane & 15, q = lane >> 4;
  const int RT16 = (r + 15) / 16;
  floatx4 R[4][8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) R[mi][mc] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (mi >= RT16) break;
    const int irow = 16 * mi + ci;
    const int col = irow < r ? sel[irow] : -1;
    for (int kc = 0; kc < kP / 4; ++kc) {
      const int j = 4 * kc + q;
      const float av = col >= 0 ? Vs[j * kLd + col] : 0.f;
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) {
        const float bv = page_elem(X, trans, j, 16 * mc + ci);
        R[mi][mc] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, R[mi][mc], 0, 0, 0);
      }
    }
  }
  // sigma_i = ||R_i||: lane (ci, q) holds rows 16 mi + 4 q + v, columns 16 mc + ci
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (mi >= RT16) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float ss = 0.f;
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) ss += R[mi][mc][v] * R[mi][mc][v];
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
      const int i = 16 * mi + 4 * q + v;
      if (ci == 0 && i < kP) sig[i] = sqrtf(ss);
    }
  }
  __syncthreads();

  // 4. store Rf = R / sigma and Lf = Q diag(sigma)
  const bool packed = job.fac != nullptr;
  PackDims pd = pack_dims(r);
  const int r_store = packed ? 8 * pd.n8 : r;
  uint8_t* part = nullptr;
  if (packed)
    part = job.fac + ((bh * job.fac_bh_pages) + job.f0 + f) * job.page_bytes +
           (int64_t)kind * job.k_part_bytes;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (16 * mi >= r_store) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = 16 * mi + 4 * q + v;
      if (i >= r_store) continue;
      const float sg = i < r ? sig[i] : 0.f;
      const float inv = sg > 0.f ? 1.f / sg : 0.f;
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) {
        const int c = 16 * mc + ci;
        const float val = (i < r) ? R[mi][mc][v] * inv : 0.f;
        int64_t idx;
        if (!packed) idx = n * (int64_t)r * kD + (int64_t)i * kD + c;
        else idx = (kind == 0) ? off_rf_k(pd, i, c) : off_rf_v(pd, i, c);
        store_elem(packed ? (void*)part : job.rf, idx, job.out_dtype, val);
      }
    }
  }
  for (int i = 0; i < r_store; ++i) {
    const int j = lane;  // page row
    float val = 0.f;
    if (i < r) {
      const float sg = sig[i];
      val = sg > 0.f ? Vs[j * kLd + sel[i]] * sg : 0.f;
    }
    int64_t idx;
    if (!packed) idx = n * (int64_t)kP * r + (int64_t)j * r + i;
    else idx = (kind == 0) ? off_lf_k(pd, j, i) : off_lf_v(pd, j, i);
    store_elem(packed ? (void*)part : job.lf, idx, job.out_dtype, val);
  }
  if (!packed && job.sigma != nullptr && lane < r) job.sigma[n * r + lane] = sig[lane];
  __syncthreads();
}

template <typename Elem>
__global__ __launch_bounds__(64) void compress_kernel(CompressJob job) {
  __shared__ float Gs[kP * kLd];
  __shared__ float Vs[kP * kLd];
  __shared__ int sel[kP];
  __shared__ float sig[kP];
  const int lane = threadIdx.x;
  for (int64_t n = blockIdx.x; n < job.n_pages; n += gridDim.x)
    compress_one<Elem>(job, n, Gs, Vs, sel, sig, lane);
}

}  // namespace

hipError_t launch_compress(const CompressJob& job, hipStream_t stream) {
  if (job.n_pages <= 0) return hipSuccess;
  const int64_t cap = 1 << 30;
  const unsigned grid = (unsigned)(job.n_pages < cap ? job.n_pages : cap);
  if (job.in_dtype == PKV_BF16)
    hipLaunchKernelGGL(compress_kernel<uint16_t>, dim3(grid), dim3(64), 0, stream, job);
  else
    hipLaunchKernelGGL(compress_kernel<float>, dim3(grid), dim3(64), 0, stream, job);
  return hipGetLastError();
}

}  // namespace pkv
