// Batched page decomposition on gfx950, tridiagonal route (ranks r <= 32).
//
// PuzzleKV (Sec. 3.3, text after Eq. 3) takes each page's factors from the
// page's P x P Gram matrix G = X X^T: its top-r eigenvectors Q are the leading
// left singular vectors, and R = Q^T X.  The page leaves the eigen-method
// open.  This kernel uses the classical symmetric route: Householder
// reduction to tridiagonal form, bisection on Sturm sequence counts for the
// r largest eigenvalues, one eigenvector per eigenvalue from a twisted
// factorization, back-transformation.  That is ~0.5 MFLOP of eigen-work per
// page against ~20 MFLOP for Jacobi sweeps, and it has no data-dependent
// iteration count.
//
// One 64-lane wavefront (one workgroup) per page.  Lane i owns row i of G and
// row i of the accumulated Householder product Q_H in registers.
//
//   1. G = X X^T on the matrix cores (bf16 inputs: v_mfma_f32_16x16x32_bf16,
//      exact products, fp32 accumulation; fp32 inputs: v_mfma_f32_16x16x4_f32),
//      staged through LDS one 16-row band at a time into the row registers.
//   2. 62 Householder steps G <- H G H (H = I - tau v v^T, the LAPACK slarfg
//      convention: v_{k+1} = 1, beta = -sign(alpha) ||x||), each a matrix-vector
//      product and a rank-2 update on the lane's row; Q_H <- Q_H H on the
//      lane's row of Q_H.  The reflector and the update vector are broadcast
//      through LDS.  Result: T = diag(a) + offdiag(b), G = Q_H T Q_H^T.
//   3. The r largest eigenvalues of T by multisection: 64 / r' lanes per
//      eigenvalue (r' = r rounded up to a power of two) each count the
//      eigenvalues below their own point (Sturm count = number of negative
//      pivots of the LDL^T factorization of T - x I), a fixed number of rounds
//      to 2^-25 of the Gershgorin span.
//   4. For each eigenvalue lambda the eigenvector of T from the twisted
//      factorization of T - lambda I: forward pivots d+_i, backward pivots
//      d-_i, twist index k = argmin |d+_k + d-_k - (a_k - lambda)|, z_k = 1 and
//      the two one-sided recurrences outward from k.
//   5'. Q_r = Q_H Z is orthonormalized: the twisted vectors of close
//      eigenvalues are orthogonal only to about eps ||T|| / gap, so one
//      Cholesky QR pass (W = Q_r^T Q_r on the matrix cores, its Cholesky
//      factor in LDS, a forward solve per row) restores orthonormality.
//      Eigenvalues the bisection cannot tell apart (an exactly repeated
//      singular value, a null space) give one vector several times; then the
//      dead columns are refilled with fixed pseudo-random vectors and Q_r is
//      refined by 8 steps of orthogonal iteration Q <- orth(X (X^T Q)).
//   5. R = Q_r^T X on the matrix cores in fp32, sigma_i = ||R_i||,
//      Lf = Q_r diag(sigma), Rf = diag(1/sigma) R (zero where sigma = 0), rounded
//      nearest-even to the output dtype.  INT4 caches (Sec. 4.3) instead
//      store Lt = Q_r diag(sigma^(1/2)) and Rt = diag(sigma^(-1/2)) R as
//      symmetric 4-bit codes with bf16 group scales (store_q4).
//
// A page of N = 32 rows sits in the 64-row frame with zero rows below it: G,
// the reflectors and Q_H are block-diagonal with an identity / zero block, T
// splits after row N - 1, and steps 2-5 run on the leading N x N block only
// (the zero block's eigenvalues are exact zeros that the search must not
// mistake for the page's smallest ones).
#include <type_traits>

#include "pkv_compress_common.h"

namespace pkv {
namespace {

using namespace cmp;

constexpr int kZs = 36;  // LDS row stride of Z and Q_r (floats; 16-byte aligned rows)

struct TriShared {
  union {
    float band[16 * kLd];  // one 16-row band of G on its way into the row registers
    float Z[kP * kZs];     // eigenvectors of T as columns, then Q_r
  } u;
  float xrow[kP];  // scratch row: bisection points, a Cholesky column, INT4 scale factors
  float v[kP];     // Householder vector
  float w[kP];     // rank-2 update vector
  float a[kP];     // diagonal of T
  float b[kP];     // b[i] = T[i][i+1], b[63] = 0
  float b2s[kP];   // b2s[i] = b[i-1]^2, b2s[0] = 0
  float sig[kTriMaxRank];
};

template <int Op>
__device__ __forceinline__ float combine(float p, float q) {
  if constexpr (Op == 0) return p + q;
  else if constexpr (Op == 1) return fmaxf(p, q);
  else return fminf(p, q);
}

template <int Ctrl>
__device__ __forceinline__ float dpp_mov(float y) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), Ctrl, 0xf, 0xf, false));
}

// Sum (Op 0) / max (1) / min (2) over the 16 lanes of each DPP row, in every
// lane of the row.
template <int Op>
__device__ __forceinline__ float row16_reduce(float x) {
  x = combine<Op>(x, dpp_mov<0xb1>(x));   // quad_perm [1,0,3,2]
  x = combine<Op>(x, dpp_mov<0x4e>(x));   // quad_perm [2,3,0,1]
  x = combine<Op>(x, dpp_mov<0x141>(x));  // row_half_mirror
  x = combine<Op>(x, dpp_mov<0x140>(x));  // row_mirror
  return x;
}

template <int Op, int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_rows(float y) {
  // lanes outside RowMask keep the identity of Op
  constexpr float id = Op == 0 ? 0.f : (Op == 1 ? -__builtin_inff() : __builtin_inff());
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(y), Ctrl, RowMask, 0xf, false));
}

// Sum / max / min over the whole wave: row reductions, then row 0 into row 1
// and row 2 into row 3 (row_bcast:15), then rows 0-1 into rows 2-3
// (row_bcast:31); lane 63 holds the result.
template <int Op>
__device__ __forceinline__ float wave_reduce(float x) {
  float s = row16_reduce<Op>(x);
  s = combine<Op>(s, dpp_rows<Op, 0x142, 0xa>(s));
  s = combine<Op>(s, dpp_rows<Op, 0x143, 0xc>(s));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 63));
}

// 1. G into the row registers: lane i gets G[i][0..63].  bf16 pages: a
// lane's operand chunks (rows 16 t + c, channels 32 ks + 8 q .. + 7) are the
// same for every tile, as A and as B operand, so the page is loaded once --
// 16 independent 16-byte loads, one memory latency -- and the 16 tiles run
// from registers.
template <typename Elem>
__device__ __forceinline__ void gram_rows(const Elem* X, int trans, int P, TriShared& sh, float (&g)[kP], int lane) {
  const int c = lane & 15, q = lane >> 4;
  if constexpr (sizeof(Elem) == 2) {
    bf16x8 op[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        op[t][ks] = 16 * t < P ? row8((const uint16_t*)X, trans, P, 16 * t + c, 32 * ks + 8 * q) : bf16x8{};
    }
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (16 * ta < P && 16 * tb < P) {  // tiles in the padding rows of a short page are zero
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[ta][ks], op[tb][ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sh.u.band[(4 * q + v) * kLd + 16 * tb + c] = acc[v];
      }
      __syncthreads();
      if (q == ta) {
#pragma unroll
        for (int j = 0; j < kP; ++j) g[j] = sh.u.band[c * kLd + j];
      }
      __syncthreads();
    }
    return;
  }
  for (int ta = 0; ta < 4; ++ta) {
    for (int tb = 0; tb < 4; ++tb) {
      __builtin_amdgcn_sched_barrier(0);
      const floatx4 acc = gram_tile(X, trans, P, ta, tb, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) sh.u.band[(4 * q + v) * kLd + 16 * tb + c] = acc[v];
    }
    __syncthreads();
    if (q == ta) {
#pragma unroll
      for (int j = 0; j < kP; ++j) g[j] = sh.u.band[c * kLd + j];
    }
    __syncthreads();
  }
}

// f(integral_constant<int, c>) for c = c0 .. NC - 1 (NC <= 16): a switch
// whose cases fall through into one unrolled chunk sequence, so register
// indices stay compile-time constants and a uniform start costs one
// dispatch, not a test per chunk.
template <int NC, class F>
__device__ __forceinline__ void from_chunk(int c0, F&& f) {
  static_assert(NC <= 16, "at most 16 chunks");
#define PKV_CHUNK(c)                                                  \
  case c:                                                             \
    if constexpr (c < NC) f(std::integral_constant<int, c>{});        \
    [[fallthrough]];
  switch (c0) {
    PKV_CHUNK(0) PKV_CHUNK(1) PKV_CHUNK(2) PKV_CHUNK(3) PKV_CHUNK(4) PKV_CHUNK(5) PKV_CHUNK(6) PKV_CHUNK(7)
    PKV_CHUNK(8) PKV_CHUNK(9) PKV_CHUNK(10) PKV_CHUNK(11) PKV_CHUNK(12) PKV_CHUNK(13) PKV_CHUNK(14)
    PKV_CHUNK(15)
    default:
      break;
  }
#undef PKV_CHUNK
}

// f(integral_constant<int, c>) for the one chunk c (NC <= 16).
template <int NC, class F>
__device__ __forceinline__ void at_chunk(int c, F&& f) {
  static_assert(NC <= 16, "at most 16 chunks");
#define PKV_CHUNK(c)                                                  \
  case c:                                                             \
    if constexpr (c < NC) f(std::integral_constant<int, c>{});        \
    break;
  switch (c) {
    PKV_CHUNK(0) PKV_CHUNK(1) PKV_CHUNK(2) PKV_CHUNK(3) PKV_CHUNK(4) PKV_CHUNK(5) PKV_CHUNK(6) PKV_CHUNK(7)
    PKV_CHUNK(8) PKV_CHUNK(9) PKV_CHUNK(10) PKV_CHUNK(11) PKV_CHUNK(12) PKV_CHUNK(13) PKV_CHUNK(14)
    PKV_CHUNK(15)
    default:
      break;
  }
#undef PKV_CHUNK
}

// 2. Householder tridiagonalization of the leading N x N block (the rest of
// G is zero).  On return lane i holds a_i (my_a), b_i (my_b) and row i of Q_H.
template <int N>
__device__ __forceinline__ void tridiagonalize(TriShared& sh, float (&g)[kP], float (&qh)[kP], int lane,
                                      float& my_a, float& my_b) {
#pragma unroll
  for (int j = 0; j < kP; ++j) qh[j] = (j == lane) ? 1.f : 0.f;
  my_a = 0.f;
  my_b = 0.f;
  for (int k = 0; k < N - 1; ++k) {
    // G stays symmetric, so G[k][lane] = G[lane][k] is the lane's own g[k]:
    // a uniform switch on the chunk of k, then a select within it
    float x = 0.f;
    at_chunk<N / 4>(k >> 2, [&](auto J) {
      constexpr int jc = decltype(J)::value;
      const int e = k & 3;
      x = e == 0 ? g[4 * jc] : (e == 1 ? g[4 * jc + 1] : (e == 2 ? g[4 * jc + 2] : g[4 * jc + 3]));
    });
    if (lane == k) my_a = x;
    const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k + 1));
    const float tail = wave_reduce<0>(lane >= k + 2 ? x * x : 0.f);
    // H_k = I - tau v v^T; tail == 0 means no reflection (tau = 0, v = e_{k+1})
    const bool refl = tail > 0.f;
    // v_sqrt_f32 / v_rcp_f32 (1 ulp): the reflector's own rounding is of that order
    const float xn = __builtin_amdgcn_sqrtf(fmaf(alpha, alpha, tail));
    const float beta = refl ? (alpha >= 0.f ? -xn : xn) : alpha;
    const float tau = refl ? (beta - alpha) * __builtin_amdgcn_rcpf(beta) : 0.f;
    const float scal = refl ? __builtin_amdgcn_rcpf(alpha - beta) : 0.f;
    const float vi = lane == k + 1 ? 1.f : (lane >= k + 2 ? x * scal : 0.f);
    sh.v[lane] = vi;
    __syncthreads();
    // p = tau G v (rows > k), t = Q_H v; v_j = 0 for j <= k, so the 4-column
    // chunks left of k + 1 are skipped: the step enters the unrolled chunk
    // sequence at its first active chunk (one uniform branch per loop)
    // (each v chunk is read one chunk ahead of its use: the LDS latency
    // overlaps the FMAs of the chunk before)
    const int jc0 = (k + 1) >> 2;
    float pacc = 0.f, tacc = 0.f;
    float4 vq = *(const float4*)&sh.v[4 * jc0];
    from_chunk<N / 4>(jc0, [&](auto J) {
      constexpr int jc = decltype(J)::value;
      __builtin_amdgcn_sched_barrier(0);
      const float4 vv = vq;
      if constexpr (jc + 1 < N / 4) vq = *(const float4*)&sh.v[4 * (jc + 1)];
      pacc = fmaf(g[4 * jc], vv.x, pacc);
      pacc = fmaf(g[4 * jc + 1], vv.y, pacc);
      pacc = fmaf(g[4 * jc + 2], vv.z, pacc);
      pacc = fmaf(g[4 * jc + 3], vv.w, pacc);
      tacc = fmaf(qh[4 * jc], vv.x, tacc);
      tacc = fmaf(qh[4 * jc + 1], vv.y, tacc);
      tacc = fmaf(qh[4 * jc + 2], vv.z, tacc);
      tacc = fmaf(qh[4 * jc + 3], vv.w, tacc);
    });
    const float pi = lane > k ? tau * pacc : 0.f;
    const float K = 0.5f * tau * wave_reduce<0>(pi * vi);
    const float wi = fmaf(-K, vi, pi);
    sh.w[lane] = wi;
    __syncthreads();
    // G <- G - v w^T - w v^T ; Q_H <- Q_H - tau (Q_H v) v^T
    const float tq = tau * tacc;
    from_chunk<N / 4>(jc0, [&](auto J) {
      constexpr int jc = decltype(J)::value;
      __builtin_amdgcn_sched_barrier(0);
      const float4 vv = *(const float4*)&sh.v[4 * jc];
      const float4 ww = *(const float4*)&sh.w[4 * jc];
      g[4 * jc] = fmaf(-vi, ww.x, fmaf(-wi, vv.x, g[4 * jc]));
      g[4 * jc + 1] = fmaf(-vi, ww.y, fmaf(-wi, vv.y, g[4 * jc + 1]));
      g[4 * jc + 2] = fmaf(-vi, ww.z, fmaf(-wi, vv.z, g[4 * jc + 2]));
      g[4 * jc + 3] = fmaf(-vi, ww.w, fmaf(-wi, vv.w, g[4 * jc + 3]));
      qh[4 * jc] = fmaf(-tq, vv.x, qh[4 * jc]);
      qh[4 * jc + 1] = fmaf(-tq, vv.y, qh[4 * jc + 1]);
      qh[4 * jc + 2] = fmaf(-tq, vv.z, qh[4 * jc + 2]);
      qh[4 * jc + 3] = fmaf(-tq, vv.w, qh[4 * jc + 3]);
    });
    if (lane == k) my_b = beta;
    __syncthreads();
  }
  // the last diagonal entry is already in place: no reflection touches it
  if (lane == N - 1) my_a = g[N - 1];
}

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Number of eigenvalues of T below x: non-positive pivots of T - x I = L D L^T.
// The couplings b2s are floored at a tiny positive value (setup), so a zero
// pivot gives rcp = inf and the next pivot -inf, never 0 * inf.
template <int N>
__device__ __forceinline__ int sturm_count(const TriShared& sh, float x) {
  int cnt = 0;
  float d = 1.f;
#pragma unroll 4
  for (int ic = 0; ic < N / 4; ++ic) {
    const float4 a4 = *(const float4*)&sh.a[4 * ic];
    const float4 b4 = *(const float4*)&sh.b2s[4 * ic];
    const float av[4] = {a4.x, a4.y, a4.z, a4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d = fmaf(-bv[e], rcp(d), av[e] - x);
      cnt += d <= 0.f ? 1 : 0;
    }
  }
  return cnt;
}

// Rounds of L-point multisection after the 65-point first round:
// 65 (L + 1)^n >= 2^25.
__device__ __forceinline__ int multisection_rounds(int L) {
  switch (L) {
    case 2: return 12;
    case 4: return 9;
    case 8: return 6;
    case 16: return 5;
    default: return 4;  // 32, 64
  }
}

// 4. Eigenvector of T for eigenvalue lam by the twisted factorization, into
// column `col` of Z (LDS, stride kZs), normalized; all zeros if it could not be
// formed.  The column doubles as the scratch for the pivots, so a lane holds
// no per-row state in registers.  Lanes sharing a column compute identical
// values; only `writer` lanes store.
template <int N>
__device__ __forceinline__ void twisted_vector(TriShared& sh, float lam, float pivmin, int col,
                                               bool writer) {
  auto guard = [pivmin](float d) { return fabsf(d) < pivmin ? -pivmin : d; };
  float* Zc = sh.u.Z + col;
  // forward pivots d+_i -> Z[i]
  float d = 1.f;
  for (int i = 0; i < N; ++i) {
    d = guard(fmaf(-sh.b2s[i], rcp(d), sh.a[i] - lam));
    if (writer) Zc[i * kZs] = d;
  }
  __syncthreads();
  // backward pivots d-_i (b2s[i + 1] = b_i^2) and the twist index
  float dm = 1.f, best = __builtin_inff();
  int kk = N - 1;
  for (int i = N - 1; i >= 0; --i) {
    const float ai = sh.a[i] - lam;
    dm = guard(fmaf(-(i < N - 1 ? sh.b2s[i + 1] : 0.f), rcp(dm), ai));
    const float gam = fabsf(Zc[i * kZs] + dm - ai);
    if (gam < best) {
      best = gam;
      kk = i;
    }
  }
  // z_kk = 1; above kk: z_i = -b_{i-1} z_{i-1} / d-_i, so the d-_i are formed
  // again top-down and kept where i > kk
  dm = 1.f;
  for (int i = N - 1; i > kk; --i) {
    dm = guard(fmaf(-(i < N - 1 ? sh.b2s[i + 1] : 0.f), rcp(dm), sh.a[i] - lam));
    if (writer) Zc[i * kZs] = dm;
  }
  __syncthreads();
  float ss = 1.f, zz = 1.f;
  for (int i = kk + 1; i < N; ++i) {
    zz = -sh.b[i - 1] * zz * rcp(Zc[i * kZs]);
    ss = fmaf(zz, zz, ss);
    if (writer) Zc[i * kZs] = zz;
  }
  // below kk: z_i = -b_i z_{i+1} / d+_i
  zz = 1.f;
  for (int i = kk - 1; i >= 0; --i) {
    zz = -sh.b[i] * zz * rcp(Zc[i * kZs]);
    ss = fmaf(zz, zz, ss);
    if (writer) Zc[i * kZs] = zz;
  }
  if (writer) Zc[kk * kZs] = 1.f;
  __syncthreads();
  const bool ok = ss > 0.f && ss < __builtin_inff();
  const float inv = ok ? rsqrtf(ss) : 0.f;
  for (int i = 0; i < N; ++i) {
    const float zi = Zc[i * kZs];
    if (writer) Zc[i * kZs] = ok ? zi * inv : 0.f;
  }
}

// 5a'. One Cholesky QR pass over the columns of Q_r (N x r, lane p holds row
// p in qr[], LDS sh.u.Z the same rows): W = Q_r^T Q_r on the matrix cores in
// fp32, W = L L^T in LDS, then each row solves y L^T = q (forward
// substitution), so the new columns are orthonormal to about eps times the
// old columns' condition number squared.  A pivot below 2^-20 of W's largest
// diagonal marks a dependent column, which becomes zero (bit j of `dead`).
// The result goes back to qr[] and to sh.u.Z.  Returns (wave-uniform)
// whether some pivot was below 1/4 of W's largest diagonal, i.e. some column
// was nearly dependent on the ones before it.
constexpr int kWs = 36;  // LDS row stride of W and L (floats; 16-byte aligned rows)

template <int N>
__device__ __forceinline__ bool orthonormalize(TriShared& sh, float (&qr)[kTriMaxRank], int r, int lane,
                                               uint32_t& dead) {
  const int c = lane & 15, q = lane >> 4;
  const int RT16 = (r + 15) / 16;
  // W tiles (ti <= tj) on the matrix cores; lane l holds W[16 ti + 4 q + v][16 tj + c]
  floatx4 Wt[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int ti = t == 2 ? 1 : 0, tj = t == 0 ? 0 : 1;
    Wt[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tj < RT16) {
#pragma unroll 4
      for (int s = 0; s < N / 4; ++s) {
        const float av = sh.u.Z[(4 * s + q) * kZs + 16 * ti + c];
        const float bv = sh.u.Z[(4 * s + q) * kZs + 16 * tj + c];
        Wt[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, Wt[t], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // Z is read; W takes its place (qr[] keeps Q_r)
  float* W = sh.u.Z;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int ti = t == 2 ? 1 : 0, tj = t == 0 ? 0 : 1;
    if (tj < RT16) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * ti + 4 * q + v, jj = 16 * tj + c;
        W[i * kWs + jj] = Wt[t][v];
        W[jj * kWs + i] = Wt[t][v];
      }
    }
  }
  __syncthreads();
  // Cholesky, right-looking, in LDS: lane (i, h) = (lane % 32, lane / 32)
  // updates row i's columns 16 h .. 16 h + 15; column k of L goes through
  // sh.xrow, and the lane whose chunk holds column k writes it into W
  const float dmax = wave_reduce<1>(lane < r ? W[lane * kWs + lane] : 0.f);
  const int i = lane & 31, h = lane >> 5;
  bool weak = false;
  dead = 0;
  for (int k = 0; k < r; ++k) {
    const float piv = W[k * kWs + k];
    const bool live = piv > 0x1p-20f * dmax;
    weak |= piv < 0.25f * dmax;
    dead |= live ? 0u : 1u << k;
    const float lkk = live ? __builtin_amdgcn_sqrtf(piv) : 0.f;
    const float inv = live ? __builtin_amdgcn_rcpf(lkk) : 0.f;
    if (h == 0) sh.xrow[i] = i < r ? (i == k ? lkk : (i > k ? W[i * kWs + k] * inv : 0.f)) : 0.f;
    __syncthreads();
    if (i >= k && i < r) {
      const float lik = sh.xrow[i];
#pragma unroll
      for (int jc = 0; jc < 4; ++jc) {
        const int j0 = 16 * h + 4 * jc;
        if (j0 + 3 >= k && j0 <= i) {
          float4 wv = *(const float4*)&W[i * kWs + j0];
          const float4 lv = *(const float4*)&sh.xrow[j0];
          float* wp = &wv.x;
          const float* lp = &lv.x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = j0 + e;
            wp[e] = j == k ? lik : (j > k && j <= i ? fmaf(-lik, lp[e], wp[e]) : wp[e]);
          }
          *(float4*)&W[i * kWs + j0] = wv;
        }
      }
    }
    __syncthreads();
  }
  // y L^T = q: y_j = (q_j - sum_{i<j} L[j][i] y_i) / L[j][j]; dead columns stay zero
#pragma unroll
  for (int j = 0; j < kTriMaxRank; ++j) {
    if (j < r) {
      float acc = qr[j];
#pragma unroll
      for (int ic = 0; ic < kTriMaxRank / 4; ++ic) {
        if (4 * ic < j) {
          const float4 l4 = *(const float4*)&W[j * kWs + 4 * ic];
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * ic + e < j) acc = fmaf(-lv[e], qr[4 * ic + e], acc);
        }
      }
      const float ljj = W[j * kWs + j];
      qr[j] = ljj > 0.f ? acc * __builtin_amdgcn_rcpf(ljj) : 0.f;
    }
  }
  __syncthreads();  // L is read; Q_r goes back to Z
#pragma unroll
  for (int jc = 0; jc < kTriMaxRank / 4; ++jc) {
    if (4 * jc < r)
      *(float4*)&sh.u.Z[lane * kZs + 4 * jc] = float4{qr[4 * jc], qr[4 * jc + 1], qr[4 * jc + 2], qr[4 * jc + 3]};
  }
  __syncthreads();
  return __ballot(weak) != 0;
}

// Y = X (X^T Q) = G Q for the columns of Q in sh.u.Z (N rows, r columns), on
// the matrix cores in fp32 (the bf16 page enters exactly): V = X^T Q is formed
// 16 channels x 16 columns at a time in LDS (the padding columns 32..35 of
// sh.u.Z, 256 floats) and folded into Y right away, so G itself is never
// stored.  Y replaces Q in sh.u.Z and in qr[] (lane p: row p).
template <typename Elem, int N>
__device__ __forceinline__ void gram_times(TriShared& sh, const Elem* X, int trans, int P, float (&qr)[kTriMaxRank],
                                           int r, int lane) {
  const int c = lane & 15, q = lane >> 4;
  const int RT16 = (r + 15) / 16;
  // V chunk [16 channels][16 columns]: element k at Z[k / 4][32 + k % 4]
  auto buf = [&sh](int k) -> float& { return sh.u.Z[(k >> 2) * kZs + kTriMaxRank + (k & 3)]; };
  floatx4 Y[4][2];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) Y[ti][0] = Y[ti][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int mc = 0; mc < kD / 16; ++mc) {
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      if (th < RT16) {
        floatx4 V = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s = 0; s < N / 4; ++s) {  // V[c][j] = sum_p X[p][c] Q[p][j]
          const float av = page_elem(X, trans, P, 4 * s + q, 16 * mc + c);
          const float bv = sh.u.Z[(4 * s + q) * kZs + 16 * th + c];
          V = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, V, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) buf((4 * q + v) * 16 + c) = V[v];
        __syncthreads();
#pragma unroll
        for (int ti = 0; ti < N / 16; ++ti) {  // Y[p][j] += sum_{c in chunk} X[p][c] V[c][j]
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float av = page_elem(X, trans, P, 16 * ti + c, 16 * mc + 4 * s + q);
            const float bv = buf((4 * s + q) * 16 + c);
            Y[ti][th] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, Y[ti][th], 0, 0, 0);
          }
        }
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int ti = 0; ti < N / 16; ++ti) {
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      if (th < RT16) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sh.u.Z[(16 * ti + 4 * q + v) * kZs + 16 * th + c] = Y[ti][th][v];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTriMaxRank; ++j) qr[j] = j < r && lane < N ? sh.u.Z[lane * kZs + j] : 0.f;
}

// Kept eigenvalues that the bisection could not tell apart (a cluster within
// rounding: an exactly repeated singular value, or a null space) give the
// same twisted vector more than once, and the Cholesky QR pass leaves such
// columns dead or nearly dependent.  The dead columns are refilled with
// fixed pseudo-random vectors and Q_r is refined by orthogonal iteration,
// Q <- orth(G Q): a column that is already an eigenvector stays (up to
// rounding), and a refilled column converges to the largest eigen-direction
// not yet held by the columns before it -- the missing copies of the cluster
// (or, beyond the page's rank, a direction with sigma ~ 0).
constexpr int kRefineSteps = 8;

__device__ __forceinline__ float refill_value(int row, int col) {
  uint32_t x = (uint32_t)row * 0x9E3779B1u ^ (uint32_t)(col + 1) * 0x85EBCA77u;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  return (float)(int)(x & 0xFFFFu) * (1.f / 32768.f) - 1.f;  // in [-1, 1)
}

template <typename Elem, int N>
__device__ __forceinline__ void orthonormal_columns(TriShared& sh, const Elem* X, int trans, int P,
                                                    float (&qr)[kTriMaxRank], int r, int lane) {
  uint32_t dead = 0;
  const bool weak = orthonormalize<N>(sh, qr, r, lane, dead);
  if (!weak && !dead) return;  // wave-uniform
#pragma unroll
  for (int j = 0; j < kTriMaxRank; ++j)
    if (j < r && ((dead >> j) & 1u) && lane < N) qr[j] = refill_value(lane, j);
#pragma unroll
  for (int jc = 0; jc < kTriMaxRank / 4; ++jc) {
    if (4 * jc < r)
      *(float4*)&sh.u.Z[lane * kZs + 4 * jc] = float4{qr[4 * jc], qr[4 * jc + 1], qr[4 * jc + 2], qr[4 * jc + 3]};
  }
  __syncthreads();
  orthonormalize<N>(sh, qr, r, lane, dead);
  for (int it = 0; it < kRefineSteps; ++it) {
    gram_times<Elem, N>(sh, X, trans, P, qr, r, lane);
    orthonormalize<N>(sh, qr, r, lane, dead);
  }
}

// 6'. INT4 factors of one page (Sec. 4.3), written into its packed part.
// Groups: columns of Lt_K, rows of Lt_V, columns of Rt_K and Rt_V; per group
// the scale is max |x| / 7 rounded nearest-even to bf16, and a code is
// rint(x / scale) clamped to -7..7 (0 where the scale is 0).  The codes go to
// LDS as nibble bytes (c + 8), then each lane assembles whole units of the
// packed layout from them.
__device__ __forceinline__ float q4_scale(float amax) { return bf16_bits_to_f32(f32_to_bf16_bits(amax / 7.f)); }

__device__ __forceinline__ float q4_inv(float s) { return s > 0.f ? 1.f / s : 0.f; }

__device__ __forceinline__ uint32_t q4_nibble(float x, float inv) {
  return (uint32_t)((int)fminf(fmaxf(rintf(x * inv), -7.f), 7.f) + 8);
}

// W nibble bytes (stride `stride`) -> one unit of the packed layout
__device__ __forceinline__ uint32_t q4_pack(const uint8_t* src, int stride, int n, int W) {
  uint32_t u = 0;
  for (int e = 0; e < W; ++e) u |= (e < n ? (uint32_t)src[e * stride] : 8u) << q4_nibble_bit(W, e);
  return u;
}

// ub = 3 units start at any byte: three byte stores
__device__ __forceinline__ void q4_store_unit(uint8_t* p, uint32_t u, int ub) {
  if (ub == 4) {
    *(uint32_t*)p = u;
  } else if (ub == 3) {
    p[0] = (uint8_t)u;
    p[1] = (uint8_t)(u >> 8);
    p[2] = (uint8_t)(u >> 16);
  } else if (ub == 2) {
    *(uint16_t*)p = (uint16_t)u;
  } else {
    *p = (uint8_t)u;
  }
}

__device__ __forceinline__ void q4_store_scale(uint8_t* p, float s) { *(uint16_t*)p = f32_to_bf16_bits(s); }

// N page rows (32: K2 units and V1 rows of page rows 32..63 are not stored).
template <int N>
__device__ __forceinline__ void store_q4(const CompressJob& job, const PageRef& pr, TriShared& sh,
                                         const floatx4 (&R)[2][8], int lane) {
  const int r = pr.r;
  const Q4Dims qd = q4_dims(r, N);
  const int A = qd.pd.A, r8 = 8 * qd.pd.n8, ub = qd.ub;
  const bool keys = pr.kind == 0;
  uint8_t* part = factor_part(job, pr);
  float* hs = sh.w;      // sigma_i^(1/2)
  float* ihs = sh.xrow;  // sigma_i^(-1/2), 0 where sigma_i = 0
  float* lsc = sh.v;     // scales of the columns of Lt_K
  float* linv = sh.b;    // their reciprocals
  if (lane < kTriMaxRank) {
    const float h = lane < r ? sqrtf(sh.sig[lane]) : 0.f;
    hs[lane] = h;
    ihs[lane] = q4_inv(h);
  }
  __syncthreads();

  // Lt row j = lane
  float lt[kTriMaxRank];
  float lmax = 0.f;
#pragma unroll
  for (int i = 0; i < kTriMaxRank; ++i) {
    lt[i] = i < r ? sh.u.Z[lane * kZs + i] * hs[i] : 0.f;
    lmax = fmaxf(lmax, fabsf(lt[i]));
  }
  if (keys) {
    // column maxima of Lt_K: lanes i and i + 32 scan half of column i each
    // (scaling by sigma_i^(1/2) > 0 commutes with the maximum)
    const int i = lane & 31, j0 = (lane >> 5) * 32;
    float m = 0.f;
    if (i < r) {
      for (int j = j0; j < j0 + 32; ++j) m = fmaxf(m, fabsf(sh.u.Z[j * kZs + i]));
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane < kTriMaxRank) {
      const float sc = i < r ? q4_scale(m * hs[i]) : 0.f;
      lsc[lane] = sc;
      linv[lane] = q4_inv(sc);
    }
  }
  __syncthreads();  // Z is read for the last time above; the codes reuse it

  uint8_t* Lc = (uint8_t*)sh.u.Z;              // [kP][32]  nibble bytes of Lt
  uint8_t* Rc = Lc + kP * kTriMaxRank;          // [32][kD]  nibble bytes of Rt
  const float lsv = keys ? 0.f : q4_scale(lmax);  // row scale of Lt_V
  {
    const float rinv = q4_inv(lsv);
#pragma unroll
    for (int i4 = 0; i4 < kTriMaxRank / 4; ++i4) {
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e;
        const uint32_t nb = i < r ? q4_nibble(lt[i], keys ? linv[i] : rinv) : 8u;
        w |= nb << (8 * e);
      }
      if (4 * i4 < r8) *(uint32_t*)&Lc[lane * kTriMaxRank + 4 * i4] = w;
    }
  }
  // Rt = diag(sigma^(-1/2)) R: lane (ci, q) holds rows 16 mi + 4 q + v of
  // channel 16 mc + ci; a channel's maximum spans the four lanes ci + 16 q
  {
    const int ci = lane & 15, q = lane >> 4;
    float ri[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) ri[mi][v] = ihs[16 * mi + 4 * q + v];
    }
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) {
      float rt[2][4];
      float m = 0.f;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          rt[mi][v] = R[mi][mc][v] * ri[mi][v];
          m = fmaxf(m, fabsf(rt[mi][v]));
        }
      }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      const float sc = q4_scale(m), inv = q4_inv(sc);
      const int c = 16 * mc + ci;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = 16 * mi + 4 * q + v;
          if (i < r8) Rc[i * kD + c] = (uint8_t)(i < r ? q4_nibble(rt[mi][v], inv) : 8u);
        }
      }
      if (q == 0) q4_store_scale(part + (keys ? q4_sr_k(qd, c) : q4_sr_v(qd, c)), sc);
    }
  }
  __syncthreads();

  // assemble and store the units
  const int full = A / 4, partial = A % 4 ? 1 : 0;
  if (keys) {
    // K1: Rt_K rank tiles, dwords of 8 channels
    for (int u = lane; u < full * 256 + partial * 128; u += kP) {
      int mt, row, ks, qk, b, v;
      if (u < full * 256) {
        mt = u / 256, row = (u % 256) / 4, ks = u % 4;
        qk = row / 16, b = (row % 16) / 4, v = row % 4;
      } else {
        const int w = u - full * 256;
        mt = full, row = w / 4, ks = w % 4;
        qk = row / 8, b = (row % 8) / 2, v = row % 2;
      }
      const int i = A * b + 4 * mt + v;
      *(uint32_t*)(part + mt * 1024 + (row * 4 + ks) * 4) = q4_pack(&Rc[i * kD + 32 * ks + 8 * qk], 1, 8, 8);
    }
    // K2: Lt_K page-row tiles, units of the lane quad's A ranks (N = 32:
    // the lanes with rho < 8, compacted)
    constexpr int kLanesK2 = N == kP ? 64 : 32;
    for (int u = lane; u < 4 * kLanesK2; u += kP) {
      const int ln = u / 4, mt = u % 4, qk = ln / (kLanesK2 / 4), rho = ln % (kLanesK2 / 4);
      const int j = 16 * (rho / 4) + 4 * mt + rho % 4;
      q4_store_unit(part + qd.k2 + (int64_t)u * ub, q4_pack(&Lc[j * kTriMaxRank + A * qk], 1, A, 2 * ub), ub);
    }
    if (lane < r8) q4_store_scale(part + q4_sl_k(qd, lane), lsc[lane]);
    // the part's tail up to its 64-byte boundary: the host packer's filler,
    // so that a part's bytes depend on the page alone
    for (int64_t b = qd.sl_k + 2 * r8 + lane; b < qd.k_bytes; b += kP) part[b] = 0x88;
  } else {
    // V1: Lt_V^T rank tiles, dwords of 8 tokens (N = 32: the rows of lanes
    // 0..31, a compacted last tile's 16)
    constexpr int kRows = N == kP ? 64 : 32;  // rows of a full tile
    for (int u = lane; u < full * 2 * kRows + partial * kRows; u += kP) {
      int mt, row, ks, qk, b, v;
      if (u < full * 2 * kRows) {
        mt = u / (2 * kRows), row = (u % (2 * kRows)) / 2, ks = u % 2;
        qk = row / 16, b = (row % 16) / 4, v = row % 4;
      } else {
        const int w = u - full * 2 * kRows;
        mt = full, row = w / 2, ks = w % 2;
        qk = row / 8, b = (row % 8) / 2, v = row % 2;
      }
      const int i = A * b + 4 * mt + v;
      *(uint32_t*)(part + mt * 8 * kRows + (row * 2 + ks) * 4) =
          q4_pack(&Lc[(16 * qk + 8 * ks) * kTriMaxRank + i], kTriMaxRank, 8, 8);
    }
    // V2: Rt_V^T channel tiles, units of the lane quad's A ranks
    for (int u = lane; u < 512; u += kP) {
      const int ln = u / 8, mt = u % 8, qk = ln / 16, c = 16 * mt + ln % 16;
      q4_store_unit(part + qd.v2 + (int64_t)u * ub, q4_pack(&Rc[A * qk * kD + c], kD, A, 2 * ub), ub);
    }
    if (lane < N) q4_store_scale(part + q4_sl_v(qd, lane), lsv);
    for (int64_t b = qd.sr_v + 2 * kD + lane; b < qd.v_bytes; b += kP) part[b] = 0x88;
  }
}

__device__ inline const CompressJob& base_job(const CompressJob& job) { return job; }
__device__ inline const CompressJob& base_job(const CompressBatch& jb) { return jb.base; }

template <typename Elem, bool kQ4, int N, class J>
__device__ __forceinline__ void compress_tri_one(const J& jobs, int64_t n, TriShared& sh, int lane) {
  const CompressJob& job = base_job(jobs);
  const PageRef pr = page_ref(jobs, n, (int)sizeof(Elem));
  const Elem* X = (const Elem*)pr.X;
  const int r = pr.r;

  float qh[kP];
  float my_a, my_b;
  {
    float g[kP];
    gram_rows<Elem>(X, pr.trans, pr.P, sh, g, lane);
    tridiagonalize<N>(sh, g, qh, lane, my_a, my_b);
  }

  // T to LDS, Gershgorin interval, pivot floor
  sh.a[lane] = my_a;
  sh.b[lane] = lane < kP - 1 ? my_b : 0.f;
  __syncthreads();
  const float bl = lane > 0 ? sh.b[lane - 1] : 0.f, br = sh.b[lane];
  const float glo = wave_reduce<2>(my_a - fabsf(bl) - fabsf(br));
  const float ghi = wave_reduce<1>(my_a + fabsf(bl) + fabsf(br));
  const float pivmin = 0x1p-126f * fmaxf(1.f, wave_reduce<1>(br * br));
  sh.b2s[lane] = fmaxf(bl * bl, 0x1p-126f);
  __syncthreads();

  // 3. the r largest eigenvalues.  First round: the 64 lanes count at 64
  // points spread over the Gershgorin interval, which brackets every
  // eigenvalue to 1/65 of it; then L lanes per eigenvalue refine their
  // bracket by L-point multisection.
  int rp = 1;
  while (rp < r) rp <<= 1;
  const int L = kP / rp;
  const int t = lane & (L - 1);
  const int jl = lane / L;
  const int j = jl < r ? jl : r - 1;  // descending index
  const int m = N - 1 - j;            // ascending index (the zero block's N below)
  float lo = glo, hi = ghi;
  {
    const float x0 = fmaf(ghi - glo, (float)(lane + 1) / (float)(kP + 1), glo);
    sh.xrow[lane] = x0;
    sh.w[lane] = __int_as_float(sturm_count<N>(sh, x0));
    __syncthreads();
#pragma unroll 8
    for (int l = 0; l < kP; ++l) {
      const float xl = sh.xrow[l];
      const int cl = __float_as_int(sh.w[l]);
      if (cl <= m) lo = fmaxf(lo, xl);
      else hi = fminf(hi, xl);
    }
  }
  const int rounds = multisection_rounds(L);
  const float frac = (float)(t + 1) / (float)(L + 1);
  for (int it = 0; it < rounds; ++it) {
    const float x = fmaf(hi - lo, frac, lo);
    const int cnt = sturm_count<N>(sh, x);
    float nlo = cnt <= m ? x : lo, nhi = cnt <= m ? hi : x;
    for (int o = 1; o < L; o <<= 1) {
      nlo = fmaxf(nlo, __shfl_xor(nlo, o));
      nhi = fminf(nhi, __shfl_xor(nhi, o));
    }
    lo = nlo;
    hi = nhi;
  }
  const float lam = 0.5f * (lo + hi);

  // 4. eigenvectors of T -> Z[:, j]
  twisted_vector<N>(sh, lam, pivmin, j, t == 0 && jl < r);
  __syncthreads();

  // 5a. Q_r = Q_H Z: lane i forms row i
  float qr[kTriMaxRank];
#pragma unroll
  for (int jc = 0; jc < kTriMaxRank / 4; ++jc) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (4 * jc < r) {
#pragma unroll
      for (int mm = 0; mm < N; ++mm) {  // Z has N rows; Q_H's other columns are e_i
        if ((mm & 3) == 0) __builtin_amdgcn_sched_barrier(0);
        const float4 z4 = *(const float4*)&sh.u.Z[mm * kZs + 4 * jc];
        acc.x = fmaf(qh[mm], z4.x, acc.x);
        acc.y = fmaf(qh[mm], z4.y, acc.y);
        acc.z = fmaf(qh[mm], z4.z, acc.z);
        acc.w = fmaf(qh[mm], z4.w, acc.w);
      }
    }
    qr[4 * jc] = acc.x;
    qr[4 * jc + 1] = acc.y;
    qr[4 * jc + 2] = acc.z;
    qr[4 * jc + 3] = acc.w;
  }
  __syncthreads();
#pragma unroll
  for (int jc = 0; jc < kTriMaxRank / 4; ++jc) {
    if (4 * jc < r)
      *(float4*)&sh.u.Z[lane * kZs + 4 * jc] = float4{qr[4 * jc], qr[4 * jc + 1], qr[4 * jc + 2], qr[4 * jc + 3]};
  }
  __syncthreads();
  // 5a'. Orthonormalize Q_r (the twisted vectors of close eigenvalues are
  // orthogonal only to about eps ||T|| / gap), and resolve clusters the
  // bisection could not split
  orthonormal_columns<Elem, N>(sh, X, pr.trans, pr.P, qr, r, lane);

  // 5b. R = Q_r^T X in fp32 on the matrix cores: lane (ci, q) holds
  // R[16 mi + 4 q + v][16 mc + ci]
  const int ci = lane & 15, q = lane >> 4;
  const int RT16 = (r + 15) / 16;
  floatx4 R[2][8];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) R[mi][mc] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll 2
  for (int kc = 0; kc < N / 4; ++kc) {  // page rows
    __builtin_amdgcn_sched_barrier(0);
    const int jr = 4 * kc + q;
    float bv[8];
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) bv[mc] = page_elem(X, pr.trans, pr.P, jr, 16 * mc + ci);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      if (mi < RT16) {
        const int col = 16 * mi + ci;
        const float av = col < r ? sh.u.Z[jr * kZs + col] : 0.f;
#pragma unroll
        for (int mc = 0; mc < 8; ++mc)
          R[mi][mc] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[mc], R[mi][mc], 0, 0, 0);
      }
    }
  }
  // sigma_i = ||R_i||
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (mi < RT16) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float ss = 0.f;
#pragma unroll
        for (int mc = 0; mc < 8; ++mc) ss = fmaf(R[mi][mc][v], R[mi][mc][v], ss);
        ss = row16_reduce<0>(ss);
        const int i = 16 * mi + 4 * q + v;
        if (ci == 0 && i < r) sh.sig[i] = sqrtf(ss);
      }
    }
  }
  __syncthreads();

  if constexpr (kQ4) {
    store_q4<N>(job, pr, sh, R, lane);
    __syncthreads();
    return;
  }

  // 6. Rf = R / sigma, Lf = Q_r diag(sigma)
  const FactorDst dst(job, pr, n);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (16 * mi < dst.rf_store) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * mi + 4 * q + v;
        if (i < dst.rf_store) {
          const float sg = i < r ? sh.sig[i] : 0.f;
          const float inv = sg > 0.f ? 1.f / sg : 0.f;
#pragma unroll
          for (int mc = 0; mc < 8; ++mc) {
            const float val = i < r ? R[mi][mc][v] * inv : 0.f;
            store_elem(dst.rf, dst.rf_idx(i, 16 * mc + ci), job.out_dtype, val);
          }
        }
      }
    }
  }
  for (int i = 0; i < dst.r_store && lane < N; ++i) {  // page rows
    float val = 0.f;
    if (i < r) {
      const float sg = sh.sig[i];
      val = sg > 0.f ? sh.u.Z[lane * kZs + i] * sg : 0.f;
    }
    store_elem(dst.lf, dst.lf_idx(lane, i), job.out_dtype, val);
  }
  if (!dst.packed && job.sigma != nullptr && lane < r) job.sigma[n * r + lane] = sh.sig[lane];
  __syncthreads();
}

// One page per workgroup (no page loop: a loop around the page body costs the
// register allocator ~70 extra VGPRs).  Page n = blockIdx.y * gridDim.x + blockIdx.x.
template <typename Elem, bool kQ4, int N>
__global__ __launch_bounds__(64, 3) void compress_tri_kernel(CompressJob job) {
  __shared__ TriShared sh;
  const int64_t n = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  if (n < job.n_pages) compress_tri_one<Elem, kQ4, N>(job, n, sh, threadIdx.x);
}

// The batch of cache jobs; the first page of a member also sets its table
// entry (read only by later launches on the stream).
template <typename Elem, bool kQ4, int N>
__global__ __launch_bounds__(64, 3) void compress_tri_batch_kernel(CompressBatch jb) {
  __shared__ TriShared sh;
  const int64_t n = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t per = jb.base.n_pages;
  if (n >= per * jb.n) return;
  const CompressMember& m = jb.m[n / per];
  if (n % per == 0 && threadIdx.x == 0 && m.table) m.table[m.table_page] = m.table_entry;
  compress_tri_one<Elem, kQ4, N>(jb, n, sh, threadIdx.x);
}

// Grid of n pages: x up to 65536, y the rest.
bool page_grid(int64_t n, dim3& grid) {
  constexpr int64_t kGx = 65536;
  const int64_t gx = n < kGx ? n : kGx;
  const int64_t gy = (n + gx - 1) / gx;
  if (gy > 65535) return false;
  grid = dim3((unsigned)gx, (unsigned)gy);
  return true;
}

}  // namespace

hipError_t launch_compress_batch(const CompressBatch& jb, hipStream_t stream) {
  const CompressJob& job = jb.base;
  if (jb.n < 1 || jb.n > kMaxBatchCaches || job.n_pages <= 0) return hipErrorInvalidValue;
  const int r_max = job.rank[1] > job.rank[0] ? job.rank[1] : job.rank[0];
  if (r_max > kTriMaxRank || job.n_kind != 2) return hipErrorNotSupported;
  const KernelEvents ev = take_kernel_events();  // pkv_time_next_kernel brackets this launch
  dim3 grid;
  if (!page_grid(job.n_pages * jb.n, grid)) return hipErrorInvalidValue;
  const bool q4 = job.out_dtype == PKV_BF16_INT4;
  if (q4 && job.in_dtype != PKV_BF16) return hipErrorInvalidValue;
  if (job.page_rows != kP && job.page_rows != kMinP) return hipErrorInvalidValue;
  const bool full = job.page_rows == kP;
  if (q4 && full)
    hipExtLaunchKernelGGL((compress_tri_batch_kernel<uint16_t, true, kP>), grid, dim3(64), 0, stream, ev.start, ev.stop, 0,
                          jb);
  else if (q4)
    hipExtLaunchKernelGGL((compress_tri_batch_kernel<uint16_t, true, kMinP>), grid, dim3(64), 0, stream, ev.start, ev.stop, 0,
                          jb);
  else if (job.in_dtype == PKV_BF16 && full)
    hipExtLaunchKernelGGL((compress_tri_batch_kernel<uint16_t, false, kP>), grid, dim3(64), 0, stream, ev.start, ev.stop, 0,
                          jb);
  else if (job.in_dtype == PKV_BF16)
    hipExtLaunchKernelGGL((compress_tri_batch_kernel<uint16_t, false, kMinP>), grid, dim3(64), 0, stream, ev.start, ev.stop, 0,
                          jb);
  else if (full)
    hipExtLaunchKernelGGL((compress_tri_batch_kernel<float, false, kP>), grid, dim3(64), 0, stream, ev.start, ev.stop, 0,
                          jb);
  else
    hipExtLaunchKernelGGL((compress_tri_batch_kernel<float, false, kMinP>), grid, dim3(64), 0, stream, ev.start, ev.stop, 0,
                          jb);
  return hipGetLastError();
}

hipError_t launch_compress_tri(const CompressJob& job, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop) {
  dim3 grid;
  if (!page_grid(job.n_pages, grid)) return hipErrorInvalidValue;
  const bool q4 = job.out_dtype == PKV_BF16_INT4;
  if (q4 && (job.fac == nullptr || job.in_dtype != PKV_BF16)) return hipErrorInvalidValue;
  if (job.page_rows != kP && job.page_rows != kMinP) return hipErrorInvalidValue;
  const bool full = job.page_rows == kP;
  if (q4 && full)
    hipExtLaunchKernelGGL((compress_tri_kernel<uint16_t, true, kP>), grid, dim3(64), 0, stream, start, stop, 0, job);
  else if (q4)
    hipExtLaunchKernelGGL((compress_tri_kernel<uint16_t, true, kMinP>), grid, dim3(64), 0, stream, start, stop, 0,
                          job);
  else if (job.in_dtype == PKV_BF16 && full)
    hipExtLaunchKernelGGL((compress_tri_kernel<uint16_t, false, kP>), grid, dim3(64), 0, stream, start, stop, 0, job);
  else if (job.in_dtype == PKV_BF16)
    hipExtLaunchKernelGGL((compress_tri_kernel<uint16_t, false, kMinP>), grid, dim3(64), 0, stream, start, stop, 0,
                          job);
  else if (full)
    hipExtLaunchKernelGGL((compress_tri_kernel<float, false, kP>), grid, dim3(64), 0, stream, start, stop, 0, job);
  else
    hipExtLaunchKernelGGL((compress_tri_kernel<float, false, kMinP>), grid, dim3(64), 0, stream, start, stop, 0, job);
  return hipGetLastError();
}

}  // namespace pkv
