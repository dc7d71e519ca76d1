// Batched page decomposition on gfx950, Jacobi route (any rank; launch_compress
// sends ranks up to 32 to the tridiagonal route in pkv_compress_tri.hip).
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
#include "pkv_compress_common.h"

namespace pkv {
namespace {

using namespace cmp;

constexpr int kMaxSweeps = 24;

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

// The 10 upper 16x16 tiles of G = X X^T, spread over the page's waves.
template <typename Elem, int WPP>
__device__ void gram(const Elem* X, int trans, int P, float* Gs, int lane, int wv) {
  for (int tile = wv; tile < 10; tile += WPP) {
    // tile -> (ta, tb), ta <= tb
    int ta = 0, rem = tile;
    while (rem >= 4 - ta) {
      rem -= 4 - ta;
      ++ta;
    }
    const int tb = ta + rem;
    const floatx4 acc = gram_tile(X, trans, P, ta, tb, lane);
    store_gram_tile(Gs, ta, tb, acc, lane);
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

struct JacobiShared {
  float c[32], s[32];
  float trace;
  int any[2];  // a rotation happened in the sweep of this parity
};

// Advance a circle-method index to the next round: every index below 63
// moves to the next seat (mod 63), index 63 stays.
__device__ inline int rr_next(int x) { return x == 63 ? 63 : (x == 62 ? 0 : x + 1); }

// Cyclic Jacobi on G (in LDS), accumulating the rotations into V.  Each round
// rotates the 32 disjoint pairs of the circle-method schedule.  G <- J^T G J
// is applied block by block: the 2x2 block at (pair i, pair j) is read once,
// rotated on both sides and written once; V <- V J in the same pass.  Each
// thread gathers all operands of its blocks before rotating, so the LDS reads
// pipeline.  A thread's blocks keep their pair numbers across rounds; their
// row/column indices advance one seat per round.  Two barriers per round and
// one sweep-level convergence test.
template <int WPP>
__device__ void jacobi(float* Gs, float* Vs, JacobiShared& sh, int lane, int wv) {
  constexpr int NT = 64 * WPP;
  constexpr int NB = 1024 / NT;  // G blocks per thread per round
  constexpr int NV = 2048 / NT;  // V (row, pair) updates per thread per round
  const int tid = wv * 64 + lane;
  if (wv == 0) {
    float tr = Gs[lane * kLd + lane];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tr += __shfl_xor(tr, o);
    if (lane == 0) {
      sh.trace = tr;
      sh.any[0] = 0;
      sh.any[1] = 0;
    }
  }
  __syncthreads();
  const float tol_abs = sh.trace * 0x1p-30f;
  const float tol_rel = 0x1p-23f;

  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    // indices at round 0 of the sweep
    int pa = 0, qa = 0;  // phase-A pair (threads < 32)
    if (tid < 32) rr_pair(0, tid, pa, qa);
    int bpi[NB], bqi[NB], bpj[NB], bqj[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int blk = tid + NT * u;
      rr_pair(0, blk >> 5, bpi[u], bqi[u]);
      rr_pair(0, blk & 31, bpj[u], bqj[u]);
    }
    int vp_[NV], vq_[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) rr_pair(0, (tid + NT * u) >> 6, vp_[u], vq_[u]);

    for (int t = 0; t < 63; ++t) {
      // phase A: thread k < 32 owns pair k
      if (tid < 32) {
        const float app = Gs[pa * kLd + pa], aqq = Gs[qa * kLd + qa], apq = Gs[pa * kLd + qa];
        const float thr = fmaxf(tol_rel * sqrtf(fabsf(app * aqq)), tol_abs);
        float c = 1.f, s = 0.f;
        if (fabsf(apq) > thr) {
          const float tau = (aqq - app) / (2.f * apq);
          const float tt = copysignf(1.f, tau) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + tt * tt);
          s = tt * c;
          sh.any[sweep & 1] = 1;
        }
        sh.c[tid] = c;
        sh.s[tid] = s;
      }
      __syncthreads();
      // every thread has read the previous sweep's flag by now: reset the
      // flag the next sweep will use
      if (t == 0 && tid == 0) sh.any[(sweep + 1) & 1] = 0;
      // G <- J^T G J over this thread's 2x2 blocks (pair i, pair j)
      {
        float g[NB][4];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          g[u][0] = Gs[bpi[u] * kLd + bpj[u]];
          g[u][1] = Gs[bpi[u] * kLd + bqj[u]];
          g[u][2] = Gs[bqi[u] * kLd + bpj[u]];
          g[u][3] = Gs[bqi[u] * kLd + bqj[u]];
        }
        float vp[NV], vq[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int row = ((tid + NT * u) & 63) * kLd;
          vp[u] = Vs[row + vp_[u]];
          vq[u] = Vs[row + vq_[u]];
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int blk = tid + NT * u;
          const int i = blk >> 5, j = blk & 31;
          const float c1 = sh.c[i], s1 = sh.s[i], c2 = sh.c[j], s2 = sh.s[j];
          // rows (J^T .): [p; q] <- [c p - s q; s p + c q]
          const float A = c1 * g[u][0] - s1 * g[u][2], Bv = c1 * g[u][1] - s1 * g[u][3];
          const float C = s1 * g[u][0] + c1 * g[u][2], D = s1 * g[u][1] + c1 * g[u][3];
          // columns (. J)
          Gs[bpi[u] * kLd + bpj[u]] = c2 * A - s2 * Bv;
          Gs[bpi[u] * kLd + bqj[u]] = s2 * A + c2 * Bv;
          Gs[bqi[u] * kLd + bpj[u]] = c2 * C - s2 * D;
          Gs[bqi[u] * kLd + bqj[u]] = s2 * C + c2 * D;
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int idx = tid + NT * u;
          const int row = (idx & 63) * kLd, j = idx >> 6;
          const float c = sh.c[j], s = sh.s[j];
          Vs[row + vp_[u]] = c * vp[u] - s * vq[u];
          Vs[row + vq_[u]] = s * vp[u] + c * vq[u];
        }
      }
      __syncthreads();
      // a rotation annihilates its pair's off-diagonal exactly; the next
      // round's phase A reads other entries and its barrier orders these
      if (tid < 32 && sh.s[tid] != 0.f) {
        Gs[pa * kLd + qa] = 0.f;
        Gs[qa * kLd + pa] = 0.f;
      }
      // next round's indices
      pa = rr_next(pa);
      qa = rr_next(qa);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        bpi[u] = rr_next(bpi[u]);
        bqi[u] = rr_next(bqi[u]);
        bpj[u] = rr_next(bpj[u]);
        bqj[u] = rr_next(bqj[u]);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        vp_[u] = rr_next(vp_[u]);
        vq_[u] = rr_next(vq_[u]);
      }
    }
    __syncthreads();
    if (!sh.any[sweep & 1]) break;
  }
}

struct CompressShared {
  float G[kP * kLd];
  float V[kP * kLd];
  JacobiShared js;
  int sel[kP];
  float sig2[16][kP];
  float sig[kP];
};

template <typename Elem, int WPP>
__device__ void compress_one(const CompressJob& job, int64_t n, CompressShared& sh, int lane,
                             int wv) {
  const int tid = wv * 64 + lane;
  const PageRef pr = page_ref(job, n, (int)sizeof(Elem));
  const int kind = pr.kind;
  const Elem* X = (const Elem*)pr.X;
  const int trans = pr.trans;
  const int r = pr.r;  // the job's largest rank is > 32, so the page has 64 rows (launch_compress)

  // 1. Gram matrix, eigenvector accumulator = I
  gram<Elem, WPP>(X, trans, kP, sh.G, lane, wv);
  for (int idx = tid; idx < kP * kP; idx += 64 * WPP) {
    const int j = idx / kP, c = idx % kP;
    sh.V[j * kLd + c] = (j == c) ? 1.f : 0.f;
  }
  __syncthreads();

  // 2. Jacobi eigen-solve
  jacobi<WPP>(sh.G, sh.V, sh.js, lane, wv);

  // 3. top-r selection: rank of each eigenvalue (descending, ties by index)
  if (wv == 0) {
    const float lam = sh.G[lane * kLd + lane];
    int rank = 0;
    for (int y = 0; y < kP; ++y) {
      const float ly = sh.G[y * kLd + y];
      rank += (ly > lam || (ly == lam && y < lane)) ? 1 : 0;
    }
    sh.sel[rank] = lane;
  }
  __syncthreads();

  // R = Q_r^T X in fp32 on the matrix cores; each wave takes 8 / WPP of the
  // 16-channel column tiles, all 16-rank row tiles
  constexpr int MC = 8 / WPP;
  const int ci = lane & 15, q = lane >> 4;
  const int RT16 = (r + 15) / 16;
  floatx4 R[4][MC];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int m = 0; m < MC; ++m) R[mi][m] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  int colsel[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int irow = 16 * mi + ci;
    colsel[mi] = irow < r ? sh.sel[irow] : -1;
  }
  // X operands of a reduction step are loaded once and reused by every rank tile
#pragma unroll 2
  for (int kc = 0; kc < kP / 4; ++kc) {
    const int j = 4 * kc + q;
    float bv[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m) bv[m] = page_elem(X, trans, kP, j, 16 * (wv * MC + m) + ci);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi < RT16) {
        const float av = colsel[mi] >= 0 ? sh.V[j * kLd + colsel[mi]] : 0.f;
#pragma unroll
        for (int m = 0; m < MC; ++m)
          R[mi][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[m], R[mi][m], 0, 0, 0);
      }
    }
  }
  // sigma_i^2 = sum over channels of R_i^2: lane (ci, q) holds rows
  // 16 mi + 4 q + v of its wave's channel tiles
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (mi < RT16) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < MC; ++m) ss += R[mi][m][v] * R[mi][m][v];
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        if (ci == 0) sh.sig2[wv][16 * mi + 4 * q + v] = ss;
      }
    }
  }
  __syncthreads();
  if (tid < kP) {
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < WPP; ++w) ss += sh.sig2[w][tid];
    sh.sig[tid] = sqrtf(ss);
  }
  __syncthreads();

  // 4. store Rf = R / sigma and Lf = Q diag(sigma)
  const bool packed = job.fac != nullptr;
  const PackDims pd = pack_dims(r);
  const int r_store = packed ? 8 * pd.n8 : r;
  // a packed value part holds Rf_V at r2 ranks (the exact rank, rounded up
  // to even, when r8 <= 32: a job's value rank may be that small while its
  // key rank takes this route)
  const int rf_store = packed && kind != 0 ? pd.r2 : r_store;
  uint8_t* part = nullptr;
  if (packed) part = factor_part(job, pr);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (16 * mi < rf_store) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * mi + 4 * q + v;
        if (i < rf_store) {
          const float sg = i < r ? sh.sig[i] : 0.f;
          const float inv = sg > 0.f ? 1.f / sg : 0.f;
#pragma unroll
          for (int m = 0; m < MC; ++m) {
            const int c = 16 * (wv * MC + m) + ci;
            const float val = (i < r) ? R[mi][m][v] * inv : 0.f;
            int64_t idx;
            if (!packed) idx = n * (int64_t)r * kD + (int64_t)i * kD + c;
            else idx = off_rf(kind == 0 ? job.key_part_kind : PKV_VALUES, pd, i, c);
            store_elem(packed ? (void*)part : job.rf, idx, job.out_dtype, val);
          }
        }
      }
    }
  }
  for (int i = wv; i < r_store; i += WPP) {
    const int j = lane;  // page row
    float val = 0.f;
    if (i < r) {
      const float sg = sh.sig[i];
      val = sg > 0.f ? sh.V[j * kLd + sh.sel[i]] * sg : 0.f;
    }
    int64_t idx;
    if (!packed) idx = n * (int64_t)kP * r + (int64_t)j * r + i;
    else idx = (kind == 0) ? off_lf_k(pd, j, i) : off_lf_v(pd, j, i);
    store_elem(packed ? (void*)part : job.lf, idx, job.out_dtype, val);
  }
  if (!packed && job.sigma != nullptr && tid < r) job.sigma[n * r + tid] = sh.sig[tid];
  __syncthreads();
}

// Throughput mode (4 waves per page) is held to 128 VGPRs so that four pages
// share a CU, as the LDS allows (measured: 507K pages/s at four pages per CU,
// 448K at three, 332K at two, 181K at one, despite the spills this costs);
// latency mode keeps the full register budget.
template <typename Elem, int WPP>
__global__ __launch_bounds__(64 * WPP, (WPP == 4 ? 4 : 1)) void compress_kernel(CompressJob job) {
  __shared__ CompressShared sh;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int64_t n = blockIdx.x; n < job.n_pages; n += gridDim.x)
    compress_one<Elem, WPP>(job, n, sh, lane, wv);
}

// Few pages (a promotion): eight waves per page to cut latency.  Many pages
// (prefill, batched compression): four waves per page, four pages per CU.
constexpr int64_t kLatencyModePages = 512;

}  // namespace

hipError_t launch_compress(const CompressJob& job, hipStream_t stream) {
  if (job.n_pages <= 0) return hipSuccess;
  const KernelEvents ev = take_kernel_events();
  const int r_max = job.n_kind == 2 && job.rank[1] > job.rank[0] ? job.rank[1] : job.rank[0];
  if (r_max <= kTriMaxRank) return launch_compress_tri(job, stream, ev.start, ev.stop);
  if (job.page_rows != kP) return hipErrorInvalidValue;  // ranks above 32 need 64-row pages
  const int64_t cap = 1 << 30;
  const unsigned grid = (unsigned)(job.n_pages < cap ? job.n_pages : cap);
  const bool few = job.n_pages <= kLatencyModePages;
  if (job.in_dtype == PKV_BF16) {
    if (few)
      hipExtLaunchKernelGGL((compress_kernel<uint16_t, 8>), dim3(grid), dim3(512), 0, stream, ev.start,
                            ev.stop, 0, job);
    else
      hipExtLaunchKernelGGL((compress_kernel<uint16_t, 4>), dim3(grid), dim3(256), 0, stream, ev.start,
                            ev.stop, 0, job);
  } else {
    if (few)
      hipExtLaunchKernelGGL((compress_kernel<float, 8>), dim3(grid), dim3(512), 0, stream, ev.start,
                            ev.stop, 0, job);
    else
      hipExtLaunchKernelGGL((compress_kernel<float, 4>), dim3(grid), dim3(256), 0, stream, ev.start,
                            ev.stop, 0, job);
  }
  return hipGetLastError();
}

}  // namespace pkv
