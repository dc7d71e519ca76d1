// Dense pools, page table and token append of the hybrid cache.
//
// PuzzleKV Sec. 3.3 (1)-(3): after prefill the sink pages and the recent
// window (completed window pages plus the page being filled) stay dense;
// Sec. 3.3 "Incremental Cache Update (5)": each new key/value pair is written
// into the most recent dense page and takes part in attention at once.
//
// Dense pages live in two pools per (sequence, KV head): n_s sink slots and a
// ring of n_w + 1 window slots (n_w completed pages plus the partial page; the
// slot of the page that leaves the window is the one the next page reuses).
// Keys are stored row-major [P][d]; values transposed [d][P] so the attention
// kernel's p V contraction reads contiguous page rows.
#include "pkv_internal.h"

namespace pkv {
namespace {

// Logical page held by a dense slot of a cache of length T (pages of P
// tokens) with n_fact factorized pages, or -1 when the slot is unused.
__device__ inline int64_t slot_page(int slot_id, int n_s, int n_w, int64_t T, int64_t n_fact, int P) {
  const int64_t n_pages = (T + P - 1) / P;
  if (slot_id < n_s) return slot_id < n_pages ? slot_id : -1;
  const int k = slot_id - n_s;
  const int64_t first = (int64_t)n_s + n_fact;  // first dense page after the factors
  if (first >= n_pages) return -1;
  const int64_t ring = n_w + 1;
  const int64_t off = ((k - (first - n_s)) % ring + ring) % ring;
  const int64_t p = first + off;
  return p < n_pages ? p : -1;
}

template <typename Elem>
__global__ __launch_bounds__(256) void prefill_dense_kernel(CacheGeom g, const Elem* K, const Elem* V,
                                                            int64_t T, int64_t n_fact) {
  __shared__ Elem tile[kP][kD + 2];  // P <= kP rows
  const int P = g.P;
  const int slot_id = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * g.Hkv + h;
  const int64_t p = slot_page(slot_id, g.n_s, g.n_w, T, n_fact, P);
  const int64_t nv = p < 0 ? 0 : ((T - p * P) < P ? (T - p * P) : P);
  Elem *dk, *dv;
  const int64_t ppg = (int64_t)P * kD;
  if (slot_id < g.n_s) {
    dk = (Elem*)(g.base + g.lay.sink_k) + (bh * g.n_s + slot_id) * ppg;
    dv = (Elem*)(g.base + g.lay.sink_v) + (bh * g.n_s + slot_id) * ppg;
  } else {
    const int k = slot_id - g.n_s;
    dk = (Elem*)(g.base + g.lay.win_k) + (bh * (g.n_w + 1) + k) * ppg;
    dv = (Elem*)(g.base + g.lay.win_v) + (bh * (g.n_w + 1) + k) * ppg;
  }
  const Elem* sk = K + (bh * T + (p < 0 ? 0 : p * P)) * kD;
  const Elem* sv = V + (bh * T + (p < 0 ? 0 : p * P)) * kD;
  for (int idx = threadIdx.x; idx < P * kD; idx += 256) {
    const int j = idx / kD, c = idx % kD;
    dk[idx] = j < nv ? sk[idx] : Elem(0);
    tile[j][c] = j < nv ? sv[idx] : Elem(0);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < P * kD; idx += 256) {
    const int c = idx / P, j = idx % P;
    dv[idx] = tile[j][c];
  }
}

// Chunked prefill: rows of pages [p_lo, p_hi) that fall in the chunk's token
// range [T0, T1) are copied from the chunk (K, V [B][H_kv][C][d], C = T1 - T0)
// into the pages' dense slots (sink slot p, or ring slot (p - n_s) mod
// (n_w + 1)); other rows of the slots are left as they are.  One workgroup per
// (page, KV head, sequence).
template <typename Elem>
__global__ __launch_bounds__(256) void chunk_dense_kernel(CacheGeom g, const Elem* K, const Elem* V,
                                                          int64_t T0, int64_t T1, int64_t p_lo) {
  __shared__ Elem tile[kP][kD + 2];  // P <= kP rows
  const int P = g.P;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t p = p_lo + blockIdx.x;
  const int64_t bh = (int64_t)b * g.Hkv + h;
  const int64_t C = T1 - T0;
  const int64_t t0 = p * P > T0 ? p * P : T0;
  const int64_t t1 = p * P + P < T1 ? p * P + P : T1;
  if (t1 <= t0) return;
  const int r0 = (int)(t0 - p * P), nr = (int)(t1 - t0);
  const int64_t ppg = (int64_t)P * kD;
  Elem *dk, *dv;
  if (p < g.n_s) {
    dk = (Elem*)(g.base + g.lay.sink_k) + (bh * g.n_s + p) * ppg;
    dv = (Elem*)(g.base + g.lay.sink_v) + (bh * g.n_s + p) * ppg;
  } else {
    const int64_t slot = (p - g.n_s) % (g.n_w + 1);
    dk = (Elem*)(g.base + g.lay.win_k) + (bh * (g.n_w + 1) + slot) * ppg;
    dv = (Elem*)(g.base + g.lay.win_v) + (bh * (g.n_w + 1) + slot) * ppg;
  }
  const Elem* sk = K + (bh * C + (t0 - T0)) * kD;
  const Elem* sv = V + (bh * C + (t0 - T0)) * kD;
  for (int idx = threadIdx.x; idx < nr * kD; idx += 256) {
    const int j = idx / kD, c = idx % kD;
    dk[(r0 + j) * kD + c] = sk[idx];
    tile[j][c] = sv[idx];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nr * kD; idx += 256) {
    const int c = idx / nr, j = idx % nr;
    dv[c * P + r0 + j] = tile[j][c];
  }
}

__device__ inline int32_t classify_entry(int64_t p, int64_t T, int n_s, int n_w, int64_t n_fact, int P) {
  const int64_t n_full = T / P, n_pages = (T + P - 1) / P;
  if (p >= n_pages) return table_entry(PKV_PAGE_UNUSED, 0);
  if (p < n_s) return table_entry(PKV_PAGE_SINK, (int)p);
  if (p < n_s + n_fact) return table_entry(PKV_PAGE_FACT, (int)(p - n_s));
  const int ring = (int)((p - n_s) % (n_w + 1));
  return table_entry(p < n_full ? PKV_PAGE_WIN : PKV_PAGE_PART, ring);
}

__global__ void table_fill_kernel(int32_t* table, int64_t max_pages, int64_t T, int n_s, int n_w,
                                  int64_t n_fact, int P) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p < max_pages) table[p] = classify_entry(p, T, n_s, n_w, n_fact, P);
}

__global__ void table_set_kernel(int32_t* table, int64_t page, int32_t entry) {
  if (threadIdx.x == 0) table[page] = entry;
}

template <typename Elem>
__global__ __launch_bounds__(128) void append_kernel(CacheGeom g, const Elem* k, const Elem* v,
                                                     int64_t T) {
  const int P = g.P;
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t bh = (int64_t)b * g.Hkv + h;
  const int64_t p = T / P;
  const int row = (int)(T % P);
  const int64_t ppg = (int64_t)P * kD;
  Elem *dk, *dv;
  if (p < g.n_s) {
    dk = (Elem*)(g.base + g.lay.sink_k) + (bh * g.n_s + p) * ppg;
    dv = (Elem*)(g.base + g.lay.sink_v) + (bh * g.n_s + p) * ppg;
  } else {
    const int64_t slot = (p - g.n_s) % (g.n_w + 1);
    dk = (Elem*)(g.base + g.lay.win_k) + (bh * (g.n_w + 1) + slot) * ppg;
    dv = (Elem*)(g.base + g.lay.win_v) + (bh * (g.n_w + 1) + slot) * ppg;
  }
  dk[row * kD + c] = k[bh * kD + c];
  dv[(int64_t)c * P + row] = v[bh * kD + c];
  if (b == 0 && h == 0 && c == 0) {
    int32_t* table = (int32_t*)(g.base + g.lay.page_table);
    int32_t e;
    if (p < g.n_s) e = table_entry(PKV_PAGE_SINK, (int)p);
    else e = table_entry(row == P - 1 ? PKV_PAGE_WIN : PKV_PAGE_PART, (int)((p - g.n_s) % (g.n_w + 1)));
    table[p] = e;
  }
}

}  // namespace

hipError_t launch_prefill_dense(const CacheGeom& g, const void* K, const void* V, int64_t T,
                                int64_t n_fact, hipStream_t stream) {
  const dim3 grid(g.n_s + g.n_w + 1, g.Hkv, g.B);
  if (dense_dtype(g.dtype) == PKV_BF16)
    hipLaunchKernelGGL(prefill_dense_kernel<uint16_t>, grid, dim3(256), 0, stream, g,
                       (const uint16_t*)K, (const uint16_t*)V, T, n_fact);
  else
    hipLaunchKernelGGL(prefill_dense_kernel<float>, grid, dim3(256), 0, stream, g, (const float*)K,
                       (const float*)V, T, n_fact);
  return hipGetLastError();
}

hipError_t launch_chunk_dense(const CacheGeom& g, const void* K, const void* V, int64_t T0, int64_t T1,
                              int64_t p_lo, int64_t p_hi, hipStream_t stream) {
  if (p_hi <= p_lo) return hipSuccess;
  const dim3 grid((unsigned)(p_hi - p_lo), g.Hkv, g.B);
  if (dense_dtype(g.dtype) == PKV_BF16)
    hipLaunchKernelGGL(chunk_dense_kernel<uint16_t>, grid, dim3(256), 0, stream, g, (const uint16_t*)K,
                       (const uint16_t*)V, T0, T1, p_lo);
  else
    hipLaunchKernelGGL(chunk_dense_kernel<float>, grid, dim3(256), 0, stream, g, (const float*)K,
                       (const float*)V, T0, T1, p_lo);
  return hipGetLastError();
}

hipError_t launch_table_fill(const CacheGeom& g, int64_t T, int64_t n_fact, hipStream_t stream) {
  const unsigned blocks = (unsigned)((g.max_pages + 255) / 256);
  hipLaunchKernelGGL(table_fill_kernel, dim3(blocks), dim3(256), 0, stream,
                     (int32_t*)(g.base + g.lay.page_table), g.max_pages, T, g.n_s, g.n_w, n_fact, g.P);
  return hipGetLastError();
}

hipError_t launch_table_set(const CacheGeom& g, int64_t page, int32_t entry, hipStream_t stream) {
  hipLaunchKernelGGL(table_set_kernel, dim3(1), dim3(64), 0, stream,
                     (int32_t*)(g.base + g.lay.page_table), page, entry);
  return hipGetLastError();
}

hipError_t launch_append(const CacheGeom& g, const void* k, const void* v, int64_t T,
                         hipStream_t stream) {
  const dim3 grid(g.Hkv, g.B);
  if (dense_dtype(g.dtype) == PKV_BF16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(kD), 0, stream, g, (const uint16_t*)k,
                       (const uint16_t*)v, T);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(kD), 0, stream, g, (const float*)k,
                       (const float*)v, T);
  return hipGetLastError();
}

}  // namespace pkv
