// Mixed dense / factorized decode attention on gfx950.
//
// PuzzleKV Sec. 3.3 (4), Eq. 4 and Eq. 5: every page of the hybrid cache --
// dense sink and window pages, and factorized history pages -- yields the
// online-softmax state (m_p, l_p, o_p); factorized pages are evaluated through
// their factors, contracting the query with the small factors first
//     s = (q Rf_K^T) Lf_K^T / sqrt(d),   o = (e^(s - m) Lf_V) Rf_V,
// so no page is ever reconstructed.  States are merged by the FlashAttention
// reduction (Eq. 5): within a wavefront as pages stream by, across the
// wavefronts of a workgroup in LDS, and across workgroups (splits) in a small
// second kernel (the kernel boundary orders the partial states across the
// 8 XCDs, which an in-kernel device-scope fence per workgroup did at a far
// higher cost).
//
// bf16 path (decode_mfma_kernel): one wavefront owns a contiguous run of pages
// of one (sequence, KV head) and all G <= 8 query heads of that KV head.  All
// four contractions run on v_mfma_f32_16x16x32_bf16.  The 16 MFMA columns
// hold the G query heads twice: columns 0..7 carry the bf16-rounded operand
// (q, t, p or u) and columns 8..15 its bf16 remainder, so the fp32 operand
// enters with ~16 significant bits while the stored bf16 factors are used
// exactly; the two column halves are summed with one row rotation (DPP).
// Scores are kept in log2 units (q is pre-scaled by log2(e)/sqrt(d)).
//
// fp32 path and shapes the matrix-core kernel does not cover
// (decode_valu_kernel): plain fp32 VALU arithmetic, one workgroup per split.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const void* q;
  const uint8_t* fac;
  const void* sink_k;
  const void* sink_v;
  const void* win_k;
  const void* win_v;
  const int32_t* table;
  float* ws_o;
  float* ws_ml;
  int B, Hkv, G, n_split;
  int P;                        // page length (the matrix-core formats fix theirs: kPageRows)
  int n_s, n_w;
  int r_k, r_v;
  int64_t T, n_fact, F_max;
  int64_t page_bytes, k_part_bytes;
  int64_t cost_dense, cost_fact;
  float qscale;
  int rope;                     // pre-RoPE keys: rotate each key at its position
  float rope_freq[kD / 2];
};

// Work list of one (sequence, KV head): D dense pages (sink pages first, then
// the window / partial pages), then F factorized pages.  Unit e maps to the
// logical page below; waves take contiguous cost-balanced ranges of units.
struct WorkList {
  int64_t n_sinkp, first_tail, D, F;
};

__device__ inline WorkList work_list(int64_t T, int64_t n_fact, int n_s, int P = kP) {
  WorkList w;
  const int64_t n_pages = (T + P - 1) / P;
  w.n_sinkp = n_pages < n_s ? n_pages : n_s;
  w.first_tail = n_s + n_fact;
  const int64_t tail = n_pages - w.first_tail;
  w.D = w.n_sinkp + (tail > 0 ? tail : 0);
  w.F = n_fact;
  return w;
}

// One cache of a batched launch (pkv_decode_attn_batch): its pools, table,
// length and factor count; its pools hold one sequence.
struct BatchSeq {
  const uint8_t* fac;
  const void* sink_k;
  const void* sink_v;
  const void* win_k;
  const void* win_v;
  const int32_t* table;
  int64_t T, n_fact, F_max;
  int split_base;  // first grid column of this cache's splits
  int n_split;     // its splits (the workspace rows keep the batch's stride)
};

// A batched launch's grid is compact: column x belongs to the cache whose
// splits [split_base, split_base + n_split) contain it.
struct DecodeBatchArgs {
  DecodeArgs a;  // what the caches share (their per-cache fields unused)
  int n_seq;
  BatchSeq seq[kMaxBatchCaches];
};

// What a workgroup attends over: sequence b of a cache's pools, or (batched
// launch) cache b of the batch, whose pools hold sequence 0.
struct SeqView {
  const uint8_t* fac;
  const void* sink_k;
  const void* sink_v;
  const void* win_k;
  const void* win_v;
  const int32_t* table;
  int64_t T, n_fact, F_max;
  int b_pool;
  int n_split;  // splits sharing this range
  int b;        // sequence row of q, the workspace and out
  int split;    // this workgroup's split
};

__device__ inline const DecodeArgs& common_args(const DecodeArgs& a) { return a; }
__device__ inline const DecodeArgs& common_args(const DecodeBatchArgs& x) { return x.a; }

__device__ inline SeqView seq_view(const DecodeArgs& a) {
  const int b = blockIdx.z;
  return SeqView{a.fac, a.sink_k, a.sink_v, a.win_k, a.win_v, a.table, a.T, a.n_fact, a.F_max,
                 b, a.n_split, b, (int)blockIdx.x};
}
__device__ inline SeqView seq_view(const DecodeBatchArgs& x) {
  const int col = blockIdx.x;
  int i = 0;
  while (i + 1 < x.n_seq && col >= x.seq[i + 1].split_base) ++i;  // uniform, <= 32 steps
  const BatchSeq& s = x.seq[i];
  return SeqView{s.fac, s.sink_k, s.sink_v, s.win_k, s.win_v, s.table, s.T, s.n_fact, s.F_max,
                 0, s.n_split, i, col - s.split_base};
}

__device__ inline int64_t unit_bound(const WorkList& w, const DecodeArgs& a, int64_t wi,
                                     int64_t W) {
  const int64_t total = w.D * a.cost_dense + w.F * a.cost_fact;
  const int64_t x = total * wi / W;
  const int64_t dc = w.D * a.cost_dense;
  if (x <= dc) return (x + a.cost_dense - 1) / a.cost_dense;
  return w.D + (x - dc + a.cost_fact - 1) / a.cost_fact;
}

__device__ inline int64_t unit_page(const WorkList& w, const DecodeArgs& a, int64_t e) {
  if (e < w.n_sinkp) return e;
  if (e < w.D) return w.first_tail + (e - w.n_sinkp);
  return a.n_s + (e - w.D);
}

__device__ inline float ror8(float x) {
  // lane n of each 16-lane row receives lane (n + 8) mod 16
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, true));
}

// bf16 part of x on lanes whose column is < 8, bf16 remainder on the others:
// rem_lane is 0 or 1 per lane; x - bf16(x) is exact (Sterbenz), so one FMA
// and one rounding give either part without computing both.
__device__ inline __bf16 split_bf16(float x, float rem_lane) {
  const float h = (float)(__bf16)x;
  return (__bf16)__builtin_fmaf(-rem_lane, h, x);
}

// 2^x on the transcendental unit (v_exp_f32); results below 2^-126 flush to
// zero, which is harmless for softmax weights.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3), aligned(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2), aligned(4)));

// Streaming loads: factor and dense pages are read once per decode step, so
// they are fetched non-temporally (measured ~13% more read bandwidth on
// gfx950 than cached loads for this access pattern).
__device__ inline bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)p));
}


// W (even, <= 8) consecutive bf16 kept at their exact width in registers.
template <int W>
struct RawW {
  uint32_t d[W / 2];
};

template <int W>
__device__ inline void ldraw(RawW<W>& r, const uint16_t* p) {
  if constexpr (W == 8) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    r.d[0] = v.x;
    r.d[1] = v.y;
    r.d[2] = v.z;
    r.d[3] = v.w;
  } else if constexpr (W == 6) {
    const u32x3 v = __builtin_nontemporal_load((const u32x3*)p);
    r.d[0] = v.x;
    r.d[1] = v.y;
    r.d[2] = v.z;
  } else if constexpr (W == 4) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    r.d[0] = v.x;
    r.d[1] = v.y;
  } else {
    r.d[0] = __builtin_nontemporal_load((const uint32_t*)p);
  }
}

// slots 0..W-1 from r, zeros above
template <int W>
__device__ inline bf16x8 operand(const RawW<W>& r) {
  uint4 u = {0u, 0u, 0u, 0u};
  u.x = r.d[0];
  if constexpr (W >= 4) u.y = r.d[1];
  if constexpr (W >= 6) u.z = r.d[2];
  if constexpr (W >= 8) u.w = r.d[3];
  return __builtin_bit_cast(bf16x8, u);
}

template <int N8>
struct FactDims {
  static constexpr int A = 2 * N8;
  static constexpr int RT = (A + 3) / 4;
  static constexpr int KS2 = (A + 7) / 8;
  static constexpr bool kPartialTile = (A % 4) != 0;
  static constexpr int64_t K1 = 1024 * N8;
  static constexpr int64_t V1 = 512 * N8;
  static constexpr int width(int ks) { return (A - 8 * ks) < 8 ? (A - 8 * ks) : 8; }
  static constexpr int W0 = width(0);
  static constexpr int W1 = KS2 > 1 ? width(1) : 2;
};

// K part / V part of one factorized page in matrix-core operand order.
template <int N8>
struct KRegs {
  using Dm = FactDims<N8>;
  bf16x8 k1[Dm::RT][4];
  RawW<Dm::W0> k2a[4];
  RawW<Dm::W1> k2b[Dm::KS2 > 1 ? 4 : 1];
  __device__ bf16x8 k2(int mt, int ks) const { return ks == 0 ? operand(k2a[mt]) : operand(k2b[mt]); }
};

template <int N8>
struct VRegs {
  using Dm = FactDims<N8>;
  bf16x8 v1[Dm::RT][2];
  RawW<Dm::W0> v2a[8];
  RawW<Dm::W1> v2b[Dm::KS2 > 1 ? 8 : 1];
  __device__ bf16x8 v2(int mt, int ks) const { return ks == 0 ? operand(v2a[mt]) : operand(v2b[mt]); }
};

// Rank tiles (K1, V1): the last tile of an odd N8 is stored compacted; lanes
// whose row is not stored read a valid address and are zeroed.
struct TileLane {
  int lam;
  bool ok;
};

__device__ inline TileLane tile_lane(int lane) {
  const int rho = lane & 15, qk = lane >> 4;
  TileLane t;
  t.ok = (rho & 3) < 2;
  t.lam = t.ok ? qk * 8 + (rho >> 2) * 2 + (rho & 3) : 0;
  return t;
}

template <int N8>
__device__ inline void load_keys(KRegs<N8>& R, const uint16_t* kp, int lane) {
  using Dm = FactDims<N8>;
  const TileLane tl = tile_lane(lane);
#pragma unroll
  for (int mt = 0; mt < Dm::RT; ++mt) {
    const bool part = Dm::kPartialTile && (mt == Dm::RT - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (!part) {
        R.k1[mt][ks] = ld16(kp + mt * 2048 + ks * 512 + lane * 8);
      } else {
        const bf16x8 v = ld16(kp + mt * 2048 + ks * 256 + tl.lam * 8);
        R.k1[mt][ks] = tl.ok ? v : bf16x8{};
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* base = kp + Dm::K1 + mt * 64 * Dm::A;
    ldraw(R.k2a[mt], base + lane * Dm::W0);
    if constexpr (Dm::KS2 > 1) ldraw(R.k2b[mt], base + 512 + lane * Dm::W1);
  }
}

// A lane's V2 operand in a value part stored at its exact rank (r8 <= 32):
// element offset within a channel tile and the tile's elements (16 r2).  A
// lane loads its quad's A slots from there.  Slots past its own ranks (the
// partial quad's last A - ap, every slot of a quad beyond it) read other
// lanes' values of the same tile.  They meet the u entries of ranks >= r2,
// which are exactly zero: Lf_V^T stores zero rows for ranks >= r.
struct V2Lane {
  int off, tile;
};

__device__ inline V2Lane v2_lane(int r, int A, int lane) {
  const int r2 = r + (r & 1), nf = r2 / A, ap = r2 % A;
  const int rho = lane & 15, qk = lane >> 4;
  V2Lane v;
  v.tile = 16 * r2;
  if (qk < nf) v.off = 16 * ap + (16 * qk + rho) * A;
  else if (qk == nf && ap > 0) v.off = rho * ap;  // the partial quad: ap of its A slots
  else v.off = 0;                                  // no ranks
  return v;
}

// V2 of a value part in the exact-rank order, through the lane's V2Lane (v2
// points at the operand).
template <int N8, bool EV>
__device__ inline void load_v2(VRegs<N8>& R, const uint16_t* v2, int, const V2Lane& vl) {
  using Dm = FactDims<N8>;
  static_assert(EV && Dm::KS2 == 1, "exact-rank V2 up to r8 = 32");
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) ldraw(R.v2a[mt], v2 + mt * vl.tile + vl.off);
}

template <int N8>
__device__ inline void load_values(VRegs<N8>& R, const uint16_t* vp, int lane) {
  using Dm = FactDims<N8>;
  const TileLane tl = tile_lane(lane);
#pragma unroll
  for (int mt = 0; mt < Dm::RT; ++mt) {
    const bool part = Dm::kPartialTile && (mt == Dm::RT - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (!part) {
        R.v1[mt][ks] = ld16(vp + mt * 1024 + ks * 512 + lane * 8);
      } else {
        const bf16x8 v = ld16(vp + mt * 1024 + ks * 256 + tl.lam * 8);
        R.v1[mt][ks] = tl.ok ? v : bf16x8{};
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const uint16_t* base = vp + Dm::V1 + mt * 64 * Dm::A;
    ldraw(R.v2a[mt], base + lane * Dm::W0);
    if constexpr (Dm::KS2 > 1) ldraw(R.v2b[mt], base + 512 + lane * Dm::W1);
  }
}

// The same from a value part whose V2 holds the exact rank.
template <int N8>
__device__ inline void load_values_ev(VRegs<N8>& R, const uint16_t* vp, int lane, const V2Lane& vl) {
  using Dm = FactDims<N8>;
  const TileLane tl = tile_lane(lane);
#pragma unroll
  for (int mt = 0; mt < Dm::RT; ++mt) {
    const bool part = Dm::kPartialTile && (mt == Dm::RT - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (!part) {
        R.v1[mt][ks] = ld16(vp + mt * 1024 + ks * 512 + lane * 8);
      } else {
        const bf16x8 v = ld16(vp + mt * 1024 + ks * 256 + tl.lam * 8);
        R.v1[mt][ks] = tl.ok ? v : bf16x8{};
      }
    }
  }
  load_v2<N8, true>(R, vp + Dm::V1, lane, vl);
}

struct SoftState {
  float m, l;
  floatx4 o[8];
};

// Fold one page's 16 NT raw scores per query (NT score tiles of MFMA output,
// hi/lo column halves not yet summed) into the running state; s receives the
// page's probabilities e^(score - m) (slot [ks][e] of the value contraction in
// s[2 ks + e / 4][e % 4]).
template <int NT = 4>
__device__ inline void softmax_probs(SoftState& st, const floatx4 (&acc)[NT], int nvalid, int q4,
                                     float (&s)[NT][4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x = acc[mt][v] + ror8(acc[mt][v]);
      const int j = 16 * q4 + 4 * mt + v;
      x = j < nvalid ? x : -INFINITY;
      s[mt][v] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float alpha = fast_exp2(st.m - m_new);
  float ps = 0.f;
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float p = fast_exp2(s[mt][v] - m_new);
      s[mt][v] = p;
      ps += p;
    }
  }
  ps += __shfl_xor(ps, 16);
  ps += __shfl_xor(ps, 32);
  st.l = st.l * alpha + ps;
  st.m = m_new;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) st.o[mt] *= alpha;
}

// ... and the probability operand pb[NT / 2] of the value contraction.
template <int NT = 4>
__device__ inline void softmax_page(SoftState& st, const floatx4 (&acc)[NT], int nvalid, int q4,
                                    float rem, bf16x8 (&pb)[NT / 2]) {
  float s[NT][4];
  softmax_probs<NT>(st, acc, nvalid, q4, s);
#pragma unroll
  for (int ks = 0; ks < NT / 2; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[ks][e] = split_bf16(s[2 * ks + e / 4][e % 4], rem);
  }
}

// Online softmax of one full page with a lazily raised reference maximum:
// st.m moves only when a score exceeds it by more than 2^kSlack (in log2
// units), so the running output is rescaled only then (the result is the
// same; weights up to 2^kSlack are exact in fp32).  Leaves 256 e^(s - m) in
// p (the factor folds a power of two of the value contraction) and adds
// sum e^(s - m) to st.l.
constexpr float kSlack = 8.f;

// x combined with lane l ^ 16 / l ^ 32 of each lane l: gfx950
// v_permlane16_swap / v_permlane32_swap with both operands x return the pair
// {x[l], x[l ^ 16]} (resp. l ^ 32) in every lane -- a VALU exchange instead
// of an LDS round trip.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (nvalid < 64: the scores of page rows from nvalid on are masked; NT score
// tiles)
template <int NT = 4>
__device__ inline void softmax_probs_lazy(SoftState& st, const floatx4 (&acc)[NT], int q4, float (&p)[NT][4],
                                          int nvalid = kP) {
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[mt][v] = acc[mt][v] + ror8(acc[mt][v]);
      if (nvalid < kP && 16 * q4 + 4 * mt + v >= nvalid) p[mt][v] = -INFINITY;
      mx = fmaxf(mx, p[mt][v]);
    }
  }
  mx = max_xor32(max_xor16(mx));
  if (__any(mx > st.m + kSlack)) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) st.o[mt] *= alpha;
    st.m = m_new;
  }
  const float mref = st.m - 8.f;  // 256 e^(s - m) = 2^(s - (m - 8))
  float ps = 0.f;
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[mt][v] = fast_exp2(p[mt][v] - mref);
      ps += p[mt][v];
    }
  }
  ps = sum_xor32(sum_xor16(ps));
  st.l = __builtin_fmaf(ps, 1.f / 256.f, st.l);
}

// hi/lo-combined rank vector of rank tiles -> B operand slots.
template <int N8>
__device__ inline void rank_operand(const floatx4 (&acc)[FactDims<N8>::RT], float rem,
                                    bf16x8 (&out)[FactDims<N8>::KS2]) {
  using Dm = FactDims<N8>;
#pragma unroll
  for (int ks = 0; ks < Dm::KS2; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int mt = 2 * ks + e / 4;
      float x = 0.f;
      if (mt < Dm::RT) x = acc[mt][e % 4] + ror8(acc[mt][e % 4]);
      out[ks][e] = split_bf16(x, rem);
    }
  }
}

// Eq. 4, key half: t = Rf_K q, s = Lf_K t, online-softmax update; returns
// the probability operand.
template <int N8>
__device__ inline void fact_keys(SoftState& st, const KRegs<N8>& R, const bf16x8 (&qb)[4], int q4,
                                 float rem, bf16x8 (&pb)[2], int nvalid = kP) {
  using Dm = FactDims<N8>;
  floatx4 at[Dm::RT];
#pragma unroll
  for (int mt = 0; mt < Dm::RT; ++mt) {
    at[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) at[mt] = mfma(R.k1[mt][ks], qb[ks], at[mt]);
  }
  bf16x8 tb[Dm::KS2];
  rank_operand<N8>(at, rem, tb);
  floatx4 as_[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    as_[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Dm::KS2; ++ks) as_[mt] = mfma(R.k2(mt, ks), tb[ks], as_[mt]);
  }
  softmax_page(st, as_, nvalid, q4, rem, pb);
}

// Eq. 4, value half: u = Lf_V^T p, o += Rf_V^T u.
template <int N8>
__device__ inline void fact_values(SoftState& st, const VRegs<N8>& R, const bf16x8 (&pb)[2],
                                   float rem) {
  using Dm = FactDims<N8>;
  floatx4 au[Dm::RT];
#pragma unroll
  for (int mt = 0; mt < Dm::RT; ++mt) {
    au[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) au[mt] = mfma(R.v1[mt][ks], pb[ks], au[mt]);
  }
  bf16x8 ub[Dm::KS2];
  rank_operand<N8>(au, rem, ub);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int ks = 0; ks < Dm::KS2; ++ks) st.o[mt] = mfma(R.v2(mt, ks), ub[ks], st.o[mt]);
  }
}

// A dense page of kRows <= 64 rows ([kRows][d] keys, [d][kRows] values) in
// the 64-row frame: the operands of rows from kRows on are zero.
template <int kRows = kP>
__device__ inline void dense_page(SoftState& st, const uint16_t* Kp, const uint16_t* Vt, int nvalid,
                                  const bf16x8 (&qb)[4], int lane, float rem) {
  const int n = lane & 15, q4 = lane >> 4;
  // score tile rows follow the page-row order of the factor path
  floatx4 as_[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int j = 16 * (n >> 2) + 4 * mt + (n & 3);
    const bool ok = kRows == kP || j < kRows;
    as_[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 k = ok ? ld16(Kp + j * kD + 32 * ks + 8 * q4) : bf16x8{};
      as_[mt] = mfma(k, qb[ks], as_[mt]);
    }
  }
  bf16x8 pb[2];
  softmax_page(st, as_, nvalid, q4, rem, pb);
  const bool vok = kRows == kP || 16 * q4 < kRows;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 v = vok ? ld16(Vt + (16 * mt + n) * kRows + 16 * q4 + 8 * ks) : bf16x8{};
      st.o[mt] = mfma(v, pb[ks], st.o[mt]);
    }
  }
}

constexpr int kWaves = 4;  // waves per workgroup of the matrix-core kernel

// Waves per SIMD the matrix-core kernel is compiled for (register budget):
// 2 up to r = 48, 1 above.  Three waves of the small ranks without key double
// buffering streamed less (Llama-shaped layer, r = 16: 4.7 TB/s at 3 waves,
// 6.45 TB/s at 2 waves with double-buffered keys).
constexpr int mfma_waves_per_simd(int n8) { return n8 <= 6 ? 2 : 1; }

// Factor formats of the matrix-core kernel.  A format supplies the register
// image of a page's K part and V part (KRegs, VRegs) and their loads, the
// per-wave query operand (Query, built from the fp32 query q log2(e)/sqrt(d)
// of the lane's 32 channels or its bf16 hi/lo operand), and the two halves of Eq. 4 on a page:
// keys() leaves the page's probabilities in Probs, values() accumulates the
// page's output.

// bf16 factors Lf = U Sigma, Rf = W^T (Sec. 3.3, Eq. 2), key rank 8 N8K and
// value rank 8 N8V (each part in its own rank's operand order).
// EV: the value part's V2 at its exact rank (r_V not a multiple of 8).
template <int N8K, int N8V = N8K, bool EV = false>
struct Bf16Factors {
  static constexpr bool kExactV = EV;
  static constexpr int kAV = 2 * N8V;  // value ranks per lane quad
  static constexpr int kN8Max = N8K > N8V ? N8K : N8V;
  static constexpr int kWavesPerSimd = mfma_waves_per_simd(kN8Max);
  // Key parts double-buffered where the extra page half fits the budget
  // without spilling (all but r/8 = 5, 6).  Qwen3-32B-shaped layer (r = 24):
  // 51.8 -> 50.7 us.
  static constexpr bool kKeyDoubleBuffer = kN8Max <= 4 || kN8Max >= 7;
  static constexpr bool kLdsRing = false;
  static constexpr bool kRope = false;
  static constexpr int kLdsBytes = 0;
  static constexpr int kPageRows = kP;
  using K = KRegs<N8K>;
  using V = VRegs<N8V>;
  struct Query {
    bf16x8 qb[4];
  };
  using Probs = bf16x8[2];
  __device__ static void query(Query& Q, const float (&)[4][8], const bf16x8 (&qb)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Q.qb[ks] = qb[ks];
  }
  // the dense pages' query operand
  __device__ static void dense_query(bf16x8 (&qd)[4], const Query& Q, float) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qd[ks] = Q.qb[ks];
  }
  __device__ static void load_keys(K& R, const uint8_t* kp, int lane) {
    pkv::load_keys<N8K>(R, (const uint16_t*)kp, lane);
  }
  __device__ static void load_values(V& R, const uint8_t* vp, int lane) {
    pkv::load_values<N8V>(R, (const uint16_t*)vp, lane);
  }
  __device__ static void load_values(V& R, const uint8_t* vp, int lane, const V2Lane& vl) {
    pkv::load_values_ev<N8V>(R, (const uint16_t*)vp, lane, vl);
  }
  __device__ static void keys(SoftState& st, const K& R, const Query& Q, int q4, float rem, Probs& pb) {
    fact_keys<N8K>(st, R, Q.qb, q4, rem, pb);
  }
  __device__ static void values(SoftState& st, const V& R, const Probs& pb, int q4, float rem) {
    fact_values<N8V>(st, R, pb, rem);
  }
};

// bf16 factors of 32-token pages (the page length of Sec. 4.1), ranks
// 8 N8K, 8 N8V <= 32, in the two-tile compact token order of
// RopeFactors<N8, 32>: score row 4 b + v of tile t is token 8 b + 4 t + v,
// slot e of lane quad b of the value contraction's one reduction step is
// token 8 b + e.  Each lane loads its tokens' K2 rows and V1 columns from
// the stored compacted 64-row layout.
template <int N8K, int N8V = N8K, bool EV = false>
struct Bf16Half : Bf16Factors<N8K, N8V, EV> {
  static_assert(N8K <= 4 && N8V <= 4, "ranks up to the page length");
  static constexpr int kPageRows = kMinP;
  using Base = Bf16Factors<N8K, N8V, EV>;
  using typename Base::Query;
  using typename Base::Probs;
  using DK = FactDims<N8K>;
  using DV = FactDims<N8V>;
  struct K {
    bf16x8 k1[DK::RT][4];
    RawW<DK::W0> k2a[2];
  };
  struct V {
    bf16x8 v1[DV::RT];
    RawW<DV::W0> v2a[8];
  };
  __device__ static void load_keys(K& R, const uint8_t* kp, int lane) {
    const uint16_t* p = (const uint16_t*)kp;
    const TileLane tl = tile_lane(lane);
#pragma unroll
    for (int mt = 0; mt < DK::RT; ++mt) {
      const bool part = DK::kPartialTile && mt == DK::RT - 1;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (!part) {
          R.k1[mt][ks] = ld16(p + mt * 2048 + ks * 512 + lane * 8);
        } else {
          const bf16x8 v = ld16(p + mt * 2048 + ks * 256 + tl.lam * 8);
          R.k1[mt][ks] = tl.ok ? v : bf16x8{};
        }
      }
    }
    // row rho of tile t: token 8 (rho / 4) + 4 t + rho % 4, stored as page
    // row 16 bq + 4 mt + v of the compacted K2 at lane 8 qk + 4 bq + v
    const int rho = lane & 15, qk = lane >> 4;
    const int lam = 8 * qk + 4 * (rho >> 3) + (rho & 3);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      ldraw(R.k2a[t], p + DK::K1 + ((2 * (rho >> 2) + t) & 3) * 32 * DK::A + lam * DK::W0);
  }
  // tokens 8 b .. 8 b + 7 of lane quad b: stored lane 16 (b / 2) + rho, step b % 2
  __device__ static void load_v1(V& R, const uint16_t* p, int lane) {
    const int rho = lane & 15, b = lane >> 4;
    const TileLane tl = tile_lane(lane);
#pragma unroll
    for (int mt = 0; mt < DV::RT; ++mt) {
      const bool part = DV::kPartialTile && mt == DV::RT - 1;
      if (!part) {
        R.v1[mt] = ld16(p + mt * 512 + (b & 1) * 256 + (16 * (b >> 1) + rho) * 8);
      } else {
        const int lam = tl.ok ? 8 * (b >> 1) + 2 * (rho >> 2) + (rho & 3) : 0;
        const bf16x8 v = ld16(p + mt * 512 + (b & 1) * 128 + lam * 8);
        R.v1[mt] = tl.ok ? v : bf16x8{};
      }
    }
  }
  __device__ static void load_values(V& R, const uint8_t* vp, int lane) {
    const uint16_t* p = (const uint16_t*)vp;
    load_v1(R, p, lane);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ldraw(R.v2a[mt], p + DV::V1 / 2 + mt * 64 * DV::A + lane * DV::W0);
  }
  __device__ static void load_values(V& R, const uint8_t* vp, int lane, const V2Lane& vl) {
    const uint16_t* p = (const uint16_t*)vp;
    load_v1(R, p, lane);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ldraw(R.v2a[mt], p + DV::V1 / 2 + mt * vl.tile + vl.off);
  }
  // Eq. 4, key half: t = Rf_K q, s = Lf_K t over the two tiles, online softmax
  __device__ static void keys(SoftState& st, const K& R, const Query& Q, int q4, float rem, Probs& pb) {
    floatx4 at[DK::RT];
#pragma unroll
    for (int mt = 0; mt < DK::RT; ++mt) {
      at[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) at[mt] = mfma(R.k1[mt][ks], Q.qb[ks], at[mt]);
    }
    bf16x8 tb[DK::KS2];
    rank_operand<N8K>(at, rem, tb);
    floatx4 as_[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) as_[t] = mfma(operand(R.k2a[t]), tb[0], floatx4{0.f, 0.f, 0.f, 0.f});
    bf16x8 p1[1];
    softmax_page<2>(st, as_, kP, q4, rem, p1);  // (every token of a factorized page is valid)
    pb[0] = p1[0];
  }
  // Eq. 4, value half: u = Lf_V^T p in one reduction step, o += Rf_V^T u
  __device__ static void values(SoftState& st, const V& R, const Probs& pb, int, float rem) {
    floatx4 au[DV::RT];
#pragma unroll
    for (int mt = 0; mt < DV::RT; ++mt) au[mt] = mfma(R.v1[mt], pb[0], floatx4{0.f, 0.f, 0.f, 0.f});
    bf16x8 ub[DV::KS2];
    rank_operand<N8V>(au, rem, ub);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) st.o[mt] = mfma(operand(R.v2a[mt]), ub[0], st.o[mt]);
  }
};

// ---------------------------------------------------------------------------
// Pre-RoPE keys (App. D.3): the key of token t enters its score rotated by the
// rotary embedding at position t, channel pair (m, m + 64) turning by the
// angle t theta_m.  A page starting at position p0 is scored as
//   s_j = (R(p0)^T q) . (R(j) k_j),
// so the query turns back by the page start once per page, and each key by
// its offset j < 64 in the page, whose cos / sin the workgroup tabulates in
// LDS at start.  Keys of factorized pages are reconstructed on the matrix
// cores 16 tokens at a time (K_p^T = Rf_K^T Lf_K^T, with Rf_K stored
// channel-major for it), rotated in fp32 and scored on the fp16 matrix cores
// against the hi/lo query operand; dense pages take the same route from their
// stored rows.  The rotated keys are rounded to fp16 (11-bit significand;
// bf16's 8 bits cost up to ~9e-3 of the output on keys with outlier
// channels) after a 2^-8 scaling folded into the cos / sin table, which keeps
// keys up to ~1.6e7 in range; the query carries the 2^8.
//
// Channel order: a lane (column n = lane & 15, quad q4 = lane >> 4) holds
// channels 16 ct + 4 q4 + v (ct < 8, v < 4) of one token -- the rows of the
// reconstruction's output tiles -- so that the pair partners (ct, ct + 4)
// share a lane; k-step ks of the score contraction takes tiles 2 ks and
// 2 ks + 1 (element 4 (ct & 1) + v), and the query operand follows suit.

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

constexpr float kRopeKeyScale = 1.f / 256.f;  // folded into the offset table
constexpr float kRopeQueryScale = 256.f;      // and undone on the query

__device__ inline floatx4 mfma_f16(halfx8 a, halfx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 part of x on lanes whose column is < 8, fp16 remainder on the others
__device__ inline _Float16 split_f16(float x, float rem_lane) {
  const float h = (float)(_Float16)x;
  return (_Float16)__builtin_fmaf(-rem_lane, h, x);
}

// cos / sin of pos * theta: the angle is formed and reduced modulo 2 pi in
// double precision (two-part 2 pi), the functions evaluated in float.
__device__ inline void rope_sincos(int64_t pos, float theta, float& c, float& s) {
  const double a = (double)pos * (double)theta;
  const double k = rint(a * 0.15915494309189535);
  double red = fma(-k, 6.283185307179586, a);
  red = fma(-k, 2.4492935982947064e-16, red);
  sincosf((float)red, &s, &c);
}

// cos / sin (j theta_m) for every in-page offset j and frequency m: row j
// holds groups [ct][q4] of {cos v0..3, sin v0..3}, padded by 16 bytes so that
// the 16 rows a lane quad reads fall in different banks; and, per wave,
// cos / sin (p0 theta_m) of its current page.
constexpr int kRopeRow = 8 * kD / 2 / 4 + 4;  // floats per table row
struct RopeLds {
  float table[kP][kRopeRow];
  float base[kWaves][2][kD / 2];
  uint4 q[kWaves][4][64];  // per wave: each lane's unrotated query (bf16 pairs), uint4 w of lane l at [w][l]
};

__device__ inline void rope_table_fill(RopeLds& L, const float* freq) {
  for (int idx = threadIdx.x; idx < kP * (kD / 2); idx += blockDim.x) {
    const int j = idx / (kD / 2), m = idx % (kD / 2);
    float c, s;
    rope_sincos(j, freq[m], c, s);
    float* grp = &L.table[j][((m >> 4) * 4 + ((m >> 2) & 3)) * 8];
    grp[m & 3] = c * kRopeKeyScale;
    grp[4 + (m & 3)] = s * kRopeKeyScale;
  }
}

// The rotated query R(p0)^T q of a page starting at p0, as the hi/lo operand
// (qlds: the lane's channels in the order above, unrotated, as bf16 pairs;
// element e of step ks is half e & 1 of word e / 2 of uint4 ks).  Lane m
// computes cos / sin (p0 theta_m), times the query's scale, into the wave's
// LDS slot; LDS operations of one wave complete in order, so the reads below
// see it.
__device__ inline void rope_page_query(halfx8 (&qb)[4], const uint4 (&qlds)[4][64], int64_t p0,
                                       const float* freq, float qscale, float (&base)[2][kD / 2], int lane,
                                       float rem) {
  const int q4 = lane >> 4;
  float c, s;
  rope_sincos(p0, freq[lane], c, s);
  base[0][lane] = c * qscale;
  base[1][lane] = s * qscale;
  uint32_t qw[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 w = qlds[ks][lane];
    qw[ks][0] = w.x;
    qw[ks][1] = w.y;
    qw[ks][2] = w.z;
    qw[ks][3] = w.w;
  }
  auto elem = [&](int ks, int e) {
    const uint32_t w = qw[ks][e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  };
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int m0 = 16 * (2 * ks + half) + 4 * q4;
      const float4 cb = *(const float4*)&base[0][m0];
      const float4 sb = *(const float4*)&base[1][m0];
      const float cv[4] = {cb.x, cb.y, cb.z, cb.w}, sv[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = 4 * half + v;
        const float x = elem(ks, e), y = elem(ks + 2, e);
        qb[ks][e] = split_f16(__builtin_fmaf(y, sv[v], x * cv[v]), rem);
        qb[ks + 2][e] = split_f16(__builtin_fmaf(-x, sv[v], y * cv[v]), rem);
      }
    }
  }
}

// lo[v], hi[v]: fp32 key channels 16 ct + 4 q4 + v and 64 more (ct < 4) of
// the lane's token, at offset j in its page (row: table row j) -> rotated by
// R(j), scaled by 2^-8, into their fp16 slots of the score contraction's A
// operand (channel tile ct' -> step ct' / 2, elements 4 (ct' & 1) + v).
__device__ inline void rope_key_pair(const floatx4& lo, const floatx4& hi, const float* row, int ct, int q4,
                                     halfx8 (&ka)[4]) {
  const float4 co = *(const float4*)(row + (ct * 4 + q4) * 8);
  const float4 si = *(const float4*)(row + (ct * 4 + q4) * 8 + 4);
  const float cv[4] = {co.x, co.y, co.z, co.w}, sv[4] = {si.x, si.y, si.z, si.w};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float x = lo[v], y = hi[v];
    ka[ct >> 1][4 * (ct & 1) + v] = (_Float16)__builtin_fmaf(-y, sv[v], x * cv[v]);
    ka[(ct >> 1) + 2][4 * (ct & 1) + v] = (_Float16)__builtin_fmaf(x, sv[v], y * cv[v]);
  }
}

// Score tile of a page from the rotated key operand and the hi/lo query.
__device__ inline floatx4 rope_scores(const halfx8 (&ka)[4], const halfx8 (&qb)[4]) {
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = mfma_f16(ka[ks], qb[ks], acc);
  return acc;
}

// A dense page of pre-RoPE keys: rows loaded in the rotation's channel
// order, rotated by their offsets; values as in dense_page.
// (kRows = 32: the operands of rows 32..63 are zero, as in dense_page)
template <int kRows = kP>
__device__ inline void dense_page_rope(SoftState& st, const uint16_t* Kp, const uint16_t* Vt, int nvalid,
                                       const halfx8 (&qb)[4], const RopeLds& L, int lane, float rem) {
  const int n = lane & 15, q4 = lane >> 4;
  floatx4 as_[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int j = 16 * (n >> 2) + 4 * mt + (n & 3);
    const bool ok = kRows == kP || j < kRows;
    auto ld4 = [&](int ct) {
      const u32x2 w = ok ? __builtin_nontemporal_load((const u32x2*)(Kp + j * kD + 16 * ct + 4 * q4))
                         : u32x2{0u, 0u};
      return floatx4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    };
    halfx8 ka[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) rope_key_pair(ld4(ct), ld4(ct + 4), &L.table[j][0], ct, q4, ka);
    as_[mt] = rope_scores(ka, qb);
  }
  bf16x8 pb[2];
  softmax_page(st, as_, nvalid, q4, rem, pb);
  const bool vok = kRows == kP || 16 * q4 < kRows;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 v = vok ? ld16(Vt + (16 * mt + n) * kRows + 16 * q4 + 8 * ks) : bf16x8{};
      st.o[mt] = mfma(v, pb[ks], st.o[mt]);
    }
  }
}

// The matrix-core pre-RoPE path takes equal padded ranks up to 64 at
// 64-token pages (one wave per SIMD above r = 32) and, at one reduction step
// per channel tile (r <= 32), every rank pair at either page length; other
// pre-RoPE caches take the VALU kernel.
constexpr int kRopeOneStepMaxN8 = 4;
constexpr int rope_waves_per_simd(int n8) { return n8 <= 4 ? mfma_waves_per_simd(n8) : 1; }

// bf16 factors of pre-RoPE keys: the key part holds Rf_K channel-major (the
// V part's Rf layout) and Lf_K as in Bf16Factors; the V part as there.
// PR: page rows.  A 32-token page is reconstructed, rotated and scored as
// two 16-token tiles in a compact token order: tile t, column n holds token
// 8 (n / 4) + 4 t + n % 4, so score row 4 b + v of tile t is token
// 8 b + 4 t + v, and slot e of lane quad b of the value contraction's single
// reduction step is token 8 b + e (eight consecutive tokens of the stored
// Lf_V^T).  Only the loads follow this order; the stored parts are the
// compacted 64-row layout.  N8 and N8V: the key and value parts' padded
// ranks over 8 (they may differ: r_K and r_V are separate budgets).
template <int N8, int PR = kP, bool EV = false, int N8V = N8>
struct RopeFactors {
  using Dm = FactDims<N8>;    // key parts
  using DmV = FactDims<N8V>;  // value parts
  static constexpr bool kExactV = EV;
  static constexpr int kAV = 2 * N8V;
  static constexpr int kWavesPerSimd = rope_waves_per_simd(N8 > N8V ? N8 : N8V);
  static constexpr bool kKeyDoubleBuffer = false;
  static constexpr bool kLdsRing = false;
  static constexpr bool kRope = true;
  static constexpr int kPageRows = PR;
  static constexpr int kLdsBytes = 0;
  static constexpr int kTiles = PR / 16;  // token tiles
  struct K {
    RawW<Dm::W0> rfa[8];
    RawW<Dm::W1> rfb[Dm::KS2 > 1 ? 8 : 1];
    RawW<Dm::W0> k2a[kTiles];
    RawW<Dm::W1> k2b[Dm::KS2 > 1 ? kTiles : 1];
    __device__ bf16x8 rf(int ct, int ks) const { return ks == 0 ? operand(rfa[ct]) : operand(rfb[ct]); }
    __device__ bf16x8 k2(int mt, int ks) const { return ks == 0 ? operand(k2a[mt]) : operand(k2b[mt]); }
  };
  using V = VRegs<N8V>;
  struct Query {
    float qscale;  // 2^8 log2(e)/sqrt(d), applied with the page's rotation
    halfx8 qb[4];  // R(p0)^T q of the current page, scaled, fp16 hi/lo columns
  };
  using Probs = bf16x8[2];
  // element e of step ks <- channel 16 (2 ks + e / 4) + 4 q4 + e % 4
  // the lane's query (element e of step ks <- channel 16 (2 ks + e / 4) +
  // 4 q4 + e % 4) into its LDS slot, read back once per page
  __device__ static void query(Query& Q, RopeLds& L, int wave, const uint16_t* qp, float qscale, bool valid,
                               int lane) {
    const int q4 = lane >> 4;
    Q.qscale = qscale * kRopeQueryScale;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x2 w0 = u32x2{0u, 0u}, w1 = w0;
      if (valid) {
        w0 = *(const u32x2*)(qp + 16 * (2 * ks) + 4 * q4);
        w1 = *(const u32x2*)(qp + 16 * (2 * ks + 1) + 4 * q4);
      }
      L.q[wave][ks][lane] = uint4{w0.x, w0.y, w1.x, w1.y};
    }
  }
  __device__ static void load_keys(K& R, const uint8_t* kp, int lane) {
    const uint16_t* p = (const uint16_t*)kp;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint16_t* base = p + ct * 64 * Dm::A;
      ldraw(R.rfa[ct], base + lane * Dm::W0);
      if constexpr (Dm::KS2 > 1) ldraw(R.rfb[ct], base + 512 + lane * Dm::W1);
    }
    if constexpr (PR == kP) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint16_t* base = p + Dm::K1 + mt * 64 * Dm::A;
        ldraw(R.k2a[mt], base + lane * Dm::W0);
        if constexpr (Dm::KS2 > 1) ldraw(R.k2b[mt], base + 512 + lane * Dm::W1);
      }
    } else {
      // column n of tile t: token tau = 8 (n / 4) + 4 t + n % 4, stored as
      // page row 16 bq + 4 mt + v of the compacted K2 (bq = tau / 16,
      // mt = tau / 4 % 4, v = tau % 4) at lane 8 qk + 4 bq + v
      const int n = lane & 15, qk = lane >> 4;
      const int lam = 8 * qk + 4 * (n >> 3) + (n & 3);
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const uint16_t* base = p + Dm::K1 + ((2 * (n >> 2) + t) & 3) * 32 * Dm::A;
        ldraw(R.k2a[t], base + lam * Dm::W0);
        if constexpr (Dm::KS2 > 1) ldraw(R.k2b[t], base + 256 + lam * Dm::W1);
      }
    }
  }
  // V1 of a 32-token page in the single reduction step: lane (rho, b) takes
  // tokens 8 b .. 8 b + 7, stored at lane 16 (b / 2) + rho, step b % 2 (a
  // compacted last rank tile: rows v < 2 of each lane quad only)
  __device__ static void load_v1_half(V& R, const uint16_t* p, int lane) {
    const int rho = lane & 15, b = lane >> 4;
    const TileLane tl = tile_lane(lane);
#pragma unroll
    for (int mt = 0; mt < DmV::RT; ++mt) {
      const bool part = DmV::kPartialTile && mt == DmV::RT - 1;
      if (!part) {
        R.v1[mt][0] = ld16(p + mt * 512 + (b & 1) * 256 + (16 * (b >> 1) + rho) * 8);
      } else {
        const int lam = tl.ok ? 8 * (b >> 1) + 2 * (rho >> 2) + (rho & 3) : 0;
        const bf16x8 v = ld16(p + mt * 512 + (b & 1) * 128 + lam * 8);
        R.v1[mt][0] = tl.ok ? v : bf16x8{};
      }
    }
  }
  __device__ static void load_values(V& R, const uint8_t* vp, int lane) {
    if constexpr (PR == kP) {
      pkv::load_values<N8V>(R, (const uint16_t*)vp, lane);
    } else {
      const uint16_t* p = (const uint16_t*)vp;
      load_v1_half(R, p, lane);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint16_t* base = p + DmV::V1 / 2 + mt * 64 * DmV::A;
        ldraw(R.v2a[mt], base + lane * DmV::W0);
        if constexpr (DmV::KS2 > 1) ldraw(R.v2b[mt], base + 512 + lane * DmV::W1);
      }
    }
  }
  __device__ static void load_values(V& R, const uint8_t* vp, int lane, const V2Lane& vl) {
    if constexpr (PR == kP) {
      pkv::load_values_ev<N8V>(R, (const uint16_t*)vp, lane, vl);
    } else {
      const uint16_t* p = (const uint16_t*)vp;
      load_v1_half(R, p, lane);
      load_v2<N8V, true>(R, p + DmV::V1 / 2, lane, vl);
    }
  }
  // token tile mt: K_p^T columns = its 16 tokens, 8 channel tiles of rows
  __device__ static void keys(SoftState& st, const K& R, const Query& Q, const RopeLds& L, int lane,
                              float rem, Probs& pb) {
    const int n = lane & 15, q4 = lane >> 4;
    floatx4 as_[kTiles];
#pragma unroll
    for (int mt = 0; mt < kTiles; ++mt) {
      const int tok = PR == kP ? 16 * (n >> 2) + 4 * mt + (n & 3) : 8 * (n >> 2) + 4 * mt + (n & 3);
      const float* row = &L.table[tok][0];
      halfx8 ka[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        floatx4 lo = floatx4{0.f, 0.f, 0.f, 0.f}, hi = lo;
#pragma unroll
        for (int ks = 0; ks < Dm::KS2; ++ks) {
          lo = mfma(R.rf(ct, ks), R.k2(mt, ks), lo);
          hi = mfma(R.rf(ct + 4, ks), R.k2(mt, ks), hi);
        }
        rope_key_pair(lo, hi, row, ct, q4, ka);
      }
      as_[mt] = rope_scores(ka, Q.qb);
    }
    if constexpr (PR == kP) {
      softmax_page(st, as_, PR, q4, rem, pb);
    } else {  // every token of a factorized page is valid
      bf16x8 p1[1];
      softmax_page<kTiles>(st, as_, kP, q4, rem, p1);
      pb[0] = p1[0];
    }
  }
  __device__ static void values(SoftState& st, const V& R, const Probs& pb, int, float rem) {
    if constexpr (PR == kP) {
      fact_values<N8V>(st, R, pb, rem);
    } else {  // Eq. 4's value half over the page's 32 tokens: one reduction step
      floatx4 au[DmV::RT];
#pragma unroll
      for (int mt = 0; mt < DmV::RT; ++mt) au[mt] = mfma(R.v1[mt][0], pb[0], floatx4{0.f, 0.f, 0.f, 0.f});
      bf16x8 ub[DmV::KS2];
      rank_operand<N8V>(au, rem, ub);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int ks = 0; ks < DmV::KS2; ++ks) st.o[mt] = mfma(R.v2(mt, ks), ub[ks], st.o[mt]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// INT4 factors (Sec. 4.3): Lt = U Sigma^(1/2), Rt = Sigma^(1/2) W^T as 4-bit
// codes c with bf16 group scales (layout: pkv_internal.h).  A code nibble
// n = c + 8 enters the matrix cores as the exact bf16 value 1 + n/16 =
// 1.5 + c/16 (n in mantissa bits 3..6 of 1.0, two codes per and-or).  One
// extra MFMA per contraction with the constant operand -1.5 starts the
// accumulator and removes the offset, leaving (1/16) sum c b.  The scales
// fold into the fp32 vector operands, and the powers of two into the query
// (x 256) and the softmax exponent (p x 256):
//   16 t = (1/16) Rq_K (sR_K o 256 q)            B operand sR_K o 256 q
//   s    = (1/16) Lq_K (sL_K o 16 t)             B operand sL_K o 16 t
//   16 u = (1/16) Lq_V^T (sL_V o 256 p)          B operand sL_V o 256 p
//   o   += sR_V o (1/16) Rq_V^T (16 u)           B operand 16 u
// each B operand as bf16 hi/lo columns (hi = the truncated top 16 bits).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// element e of a bf16 array held as dwords
template <int E>
__device__ __forceinline__ float bf16_at(const uint32_t* d) {
  return E % 2 ? bf16_hi(d[E / 2]) : bf16_lo(d[E / 2]);
}

// A 32-bit constant materialized in a VGPR: VOP3 forms such as v_and_or_b32
// take no literal operand on gfx950, and an SGPR operand is limited to one.
// (The asm is side-effect free, so the compiler hoists it out of loops.)
template <uint32_t C>
__device__ __forceinline__ uint32_t vgpr_const() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(C));
  return r;
}

// codes 2k, 2k + 1 of a unit (bits 4k.. of each 16-bit half) -> bf16 pair
template <int K>
__device__ __forceinline__ uint32_t q4_pair(uint32_t u) {
  const uint32_t sh = K == 0 ? (u << 3) : (u >> (4 * K - 3));
  return (sh & vgpr_const<0x00780078u>()) | vgpr_const<0x3f803f80u>();
}

// Operand pair (x0, x1) as bf16 hi/lo columns: on hi lanes (rem 0) the top
// 16 bits of x, on lo lanes (rem 1) the top 16 bits of x minus its top 16
// bits (an exact fp32 difference); x0 in the low half.
__device__ __forceinline__ uint32_t split2(float x0, float x1, float rem) {
  const float y0 = __builtin_fmaf(-rem, __uint_as_float(__float_as_uint(x0) & 0xffff0000u), x0);
  const float y1 = __builtin_fmaf(-rem, __uint_as_float(__float_as_uint(x1) & 0xffff0000u), x1);
  return __builtin_amdgcn_perm(__float_as_uint(y1), __float_as_uint(y0), 0x07060302u);
}

// unit of W nibbles in the low 4 W bits of x -> operand slots 0 .. 2 NP - 1
// (slots above are 0; a 6-nibble unit's halves are nibbles 0..2 and 3..5)
template <int W, int NP>
__device__ __forceinline__ bf16x8 q4_operand(uint32_t x) {
  uint32_t u = x;
  if constexpr (W == 6) u = __builtin_amdgcn_ubfe(x, 0, 12) | ((x << 4) & vgpr_const<0x0fff0000u>());
  else if constexpr (W == 4) u = x | (x << 8);
  else if constexpr (W == 2) u = x | (x << 12);
  uint4 w = {q4_pair<0>(u), 0u, 0u, 0u};
  if constexpr (NP > 1) w.y = q4_pair<1>(u);
  if constexpr (NP > 2) w.z = q4_pair<2>(u);
  if constexpr (NP > 3) w.w = q4_pair<3>(u);
  return __builtin_bit_cast(bf16x8, w);
}

// unit m of UB bytes from consecutive dwords (UB = 3: the unit's bytes
// 3 m .. 3 m + 2 in the low 24 bits, the bits above it unspecified)
template <int UB>
__device__ __forceinline__ uint32_t q4_unit(const uint32_t* d, int m) {
  if constexpr (UB == 4) {
    return d[m];
  } else if constexpr (UB == 3) {
    const int i = 3 * m / 4, o = 3 * m % 4;
    if (o == 0) return d[i];
    if (o == 1) return d[i] >> 8;
    return __builtin_amdgcn_alignbyte(d[i + 1], d[i], o);
  } else if constexpr (UB == 2) {
    return __builtin_amdgcn_ubfe(d[m / 2], 16 * (m % 2), 16);
  } else {
    return __builtin_amdgcn_ubfe(d[m / 4], 8 * (m % 4), 8);
  }
}

__device__ __forceinline__ bf16x8 q4_offset_operand() {
  const uint4 w = {0xbfc0bfc0u, 0xbfc0bfc0u, 0xbfc0bfc0u, 0xbfc0bfc0u};  // -1.5
  return __builtin_bit_cast(bf16x8, w);
}

// Direct global -> LDS load of 16 bytes per lane (gfx950
// global_load_lds_dwordx4, non-temporal as the streamed register loads):
// lane l's bytes land at LDS address lds_base + 16 l.  Issued as inline
// assembly, so the compiler neither tracks nor waits for it: the caller
// waits with vm_wait before reading the LDS it fills.  lds_base must be
// wave-uniform.  The load takes its LDS base from M0, which the compiler
// reserves: M0 is saved and restored around it, with one wait state after
// each M0 write (the SALU-write-M0 -> LDS-DMA hazard).
__device__ __forceinline__ void lds_load16(const uint8_t* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt unconstrained), then a compiler
// barrier so that no LDS access moves above it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// N consecutive dwords, streamed
template <int N>
__device__ __forceinline__ void ldw(uint32_t* d, const uint8_t* p) {
  if constexpr (N == 6) {  // 8-byte aligned
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    const u32x2 w = __builtin_nontemporal_load((const u32x2*)(p + 16));
    d[0] = v.x, d[1] = v.y, d[2] = v.z, d[3] = v.w, d[4] = w.x, d[5] = w.y;
  } else if constexpr (N == 4) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    d[0] = v.x, d[1] = v.y, d[2] = v.z, d[3] = v.w;
  } else if constexpr (N == 3) {
    const u32x3 v = __builtin_nontemporal_load((const u32x3*)p);
    d[0] = v.x, d[1] = v.y, d[2] = v.z;
  } else if constexpr (N == 2) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    d[0] = v.x, d[1] = v.y;
  } else {
    d[0] = __builtin_nontemporal_load((const uint32_t*)p);
  }
}

// LDS budget of a four-wave workgroup at two workgroups per CU (160 KB).
constexpr int kWgLdsBytes = 80 * 1024;

// PR page rows.  A 32-token page is scored in two 16-row tiles in the
// compact token order of RopeFactors<N8, 32>: row rho of tile t is token
// 8 (rho / 4) + 4 t + rho % 4, and slot e of lane quad b of the value
// contraction's single reduction step is token 8 b + e.  Each lane reads the
// two K2 units of its rows (adjacent in the stored compacted layout) and the
// V1 dword of its eight tokens; the stored parts are unchanged.
template <int N8K, int N8V, int PR = kP>
struct Int4Factors {
  static constexpr int AK = 2 * N8K, AV = 2 * N8V;  // ranks per lane quad
  static constexpr int RTK = (AK + 3) / 4, RTV = (AV + 3) / 4;
  static constexpr bool kPartK = AK % 4 != 0, kPartV = AV % 4 != 0;
  static constexpr Q4Dims kQK = q4_dims(8 * N8K, PR), kQV = q4_dims(8 * N8V, PR);
  static constexpr int UK = kQK.ub, UV = kQV.ub;  // K2 / V2 unit bytes
  // byte offsets within the parts
  static constexpr int kK2 = kQK.k2, kSRK = kQK.sr_k, kSLK = kQK.sl_k;
  static constexpr int kV2 = kQV.v2, kSLV = kQV.sl_v, kSRV = kQV.sr_v;
  static constexpr int kKBytes = kQK.k_bytes, kPageBytes = kQK.k_bytes + kQV.v_bytes;
  static constexpr int kWavesPerSimd = 2;
  static constexpr bool kKeyDoubleBuffer = false;
  static constexpr bool kRope = false;
  static constexpr bool kExactV = false;  // (INT4 parts: their own layout)
  static constexpr int kAV = 2 * N8V;
  static constexpr int kPageRows = PR;
  static constexpr int kTiles = PR / 16;  // score tiles of a page
  // Factor pages stream through a per-wave ring of kRingSlots page slots in
  // LDS, filled by direct global -> LDS loads kRingSlots - 1 pages ahead of
  // the page being computed (registers cannot hold that much prefetch).
  static constexpr bool kLdsRing = true;
  static constexpr int kRingSlots = (kWgLdsBytes / kWaves) / kPageBytes < 4
                                        ? (kWgLdsBytes / kWaves) / kPageBytes : 4;
  static constexpr int kStageLoads = (kPageBytes + 1023) / 1024;  // 1 KB per wave load
  static constexpr int kLdsBytes = kWaves * kRingSlots * kPageBytes;
  static_assert(kRingSlots >= 2, "an INT4 page pair must fit twice per wave");

  struct K {
    uint32_t k1[RTK][4];                          // Rq_K rank tiles, one dword per reduction step
    uint32_t k2[PR == kP ? UK : (UK + 1) / 2];     // Lq_K units of the page-row tiles
    uint32_t sr[16];                              // sR_K of channels 32 ks + 8 q4 + e: [ks][e] as bf16 pairs
    uint32_t sl[N8K];                             // sL_K of the lane quad's ranks
  };
  struct V {
    uint32_t v1[RTV][kTiles / 2];  // Lq_V^T rank tiles
    uint32_t v2[2 * UV];           // Rq_V^T units of the 8 channel tiles
    uint32_t sl[2 * kTiles];       // sL_V of the lane quad's tokens (16 q4 .. + 15; compact: 8 q4 .. + 7)
    uint32_t sr[16];               // sR_V of channels 16 mt + 4 q4 + v: [mt][v]
  };
  struct Query {
    float qf[4][8];
  };
  using Probs = float[kTiles][4];

  __device__ static void query(Query& Q, const float (&qs)[4][8], const bf16x8 (&)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) Q.qf[ks][e] = 256.f * qs[ks][e];
    }
  }
  // the dense pages' query operand (q log2(e)/sqrt(d) as bf16 + remainder)
  __device__ static void dense_query(bf16x8 (&qd)[4], const Query& Q, float rem) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qd[ks][e] = split_bf16(Q.qf[ks][e] * (1.f / 256.f), rem);
    }
  }

  // Direct global -> LDS copy of one page pair (K part, then V part): load i
  // moves bytes 1024 i + 16 lane .. + 15 of the page to the same offset of
  // the slot.
  __device__ static void stage(uint8_t* slot, const uint8_t* page, int lane) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(slot));  // wave-uniform
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const int off = 1024 * i + 16 * lane;
      if (off < kPageBytes) lds_load16(page + off, base + 1024 * i);
    }
  }

  // Wait until at most `pending` pages of staging loads are in flight.
  __device__ static void wait_staged(int pending) {
    static_assert(kStageLoads * (kRingSlots - 1) < 64, "vmcnt range");
    switch (pending) {
      case 0: vm_wait<0>(); break;
      case 1: vm_wait<kStageLoads>(); break;
      case 2: vm_wait<2 * kStageLoads>(); break;
      default: vm_wait<3 * kStageLoads>(); break;
    }
  }

  __device__ static void load_keys(K& R, const uint8_t* kp, int lane) {
    const TileLane tl = tile_lane(lane);
    const int q4 = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < RTK; ++mt) {
      const bool part = kPartK && mt == RTK - 1;
      ldw<4>(R.k1[mt], kp + mt * 1024 + (part ? tl.lam : lane) * 16);
    }
    if constexpr (PR == kP) {
      ldw<UK>(R.k2, kp + kK2 + lane * 4 * UK);
    } else {
      // rows of tiles 0, 1: tokens 8 (rho / 4) + rho % 4 (+ 4), stored as
      // units m0, m0 + 1 (m0 = 0 or 2) of compacted lane 8 qk + 4 (rho / 8) + rho % 4
      const int rho = lane & 15;
      const int m0 = (2 * (rho >> 2)) & 2;
      const uint8_t* u = kp + kK2 + (8 * q4 + 4 * (rho >> 3) + (rho & 3)) * 4 * UK;
      if constexpr (UK == 1) {
        R.k2[0] = *(const uint32_t*)u >> (8 * m0);
      } else if constexpr (UK == 2) {
        R.k2[0] = *(const uint32_t*)(u + 2 * m0);
      } else if constexpr (UK == 3) {  // 6 bytes from byte 3 m0: two dwords from 2 m0, shifted by m0 bytes
        const uint32_t x0 = *(const uint32_t*)(u + 2 * m0), x1 = *(const uint32_t*)(u + 2 * m0 + 4);
        R.k2[0] = __builtin_amdgcn_alignbyte(x1, x0, m0);
        R.k2[1] = x1 >> (8 * m0);
      } else {
        const u32x2 x = *(const u32x2*)(u + 4 * m0);
        R.k2[0] = x.x;
        R.k2[1] = x.y;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ldw<4>(&R.sr[4 * ks], kp + kSRK + 2 * (32 * ks + 8 * q4));
    ldw<N8K>(R.sl, kp + kSLK + 2 * AK * q4);
  }

  __device__ static void load_values(V& R, const uint8_t* vp, int lane) {
    const TileLane tl = tile_lane(lane);
    const int q4 = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < RTV; ++mt) {
      const bool part = kPartV && mt == RTV - 1;
      if constexpr (PR == kP) {
        ldw<2>(R.v1[mt], vp + mt * 512 + (part ? tl.lam : lane) * 8);
      } else {  // tokens 8 q4 .. + 7: stored lane 16 (q4 / 2) + rho, step q4 % 2
        const int rho = lane & 15;
        const int lam = part ? (tl.ok ? 8 * (q4 >> 1) + 2 * (rho >> 2) + (rho & 3) : 0) : 16 * (q4 >> 1) + rho;
        R.v1[mt][0] = *(const uint32_t*)(vp + mt * 256 + lam * 8 + (q4 & 1) * 4);
      }
    }
    if constexpr (UV == 4) {
      ldw<4>(R.v2, vp + kV2 + lane * 32);
      ldw<4>(R.v2 + 4, vp + kV2 + lane * 32 + 16);
    } else {
      ldw<2 * UV>(R.v2, vp + kV2 + lane * 8 * UV);
    }
    if constexpr (PR == kP) {
      ldw<4>(R.sl, vp + kSLV + 32 * q4);
      ldw<4>(R.sl + 4, vp + kSLV + 32 * q4 + 16);
    } else {
      ldw<4>(R.sl, vp + kSLV + 16 * q4);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) ldw<4>(&R.sr[4 * k], vp + kSRV + 64 * q4 + 16 * k);
  }

  // Eq. 4, key half on the codes: t = Rt_K q, s = Lt_K t, online softmax.
  // Rank slots e >= A of the second contraction are zero: they belong to no
  // rank (rows of the compacted tile that lanes only read as filler).
  // Leaves 256 p in p (see softmax_probs_lazy).
  __device__ static void keys(SoftState& st, const K& R, const Query& Q, int q4, float rem, Probs& p) {
    const bf16x8 off = q4_offset_operand();
    bf16x8 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t d = R.sr[4 * ks + k];
        (&w.x)[k] = split2(Q.qf[ks][2 * k] * bf16_lo(d), Q.qf[ks][2 * k + 1] * bf16_hi(d), rem);
      }
      qb[ks] = __builtin_bit_cast(bf16x8, w);
    }
    floatx4 base = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) base = mfma(off, qb[ks], base);
    floatx4 at[RTK];
#pragma unroll
    for (int mt = 0; mt < RTK; ++mt) {
      at[mt] = base;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) at[mt] = mfma(q4_operand<8, 4>(R.k1[mt][ks]), qb[ks], at[mt]);
    }
    uint4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < N8K; ++k) {  // slots 2k, 2k + 1 < AK
      const uint32_t d = R.sl[k];
      const float t0 = at[k / 2][2 * (k % 2)] + ror8(at[k / 2][2 * (k % 2)]);
      const float t1 = at[k / 2][2 * (k % 2) + 1] + ror8(at[k / 2][2 * (k % 2) + 1]);
      (&w.x)[k] = split2(t0 * bf16_lo(d), t1 * bf16_hi(d), rem);
    }
    const bf16x8 tb = __builtin_bit_cast(bf16x8, w);
    const floatx4 base2 = mfma(off, tb, floatx4{0.f, 0.f, 0.f, 0.f});
    floatx4 as_[kTiles];
#pragma unroll
    for (int mt = 0; mt < kTiles; ++mt)
      as_[mt] = mfma(q4_operand<2 * UK, N8K>(q4_unit<UK>(R.k2, mt)), tb, base2);
    softmax_probs_lazy<kTiles>(st, as_, q4, p);  // (every token of a factorized page is valid)
  }

  // Eq. 4, value half on the codes: u = Lt_V^T p, o += Rt_V^T u.
  __device__ static void values(SoftState& st, const V& R, const Probs& p, int q4, float rem) {
    const bf16x8 off = q4_offset_operand();
    constexpr int KS = kTiles / 2;  // reduction steps over the page's tokens
    bf16x8 pb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // tokens 16 q4 + 8 ks + 2k, + 1 (compact: 8 q4 + 2k, + 1)
        const uint32_t d = R.sl[4 * ks + k];
        const int mt = 2 * ks + k / 2, v = 2 * (k % 2);
        (&w.x)[k] = split2(p[mt][v] * bf16_lo(d), p[mt][v + 1] * bf16_hi(d), rem);
      }
      pb[ks] = __builtin_bit_cast(bf16x8, w);
    }
    floatx4 base = mfma(off, pb[0], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) base = mfma(off, pb[ks], base);
    floatx4 au[RTV];
#pragma unroll
    for (int mt = 0; mt < RTV; ++mt) {
      au[mt] = base;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) au[mt] = mfma(q4_operand<8, 4>(R.v1[mt][ks]), pb[ks], au[mt]);
    }
    uint4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < N8V; ++k) {
      const float u0 = au[k / 2][2 * (k % 2)] + ror8(au[k / 2][2 * (k % 2)]);
      const float u1 = au[k / 2][2 * (k % 2) + 1] + ror8(au[k / 2][2 * (k % 2) + 1]);
      (&w.x)[k] = split2(u0, u1, rem);
    }
    const bf16x8 ub = __builtin_bit_cast(bf16x8, w);
    const floatx4 base2 = mfma(off, ub, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const floatx4 acc = mfma(q4_operand<2 * UV, N8V>(q4_unit<UV>(R.v2, mt)), ub, base2);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t d = R.sr[(4 * mt + v) / 2];
        st.o[mt][v] = __builtin_fmaf(v % 2 ? bf16_hi(d) : bf16_lo(d), acc[v], st.o[mt][v]);
      }
    }
  }
};

constexpr int kMaxSplits = kMaxDecodeSplits;

// LDS of the cross-wave merge; a format's page ring shares the space (the
// ring is drained before the merge writes it).
struct WaveMergeLds {
  float o[kWaves][kMaxG][kD];
  float m[kWaves][kMaxG];
  float l[kWaves][kMaxG];
};

// A format's value-part loads (formats reading exact-rank value parts take
// the lane's V2Lane).
#define PKV_LOAD_V(R, VP)                                                   \
  do {                                                                      \
    if constexpr (F::kExactV) F::load_values(R, VP, lane, v2_lane(a.r_v, F::kAV, lane)); \
    else F::load_values(R, VP, lane);                                       \
  } while (0)

template <class F, class KA>
__global__ __launch_bounds__(256, F::kWavesPerSimd) void decode_mfma_kernel(KA kargs) {
  const DecodeArgs& a = common_args(kargs);
  const SeqView sv = seq_view(kargs);
  constexpr int kLdsMain = F::kLdsBytes > (int)sizeof(WaveMergeLds) ? F::kLdsBytes : (int)sizeof(WaveMergeLds);
  constexpr int kLdsMainAligned = (kLdsMain + 15) / 16 * 16;
  constexpr int kLds = kLdsMainAligned + (F::kRope ? (int)sizeof(RopeLds) : 0);
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  WaveMergeLds& mg = *reinterpret_cast<WaveMergeLds*>(lds);
  RopeLds& rl = *reinterpret_cast<RopeLds*>(lds + kLdsMainAligned);  // pre-RoPE formats only
  auto& sm_o = mg.o;
  auto& sm_m = mg.m;
  auto& sm_l = mg.l;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const float rem = n >= 8 ? 1.f : 0.f;  // remainder column
  const int g = n & 7;
  const int split = sv.split, h = blockIdx.y, b = sv.b;
  const int Hq = a.Hkv * a.G;
  const int64_t bh = (int64_t)sv.b_pool * a.Hkv + h;  // (sequence, KV head) in the pools

  constexpr int PR = F::kPageRows;
  const WorkList wl = work_list(sv.T, sv.n_fact, a.n_s, PR);
  const int64_t W = (int64_t)sv.n_split * kWaves;
  const int64_t wi = (int64_t)split * kWaves + wave;
  const int64_t e0 = unit_bound(wl, a, wi, W), e1 = unit_bound(wl, a, wi + 1, W);
  // the factor slot of logical page n_s + f is f (pages are factorized in
  // order and never revisited), so unit e >= D lives in slot e - D
  const uint8_t* fac_bh = sv.fac + bh * sv.F_max * a.page_bytes;
  auto kptr = [&](int64_t ee) { return fac_bh + (ee - wl.D) * a.page_bytes; };
  auto vptr = [&](int64_t ee) { return fac_bh + (ee - wl.D) * a.page_bytes + a.k_part_bytes; };
  const int64_t f0 = e0 > wl.D ? e0 : wl.D;  // first factorized unit of this wave

  // the first factorized pages are requested before the query is read, so
  // the two memory latencies overlap: staged into the LDS ring (ring
  // formats) or loaded into the register images
  int64_t next = f0;  // next page to stage
  int s_next = 0;
  typename F::K ka, kb;
  typename F::V vr;
  if constexpr (F::kLdsRing) {
    uint8_t* ring = lds + wave * F::kRingSlots * F::kPageBytes;
    for (; next < e1 && next < f0 + F::kRingSlots - 1; ++next) {
      F::stage(ring + s_next * F::kPageBytes, kptr(next), lane);
      s_next = s_next + 1 == F::kRingSlots ? 0 : s_next + 1;
    }
  } else if constexpr (F::kKeyDoubleBuffer) {
    // (single-buffered formats are the register-tight ranks: their first
    // loads wait for the factorized section, which keeps them spill-free)
    if (f0 < e1) {
      F::load_keys(ka, kptr(f0), lane);
      PKV_LOAD_V(vr, vptr(f0));
      if (f0 + 1 < e1) F::load_keys(kb, kptr(f0 + 1), lane);
    }
  } else if constexpr (F::kRope) {
    // the first page's loads overlap the rotation table's construction
    if (f0 < e1) {
      F::load_keys(ka, kptr(f0), lane);
      PKV_LOAD_V(vr, vptr(f0));
    }
  }
  if constexpr (F::kRope) {
    rope_table_fill(rl, a.rope_freq);
    __syncthreads();
  }

  // query q * log2(e)/sqrt(d) of the lane's channels 32 ks + 8 q4 + e; as
  // an operand split into bf16 + remainder columns
  float qs[4][8];
  bf16x8 qb[4];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)b * Hq + (int64_t)h * a.G + g) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 raw = g < a.G ? __builtin_bit_cast(bf16x8, *(const uint4*)(qp + 32 * ks + 8 * q4))
                           : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[ks][e] = (float)raw[e] * a.qscale;
        qb[ks][e] = split_bf16(qs[ks][e], rem);
      }
    }
  }

  SoftState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) st.o[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // factorized pages: the next page's key part streams in while this page's
  // value half runs, and its value part while its key half runs; where the
  // register budget allows (kKeyDoubleBuffer), key parts are double-buffered
  // so that K(e + 2) streams in from the end of page e's key half
  int64_t e = f0;
  typename F::Query fq;
  if constexpr (F::kRope)
    F::query(fq, rl, wave, (const uint16_t*)a.q + ((int64_t)b * Hq + (int64_t)h * a.G + g) * kD, a.qscale,
             g < a.G, lane);
  else
    F::query(fq, qs, qb);
  if (e < e1) {
    if constexpr (F::kLdsRing) {
      // ring slot s holds pages e with e = s (mod kRingSlots); pages up to
      // e + kRingSlots - 1 are staged while page e is computed.  Register
      // images are read from the ring half a page ahead of use: page e's V
      // part before its key half, page e + 1's K part before e's value half.
      constexpr int NS = F::kRingSlots;
      uint8_t* ring = lds + wave * NS * F::kPageBytes;
      int s_cur = 0;
      typename F::K& kr = ka;
      F::wait_staged((int)(next - 1 - e));
      F::load_keys(kr, ring, lane);
      for (; e < e1; ++e) {
        if (next < e1) {  // into the slot of page e - 1, read in full last iteration
          F::stage(ring + s_next * F::kPageBytes, kptr(next), lane);
          s_next = s_next + 1 == NS ? 0 : s_next + 1;
          ++next;
        }
        const uint8_t* slot = ring + s_cur * F::kPageBytes;
        s_cur = s_cur + 1 == NS ? 0 : s_cur + 1;
        PKV_LOAD_V(vr, slot + F::kKBytes);
        typename F::Probs pb;
        F::keys(st, kr, fq, q4, rem, pb);
        if (e + 1 < e1) {
          F::wait_staged((int)(next - 2 - e));
          F::load_keys(kr, ring + s_cur * F::kPageBytes, lane);
        }
        F::values(st, vr, pb, q4, rem);
      }
    } else if constexpr (F::kKeyDoubleBuffer) {
      auto step = [&](typename F::K& kc) {
        typename F::Probs pb;
        F::keys(st, kc, fq, q4, rem, pb);
        if (e + 2 < e1) F::load_keys(kc, kptr(e + 2), lane);
        F::values(st, vr, pb, q4, rem);
        if (e + 1 < e1) PKV_LOAD_V(vr, vptr(e + 1));
      };
      while (true) {
        step(ka);
        if (++e >= e1) break;
        step(kb);
        if (++e >= e1) break;
      }
    } else {
      typename F::K& kr = ka;
      if constexpr (!F::kRope) {  // (pre-RoPE formats loaded the first page above)
        F::load_keys(kr, kptr(e), lane);
        PKV_LOAD_V(vr, vptr(e));
      }
      for (; e < e1; ++e) {
        typename F::Probs pb;
        if constexpr (F::kRope) {
          rope_page_query(fq.qb, rl.q[wave], unit_page(wl, a, e) * PR, a.rope_freq, fq.qscale, rl.base[wave],
                          lane, rem);
          F::keys(st, kr, fq, rl, lane, rem, pb);
        } else {
          F::keys(st, kr, fq, q4, rem, pb);
        }
        const bool more = e + 1 < e1;
        if (more) F::load_keys(kr, kptr(e + 1), lane);
        F::values(st, vr, pb, q4, rem);
        if (more) PKV_LOAD_V(vr, vptr(e + 1));
      }
    }
  }

  // dense pages of this range (after the factorized ones: the query operand
  // of the dense contraction is rebuilt here rather than kept live)
  bf16x8 qd[4];
  if constexpr (!F::kRope) F::dense_query(qd, fq, rem);
  const int64_t d_end = e1 < wl.D ? e1 : wl.D;
  for (int64_t e = e0; e < d_end; ++e) {
    const int64_t p = unit_page(wl, a, e);
    const int32_t ent = sv.table[p];
    const int cls = table_class(ent), slot = table_slot(ent);
    const int64_t ppg = (int64_t)PR * kD;
    const uint16_t *Kp, *Vt;
    if (cls == PKV_PAGE_SINK) {
      Kp = (const uint16_t*)sv.sink_k + (bh * a.n_s + slot) * ppg;
      Vt = (const uint16_t*)sv.sink_v + (bh * a.n_s + slot) * ppg;
    } else {
      Kp = (const uint16_t*)sv.win_k + (bh * (a.n_w + 1) + slot) * ppg;
      Vt = (const uint16_t*)sv.win_v + (bh * (a.n_w + 1) + slot) * ppg;
    }
    const int64_t left = sv.T - p * PR;
    if constexpr (F::kRope) {
      rope_page_query(fq.qb, rl.q[wave], p * PR, a.rope_freq, fq.qscale, rl.base[wave], lane, rem);
      dense_page_rope<PR>(st, Kp, Vt, (int)(left < PR ? left : PR), fq.qb, rl, lane, rem);
    } else {
      dense_page<PR>(st, Kp, Vt, (int)(left < PR ? left : PR), qd, lane, rem);
    }
  }


  // combine the hi/lo column halves of o, then merge the waves in LDS
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) st.o[mt][v] += ror8(st.o[mt][v]);
  }
  if constexpr (F::kLdsRing) __syncthreads();  // every wave is done with its ring
  if (n < 8) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sm_o[wave][n][16 * mt + 4 * q4 + v] = st.o[mt][v];
    }
    if (q4 == 0) {
      sm_m[wave][n] = st.m;
      sm_l[wave][n] = st.l;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.G * kD; idx += blockDim.x) {
    const int gg = idx / kD, c = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][gg]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = exp2f(sm_m[w][gg] - M);  // empty waves: exp2(-inf) = 0
        L += wt * sm_l[w][gg];
        O += wt * sm_o[w][gg][c];
      }
    }
    const int64_t row = ((int64_t)b * Hq + (int64_t)h * a.G + gg) * a.n_split + split;
    a.ws_o[row * kD + c] = O;
    if (c == 0) {
      a.ws_ml[row * 2 + 0] = M;
      a.ws_ml[row * 2 + 1] = L;
    }
  }
}

#undef PKV_LOAD_V

// ---------------------------------------------------------------------------
// Generic VALU kernel (fp32 or bf16 storage, any rank <= 64, G <= 8)
// ---------------------------------------------------------------------------

template <typename Elem>
__device__ inline float ld_elem(const void* base, int64_t idx) {
  if constexpr (sizeof(Elem) == 2)
    return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
  else
    return ((const float*)base)[idx];
}

template <typename Elem, bool kRope, class KA>
__global__ __launch_bounds__(256) void decode_valu_kernel(KA kargs) {
  const DecodeArgs& a = common_args(kargs);
  const SeqView sv = seq_view(kargs);
  // pre-RoPE keys: the page's keys, stored or reconstructed, then rotated
  __shared__ float kr[kRope ? kP : 1][kRope ? kD + 1 : 1];  // rows < P <= kP
  __shared__ float qs[kMaxG][kD];
  __shared__ float ts[kMaxG][kP];
  __shared__ float ss[kMaxG][kP];
  __shared__ float us[kMaxG][kP];
  __shared__ float sh_alpha[kMaxG];
  __shared__ float sh_m[kMaxG];
  __shared__ float sh_l[kMaxG];

  const int tid = threadIdx.x;
  const int split = sv.split, h = blockIdx.y, b = sv.b;
  const int G = a.G;
  const int Hq = a.Hkv * G;
  const int64_t bh = (int64_t)sv.b_pool * a.Hkv + h;  // (sequence, KV head) in the pools
  const int P = a.P;  // <= P
  const PackDims pk = pack_dims(a.r_k, P), pv = pack_dims(a.r_v, P);
  constexpr int kEsz = sizeof(Elem);

  for (int idx = tid; idx < G * kD; idx += 256) {
    const int g = idx / kD, c = idx % kD;
    qs[g][c] = ld_elem<Elem>(a.q, ((int64_t)b * Hq + (int64_t)h * G + g) * kD + c) * a.qscale;
  }
  if (tid < kMaxG) {
    sh_m[tid] = -INFINITY;
    sh_l[tid] = 0.f;
  }
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const WorkList wl = work_list(sv.T, sv.n_fact, a.n_s, P);
  const int64_t e0 = unit_bound(wl, a, split, sv.n_split), e1 = unit_bound(wl, a, split + 1, sv.n_split);
  for (int64_t e = e0; e < e1; ++e) {
    const int64_t p = unit_page(wl, a, e);
    const int32_t ent = sv.table[p];
    const int cls = table_class(ent), slot = table_slot(ent);
    const bool dense = e < wl.D;
    const int64_t rem = sv.T - p * P;
    const int nv = dense ? (int)(rem < P ? rem : P) : P;
    const void *Kp = nullptr, *Vt = nullptr, *kpart = nullptr, *vpart = nullptr;
    if (kRope) {
      const int64_t ppg = (int64_t)P * kD;
      if (!dense) {
        kpart = sv.fac + (bh * sv.F_max + slot) * a.page_bytes;
        vpart = (const uint8_t*)kpart + a.k_part_bytes;
      } else if (cls == PKV_PAGE_SINK) {
        Kp = (const uint8_t*)sv.sink_k + (bh * a.n_s + slot) * ppg * kEsz;
        Vt = (const uint8_t*)sv.sink_v + (bh * a.n_s + slot) * ppg * kEsz;
      } else {
        Kp = (const uint8_t*)sv.win_k + (bh * (a.n_w + 1) + slot) * ppg * kEsz;
        Vt = (const uint8_t*)sv.win_v + (bh * (a.n_w + 1) + slot) * ppg * kEsz;
      }
      for (int idx = tid; idx < P * kD; idx += 256) {
        const int j = idx / kD, c = idx % kD;
        float x = 0.f;
        if (dense) {
          if (j < nv) x = ld_elem<Elem>(Kp, (int64_t)j * kD + c);
        } else {
          for (int i = 0; i < a.r_k; ++i)
            x += ld_elem<Elem>(kpart, off_lf_k(pk, j, i)) * ld_elem<Elem>(kpart, off_rf_k_cm(pk, i, c));
        }
        kr[j][c] = x;
      }
      __syncthreads();
      for (int idx = tid; idx < P * (kD / 2); idx += 256) {
        const int j = idx / (kD / 2), m = idx % (kD / 2);
        float cs, sn;
        rope_sincos(p * P + j, a.rope_freq[m], cs, sn);
        const float x = kr[j][m], y = kr[j][m + kD / 2];
        kr[j][m] = x * cs - y * sn;
        kr[j][m + kD / 2] = y * cs + x * sn;
      }
      __syncthreads();
      for (int idx = tid; idx < G * P; idx += 256) {
        const int g = idx / P, j = idx % P;
        float acc = -INFINITY;
        if (j < nv) {
          acc = 0.f;
          for (int c = 0; c < kD; ++c) acc += qs[g][c] * kr[j][c];
        }
        ss[g][j] = acc;
      }
    } else if (dense) {
      const int64_t ppg = (int64_t)P * kD;
      if (cls == PKV_PAGE_SINK) {
        Kp = (const uint8_t*)sv.sink_k + (bh * a.n_s + slot) * ppg * kEsz;
        Vt = (const uint8_t*)sv.sink_v + (bh * a.n_s + slot) * ppg * kEsz;
      } else {
        Kp = (const uint8_t*)sv.win_k + (bh * (a.n_w + 1) + slot) * ppg * kEsz;
        Vt = (const uint8_t*)sv.win_v + (bh * (a.n_w + 1) + slot) * ppg * kEsz;
      }
      for (int idx = tid; idx < G * P; idx += 256) {
        const int g = idx / P, j = idx % P;
        float acc = -INFINITY;
        if (j < nv) {
          acc = 0.f;
          for (int c = 0; c < kD; ++c) acc += qs[g][c] * ld_elem<Elem>(Kp, (int64_t)j * kD + c);
        }
        ss[g][j] = acc;
      }
    } else {
      kpart = sv.fac + (bh * sv.F_max + slot) * a.page_bytes;
      vpart = (const uint8_t*)kpart + a.k_part_bytes;
      for (int idx = tid; idx < G * a.r_k; idx += 256) {
        const int g = idx / a.r_k, i = idx % a.r_k;
        float acc = 0.f;
        for (int c = 0; c < kD; ++c) acc += ld_elem<Elem>(kpart, off_rf_k(pk, i, c)) * qs[g][c];
        ts[g][i] = acc;
      }
      __syncthreads();
      for (int idx = tid; idx < G * P; idx += 256) {
        const int g = idx / P, j = idx % P;
        float acc = 0.f;
        for (int i = 0; i < a.r_k; ++i) acc += ld_elem<Elem>(kpart, off_lf_k(pk, j, i)) * ts[g][i];
        ss[g][j] = acc;
      }
    }
    __syncthreads();
    if (tid < G) {
      float mx = -INFINITY;
      for (int j = 0; j < P; ++j) mx = fmaxf(mx, ss[tid][j]);
      const float m_new = fmaxf(sh_m[tid], mx);
      const float alpha = exp2f(sh_m[tid] - m_new);
      float sum = 0.f;
      for (int j = 0; j < P; ++j) {
        const float pj = exp2f(ss[tid][j] - m_new);
        ss[tid][j] = pj;
        sum += pj;
      }
      sh_l[tid] = sh_l[tid] * alpha + sum;
      sh_m[tid] = m_new;
      sh_alpha[tid] = alpha;
    }
    __syncthreads();
    if (dense) {
      for (int k = 0; k < 4; ++k) {
        const int idx = tid + 256 * k, g = idx / kD, c = idx % kD;
        if (g >= G) break;
        float acc = o[k] * sh_alpha[g];
        for (int j = 0; j < nv; ++j) acc += ss[g][j] * ld_elem<Elem>(Vt, (int64_t)c * P + j);
        o[k] = acc;
      }
    } else {
      for (int idx = tid; idx < G * a.r_v; idx += 256) {
        const int g = idx / a.r_v, i = idx % a.r_v;
        float acc = 0.f;
        for (int j = 0; j < P; ++j) acc += ld_elem<Elem>(vpart, off_lf_v(pv, j, i)) * ss[g][j];
        us[g][i] = acc;
      }
      __syncthreads();
      for (int k = 0; k < 4; ++k) {
        const int idx = tid + 256 * k, g = idx / kD, c = idx % kD;
        if (g >= G) break;
        float acc = o[k] * sh_alpha[g];
        for (int i = 0; i < a.r_v; ++i) acc += ld_elem<Elem>(vpart, off_rf_v(pv, i, c)) * us[g][i];
        o[k] = acc;
      }
    }
    __syncthreads();
  }
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 256 * k, g = idx / kD, c = idx % kD;
    if (g >= G) break;
    const int64_t row = ((int64_t)b * Hq + (int64_t)h * G + g) * a.n_split + split;
    a.ws_o[row * kD + c] = o[k];
    if (c == 0) {
      a.ws_ml[row * 2 + 0] = sh_m[g];
      a.ws_ml[row * 2 + 1] = sh_l[g];
    }
  }
}

// Arguments of the cross-split merge.  With k_new set, the merge also takes
// the token appended in this decode step: its state (score q.k_new in log2
// units, l = 1, o = v_new) joins the n_split partial states, and the token is
// stored in row app_row of its dense page for later steps.
// Where one sequence's appended token goes: its key row and value column
// in page app_page of its (sequence, KV head) pages -- the pages of
// (b, h) = (0, 0) at k_dst / v_dst, those of consecutive (b, h)
// dst_bh_stride bytes apart -- and its page's table entry.
struct AppendDst {
  uint8_t* k_dst;
  uint8_t* v_dst;
  int64_t dst_bh_stride;
  int32_t* table_w;
  int64_t app_page;
  int app_row;
  int32_t app_entry;
  int P;  // page length of the destination cache
};

struct MergeArgs {
  const float* ws_o;
  const float* ws_ml;
  float* out;
  int n_split;
  const void* q;
  const void* k_new;
  const void* v_new;
  int dtype;
  float qscale;
  int G, Hkv;
  AppendDst app;                  // one cache: sequence b's pages are the (b, h) above
  int rope;                       // pre-RoPE keys: k_new turns by its position's angles
  float rope_freq[kD / 2];
};

// The merge of a batch of caches of batch 1 (pkv_decode_step_batch): rows of
// cache i follow those of cache i - 1; cache i's token goes to app[i].
struct MergeBatchArgs {
  MergeArgs m;                    // m.n_split: the workspace's row stride
  AppendDst app[kMaxBatchCaches];
  int ns[kMaxBatchCaches];        // splits holding cache i's states
};

__device__ inline const MergeArgs& merge_common(const MergeArgs& m) { return m; }
__device__ inline const MergeArgs& merge_common(const MergeBatchArgs& x) { return x.m; }
// the append destination of sequence seq, and the sequence's index in those pages
__device__ inline const AppendDst& append_dst(const MergeArgs& m, int64_t) { return m.app; }
__device__ inline const AppendDst& append_dst(const MergeBatchArgs& x, int64_t seq) { return x.app[seq]; }
__device__ inline int64_t append_pool_seq(const MergeArgs&, int64_t seq) { return seq; }
__device__ inline int64_t append_pool_seq(const MergeBatchArgs&, int64_t) { return 0; }
// whether sequence seq's first workgroup writes the table entry (one table
// per cache: once per launch, or once per cache of a batch)
__device__ inline bool writes_table(const MergeArgs&, int64_t seq) { return seq == 0; }
__device__ inline bool writes_table(const MergeBatchArgs&, int64_t) { return true; }
__device__ inline int split_count(const MergeArgs& m, int64_t) { return m.n_split; }
__device__ inline int split_count(const MergeBatchArgs& x, int64_t seq) { return x.ns[seq]; }

__device__ inline float load_elem(const void* p, int64_t i, int dtype) {
  if (dtype == PKV_BF16) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
  return ((const float*)p)[i];
}

// Eq. 5 across splits: one wavefront per (sequence, query head, quarter of
// the channels), four per row, so a launch spreads over 4 B H_q workgroups.
// Lane l = 8 s + c4 owns channels 32 qt + 4 c4 .. + 3 of the splits s, s + 8,
// ...  Every load of the merge (the split maxima, the lane's own split states
// and partial outputs, q and the new key) is issued up front.  The maximum,
// the new token's score and the sums over splits are lane exchanges; there
// is no LDS and no barrier.  Each of the row's four wavefronts forms the new
// token's score from the whole q and k_new (lane l: channels l and l + 64, a
// rotary pair), and writes its own 32 channels of the token into the page.
constexpr int kMergeThreads = 64;
constexpr int kMergeQuarters = 4;                 // wavefronts per row
constexpr int kMergeCh = kD / kMergeQuarters;      // channels per wavefront
constexpr int kMergeGroups = kMergeThreads / (kMergeCh / 4);  // split lanes: 8
constexpr int kMergePrefetch = 8;  // splits per lane held in registers (n_split <= 64)

template <class MA>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MA margs) {
  const MergeArgs& m = merge_common(margs);
  const int64_t row = blockIdx.x / kMergeQuarters;
  const int qt = blockIdx.x % kMergeQuarters;
  const int lane = threadIdx.x;
  const int grp = lane / (kMergeCh / 4), c4 = lane % (kMergeCh / 4);
  const int ch0 = kMergeCh * qt + 4 * c4;  // this lane's first channel
  const int Hq = m.G * m.Hkv;
  const int hq = (int)(row % Hq);
  const int64_t seq = row / Hq;
  const int n_split = split_count(margs, seq);  // this row's states, m.n_split apart
  const float2* ml = (const float2*)(m.ws_ml + row * m.n_split * 2);
  const float4* op = (const float4*)(m.ws_o + row * m.n_split * kD + ch0);

  // loads
  float qk = 0.f;
  const int64_t bh = seq * m.Hkv + hq / m.G;  // (sequence, KV head) of k_new / v_new
  const AppendDst& ad = append_dst(margs, seq);
  if (m.k_new) {
    const float k0 = load_elem(m.k_new, bh * kD + lane, m.dtype);
    const float k1 = load_elem(m.k_new, bh * kD + lane + kD / 2, m.dtype);
    float kr0 = k0, kr1 = k1;
    if (m.rope) {  // pair (lane, lane + d/2) of the new key, rotated at its position
      float cs, sn;
      rope_sincos(ad.app_page * ad.P + ad.app_row, m.rope_freq[lane], cs, sn);
      kr0 = __builtin_fmaf(-k1, sn, k0 * cs);
      kr1 = __builtin_fmaf(k0, sn, k1 * cs);
    }
    qk = load_elem(m.q, row * kD + lane, m.dtype) * kr0 +
         load_elem(m.q, row * kD + lane + kD / 2, m.dtype) * kr1;
  }
  float4 vnew = {0.f, 0.f, 0.f, 0.f};
  if (m.k_new && grp == 0) {
    const int64_t vb = bh * kD + ch0;
    vnew = float4{load_elem(m.v_new, vb, m.dtype), load_elem(m.v_new, vb + 1, m.dtype),
                  load_elem(m.v_new, vb + 2, m.dtype), load_elem(m.v_new, vb + 3, m.dtype)};
  }
  float mx = -INFINITY;
  for (int sp = lane; sp < n_split; sp += kMergeThreads) mx = fmaxf(mx, ml[sp].x);
  float2 own[kMergePrefetch];
  float4 ov[kMergePrefetch];
#pragma unroll
  for (int i = 0; i < kMergePrefetch; ++i) {
    const int sp = grp + kMergeGroups * i;
    if (sp < n_split) {
      own[i] = ml[sp];
      ov[i] = op[(int64_t)sp * (kD / 4)];
    }
  }
  // the new token goes into its dense page (the wavefronts of one query head
  // per (sequence, KV head), 32 channels each) and its table entry is set
  // (one wavefront)
  if (m.k_new) {
    if (hq % m.G == 0 && lane < kMergeCh) {
      const int c = kMergeCh * qt + lane;
      const int esz = m.dtype == PKV_BF16 ? 2 : 4;
      const int64_t bhp = append_pool_seq(margs, seq) * m.Hkv + hq / m.G;  // its pages
      uint8_t* kd = ad.k_dst + bhp * ad.dst_bh_stride + ((int64_t)ad.app_row * kD + c) * esz;
      uint8_t* vd = ad.v_dst + bhp * ad.dst_bh_stride + ((int64_t)c * ad.P + ad.app_row) * esz;
      if (esz == 2) {
        *(uint16_t*)kd = ((const uint16_t*)m.k_new)[bh * kD + c];
        *(uint16_t*)vd = ((const uint16_t*)m.v_new)[bh * kD + c];
      } else {
        *(float*)kd = ((const float*)m.k_new)[bh * kD + c];
        *(float*)vd = ((const float*)m.v_new)[bh * kD + c];
      }
    }
    if (hq == 0 && qt == 0 && lane == 0 && writes_table(margs, seq)) ad.table_w[ad.app_page] = ad.app_entry;
  }

  // global maximum and the new token's score (log2 units), in every lane
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    qk += __shfl_xor(qk, o);
  }
  float M = mx, s_new = -INFINITY;
  if (m.k_new) s_new = qk * m.qscale;
  M = fmaxf(M, s_new);

  // this lane's splits, weighted e^(m_s - M) (empty split: weight 0)
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  auto add = [&](float2 st, float4 v) {
    const float wt = M == -INFINITY ? 0.f : exp2f(st.x - M);
    acc.x += wt * v.x;
    acc.y += wt * v.y;
    acc.z += wt * v.z;
    acc.w += wt * v.w;
    lsum += wt * st.y;
  };
#pragma unroll
  for (int i = 0; i < kMergePrefetch; ++i)
    if (grp + kMergeGroups * i < n_split) add(own[i], ov[i]);
  for (int sp = grp + kMergeGroups * kMergePrefetch; sp < n_split; sp += kMergeGroups)
    add(ml[sp], op[(int64_t)sp * (kD / 4)]);
  // sum over the 8 split lanes of each channel group (lanes c4, c4 + 8, ...)
#pragma unroll
  for (int o = kMergeCh / 4; o < kMergeThreads; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o);
    acc.y += __shfl_xor(acc.y, o);
    acc.z += __shfl_xor(acc.z, o);
    acc.w += __shfl_xor(acc.w, o);
    lsum += __shfl_xor(lsum, o);
  }
  if (grp == 0) {
    float4 t = acc;
    float L = lsum;
    if (m.k_new) {
      const float w_new = exp2f(s_new - M);
      t.x += w_new * vnew.x;
      t.y += w_new * vnew.y;
      t.z += w_new * vnew.z;
      t.w += w_new * vnew.w;
      L += w_new;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *(float4*)(m.out + row * kD + ch0) = float4{t.x * inv, t.y * inv, t.z * inv, t.w * inv};
  }
}

}  // namespace

int decode_default_splits(const CacheGeom& g, int64_t T, int64_t n_fact) {
  (void)n_fact;
  const int64_t pages = (T + g.P - 1) / g.P;
  const int64_t bh = (int64_t)g.B * g.Hkv;
  // Two four-wave workgroups per CU fill the chip at 2 waves per SIMD; halve
  // the split count while a wave would get fewer than min_run pages and a CU
  // would still get a workgroup.  bf16 pages: long runs per wave stream
  // better than more waves (Qwen3-32B-shaped 128K layer: 32 splits 48.0 us,
  // 64 splits 49.5 us); INT4 pages are a third of the bytes and compute-bound
  // per wave, so both workgroups per CU pay off (same layer: 32 splits
  // 37.1 us, 64 splits 35.0 us), and so do pre-RoPE keys, whose rotation is
  // vector-ALU work (same layer: 32 splits 72.6 us, 64 splits 64.4 us).
  const int n8 = (g.r_k > g.r_v ? g.r_k + 7 : g.r_v + 7) / 8;
  const int wps = g.dtype != PKV_BF16 ? 2 : g.rope ? rope_waves_per_simd(n8) : mfma_waves_per_simd(n8);  // INT4, fp32: 2
  const int64_t min_run = (g.dtype == PKV_BF16_INT4 || g.rope) ? 8 : 16;
  int64_t s = (256LL * wps + bh - 1) / bh;
  while (s > 1 && pages < min_run * 4 * s && (s / 2) * bh >= 256) s /= 2;
  const int64_t cap = (pages + 3) / 4;  // at least ~4 pages per workgroup
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

namespace {

MergeArgs merge_args(const CacheGeom& g, const AttnJob& job) {
  MergeArgs m;
  m.ws_o = job.ws_o;
  m.ws_ml = job.ws_ml;
  m.out = job.out;
  m.n_split = job.n_split;
  m.q = job.q;
  m.k_new = job.k_new;
  m.v_new = job.v_new;
  m.dtype = dense_dtype(g.dtype);
  m.qscale = kLog2e / sqrtf((float)kD);
  m.G = g.G;
  m.Hkv = g.Hkv;
  m.app = AppendDst{nullptr, nullptr, 0, nullptr, -1, -1, 0, g.P};
  m.rope = g.rope && job.k_new;
  std::memcpy(m.rope_freq, g.rope_freq, sizeof(m.rope_freq));
  return m;
}

// The append destination of job's token in cache g (page app_page: a sink
// page or a ring slot).
AppendDst append_dst_of(const CacheGeom& g, const AttnJob& job) {
  AppendDst d{nullptr, nullptr, 0, (int32_t*)(g.base + g.lay.page_table), job.app_page, job.app_row,
              job.app_entry, g.P};
  const int64_t ppg_bytes = (int64_t)g.P * kD * g.lay.elem_bytes;
  const int64_t p = job.app_page;
  if (p < g.n_s) {
    d.k_dst = g.base + g.lay.sink_k + p * ppg_bytes;
    d.v_dst = g.base + g.lay.sink_v + p * ppg_bytes;
    d.dst_bh_stride = g.n_s * ppg_bytes;
  } else {
    const int64_t slot = (p - g.n_s) % (g.n_w + 1);
    d.k_dst = g.base + g.lay.win_k + slot * ppg_bytes;
    d.v_dst = g.base + g.lay.win_v + slot * ppg_bytes;
    d.dst_bh_stride = (int64_t)(g.n_w + 1) * ppg_bytes;
  }
  return d;
}

}  // namespace

bool batched_kernel(const CacheGeom& g) {
  const int n8k = (g.r_k + 7) / 8, n8v = (g.r_v + 7) / 8;
  if (n8k != n8v) return false;
  if (g.P != kP) return g.dtype == PKV_BF16 || g.dtype == PKV_BF16_INT4;  // the 32-row formats (r <= 32)
  if (g.dtype == PKV_BF16_INT4) return n8k <= 4;
  return g.dtype == PKV_BF16 && n8k <= 8;
}

int decode_batch_splits(const CacheGeom& g, const int64_t* T, int n, int* ns) {
  // Workgroups that fill the chip in one round (two per CU at two waves per
  // SIMD), shared in proportion to the caches' pages: each cache's split
  // gets about q pages, the smallest q (at least 8 pages per wave) whose
  // splits all fit.  The longest cache then bounds the launch with runs as
  // short as the others'.
  const int n8 = (g.r_k > g.r_v ? g.r_k + 7 : g.r_v + 7) / 8;
  const int wps = g.dtype != PKV_BF16 ? 2 : g.rope ? rope_waves_per_simd(n8) : mfma_waves_per_simd(n8);
  const int64_t budget = (256LL * wps) / g.Hkv;  // splits over all caches
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += (T[i] + g.P - 1) / g.P;
  int64_t q = budget > 0 ? (total + budget - 1) / budget : total;
  if (q < 4 * 8) q = 4 * 8;
  for (;; ++q) {
    int64_t sum = 0;
    for (int i = 0; i < n; ++i) sum += std::max<int64_t>(1, ((T[i] + g.P - 1) / g.P + q - 1) / q);
    if (sum <= std::max<int64_t>(budget, n)) break;
  }
  int grid = 1;
  for (int i = 0; i < n; ++i) {
    int64_t s = std::max<int64_t>(1, ((T[i] + g.P - 1) / g.P + q - 1) / q);
    if (s > kMaxSplits) s = kMaxSplits;
    ns[i] = (int)s;
    grid = std::max(grid, ns[i]);
  }
  return grid;
}

hipError_t launch_merge(const CacheGeom& g, const AttnJob& job, hipStream_t stream) {
  MergeArgs m = merge_args(g, job);
  if (job.k_new) m.app = append_dst_of(g, job);
  hipLaunchKernelGGL(merge_kernel<MergeArgs>, dim3((unsigned)((int64_t)g.B * g.Hq * kMergeQuarters)),
                     dim3(kMergeThreads), 0, stream, m);
  return hipGetLastError();
}

hipError_t launch_merge_batch(const CacheGeom* gs, int n, const AttnJob& job, const AttnJob* apps, const int* ns,
                              hipStream_t stream) {
  if (n < 1 || n > kMaxBatchCaches) return hipErrorInvalidValue;
  MergeBatchArgs x;
  x.m = merge_args(gs[0], job);
  for (int i = 0; i < n; ++i) {
    x.app[i] = job.k_new ? append_dst_of(gs[i], apps[i]) : AppendDst{nullptr, nullptr, 0, nullptr, -1, -1, 0, gs[i].P};
    x.ns[i] = ns[i];
  }
  hipLaunchKernelGGL(merge_kernel<MergeBatchArgs>, dim3((unsigned)((int64_t)n * gs[0].Hq * kMergeQuarters)),
                     dim3(kMergeThreads), 0, stream, x);
  return hipGetLastError();
}

namespace {

DecodeArgs make_args(const CacheGeom& g, const AttnJob& job) {
  DecodeArgs a;
  a.q = job.q;
  a.fac = g.base + g.lay.factors;
  a.sink_k = g.base + g.lay.sink_k;
  a.sink_v = g.base + g.lay.sink_v;
  a.win_k = g.base + g.lay.win_k;
  a.win_v = g.base + g.lay.win_v;
  a.table = (const int32_t*)(g.base + g.lay.page_table);
  a.ws_o = job.ws_o;
  a.ws_ml = job.ws_ml;
  a.B = g.B;
  a.Hkv = g.Hkv;
  a.G = g.G;
  a.n_split = job.n_split;
  a.P = g.P;
  a.n_s = g.n_s;
  a.n_w = g.n_w;
  a.r_k = g.r_k;
  a.r_v = g.r_v;
  a.T = job.T;
  a.n_fact = job.n_fact;
  a.F_max = g.F_max;
  a.page_bytes = g.lay.factor_page_bytes;
  a.k_part_bytes = g.lay.factor_k_bytes;
  // cost of a unit ~ bytes it streams (dense: K and V pages)
  a.cost_dense = 2 * g.lay.dense_page_bytes / 64;
  a.cost_fact = g.lay.factor_page_bytes / 64;
  a.qscale = kLog2e / sqrtf((float)kD);
  a.rope = g.rope;
  std::memcpy(a.rope_freq, g.rope_freq, sizeof(a.rope_freq));
  return a;
}

// The partial kernel of the cache format, with kernel arguments ka (one
// cache, or a batch of caches: DecodeBatchArgs).  A batch covers the formats
// with equal K and V ranks per 8; hipErrorNotSupported otherwise.
template <class KA>
hipError_t dispatch_partial(const CacheGeom& g, const KA& ka, dim3 grid, hipStream_t stream) {
  constexpr bool kBatch = std::is_same<KA, DecodeBatchArgs>::value;
  const KernelEvents kev = take_kernel_events();
  const int n8k = (g.r_k + 7) / 8, n8v = (g.r_v + 7) / 8;
  // bf16 value parts below r8 = 32 whose rank 8 does not divide keep V2 at
  // the exact rank: their formats' EV instantiations
  const bool ev = g.r_v % 8 != 0 && n8v <= 4;
  if (g.dtype == PKV_BF16_INT4 && g.P == kMinP) {
    if (kBatch && n8k != n8v) return hipErrorNotSupported;
    switch (n8k * 8 + n8v) {
#define PKV_Q4H(NK, NV)                                                                                    \
  case NK * 8 + NV:                                                                                        \
    if constexpr (!kBatch || NK == NV)                                                                     \
      hipExtLaunchKernelGGL((decode_mfma_kernel<Int4Factors<NK, NV, kMinP>, KA>), grid, dim3(256), 0, stream, \
                            kev.start, kev.stop, 0, ka);                                                     \
    break;
#define PKV_Q4H_ROW(NK) PKV_Q4H(NK, 1) PKV_Q4H(NK, 2) PKV_Q4H(NK, 3) PKV_Q4H(NK, 4)
      PKV_Q4H_ROW(1)
      PKV_Q4H_ROW(2)
      PKV_Q4H_ROW(3)
      PKV_Q4H_ROW(4)
#undef PKV_Q4H_ROW
#undef PKV_Q4H
      default:
        return hipErrorInvalidValue;
    }
  } else if (g.dtype == PKV_BF16_INT4) {
    if (kBatch && n8k != n8v) return hipErrorNotSupported;
    switch (n8k * 8 + n8v) {
#define PKV_Q4(NK, NV)                                                                              \
  case NK * 8 + NV:                                                                                 \
    if constexpr (!kBatch || NK == NV)                                                              \
      hipExtLaunchKernelGGL((decode_mfma_kernel<Int4Factors<NK, NV>, KA>), grid, dim3(256), 0, stream, \
                            kev.start, kev.stop, 0, ka);                                              \
    break;
#define PKV_Q4_ROW(NK) PKV_Q4(NK, 1) PKV_Q4(NK, 2) PKV_Q4(NK, 3) PKV_Q4(NK, 4)
      PKV_Q4_ROW(1)
      PKV_Q4_ROW(2)
      PKV_Q4_ROW(3)
      PKV_Q4_ROW(4)
#undef PKV_Q4_ROW
#undef PKV_Q4
      default:
        return hipErrorInvalidValue;
    }
  } else if (g.dtype == PKV_BF16 && g.P == kP && n8k == n8v) {
    switch (n8k * 2 + (g.rope ? 1 : 0)) {
#define PKV_CASE(N)                                                                                        \
  case 2 * N:                                                                                              \
    if constexpr (N <= 4) {                                                                                \
      if (ev) {                                                                                            \
        hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Factors<N, N, true>, KA>), grid, dim3(256), 0, stream, \
                              kev.start, kev.stop, 0, ka);                                                 \
        break;                                                                                             \
      }                                                                                                    \
    }                                                                                                      \
    hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Factors<N>, KA>), grid, dim3(256), 0, stream, kev.start, \
                          kev.stop, 0, ka);                                                                \
    break;
#define PKV_ROPE(N)                                                                                        \
  case 2 * N + 1:                                                                                          \
    if constexpr (N <= 4) {                                                                                \
      if (ev) {                                                                                            \
        hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<N, kP, true>, KA>), grid, dim3(256), 0,      \
                              stream, kev.start, kev.stop, 0, ka);                                         \
        break;                                                                                             \
      }                                                                                                    \
    }                                                                                                      \
    hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<N>, KA>), grid, dim3(256), 0, stream, kev.start,   \
                          kev.stop, 0, ka);                                                                \
    break;
      PKV_CASE(1)
      PKV_CASE(2)
      PKV_CASE(3)
      PKV_CASE(4)
      PKV_CASE(5)
      PKV_CASE(6)
      PKV_CASE(7)
      PKV_CASE(8)
      PKV_ROPE(1)
      PKV_ROPE(2)
      PKV_ROPE(3)
      PKV_ROPE(4)
      PKV_ROPE(5)
      PKV_ROPE(6)
      PKV_ROPE(7)
      PKV_ROPE(8)
#undef PKV_ROPE
#undef PKV_CASE
      default:
        return hipErrorInvalidValue;
    }
  } else if (g.dtype == PKV_BF16 && g.P == kMinP && n8k == n8v && g.rope && n8k <= kRopeOneStepMaxN8) {
    switch (n8k) {
#define PKV_HALF_ROPE(N)                                                                                   \
  case N:                                                                                                  \
    if (ev)                                                                                                \
      hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<N, kMinP, true>, KA>), grid, dim3(256), 0,     \
                            stream, kev.start, kev.stop, 0, ka);                                           \
    else                                                                                                   \
      hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<N, kMinP>, KA>), grid, dim3(256), 0, stream,   \
                            kev.start, kev.stop, 0, ka);                                                   \
    break;
      PKV_HALF_ROPE(1)
      PKV_HALF_ROPE(2)
      PKV_HALF_ROPE(3)
      PKV_HALF_ROPE(4)
#undef PKV_HALF_ROPE
      default:
        return hipErrorInvalidValue;
    }
  } else if (g.dtype == PKV_BF16 && g.P == kMinP && n8k == n8v && !g.rope) {
    switch (n8k) {
#define PKV_HALF(N)                                                                                    \
  case N:                                                                                              \
    if (ev)                                                                                            \
      hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Half<N, N, true>, KA>), grid, dim3(256), 0, stream, \
                            kev.start, kev.stop, 0, ka);                                               \
    else                                                                                               \
      hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Half<N>, KA>), grid, dim3(256), 0, stream, kev.start, \
                            kev.stop, 0, ka);                                                          \
    break;
      PKV_HALF(1)
      PKV_HALF(2)
      PKV_HALF(3)
      PKV_HALF(4)
#undef PKV_HALF
      default:
        return hipErrorInvalidValue;
    }
  } else if (g.dtype == PKV_BF16 && !g.rope && n8k != n8v && n8k <= 4 && n8v <= 4) {
    // unequal padded ranks up to 32 (batches launch once per cache: the
    // batched kernel's caches share one format)
    if constexpr (kBatch) {
      return hipErrorNotSupported;
    } else {
      switch ((g.P == kMinP ? 64 : 0) + n8k * 8 + n8v) {
#define PKV_ASYM(NK, NV)                                                                                 \
  case NK * 8 + NV:                                                                                      \
    if constexpr (NK != NV) {                                                                            \
      if (ev)                                                                                            \
        hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Factors<NK, NV, true>, KA>), grid, dim3(256), 0,   \
                              stream, kev.start, kev.stop, 0, ka);                                       \
      else                                                                                               \
        hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Factors<NK, NV>, KA>), grid, dim3(256), 0, stream, \
                              kev.start, kev.stop, 0, ka);                                               \
    }                                                                                                    \
    break;                                                                                               \
  case 64 + NK * 8 + NV:                                                                                 \
    if constexpr (NK != NV) {                                                                            \
      if (ev)                                                                                            \
        hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Half<NK, NV, true>, KA>), grid, dim3(256), 0,      \
                              stream, kev.start, kev.stop, 0, ka);                                       \
      else                                                                                               \
        hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Half<NK, NV>, KA>), grid, dim3(256), 0, stream,    \
                              kev.start, kev.stop, 0, ka);                                               \
    }                                                                                                    \
    break;
#define PKV_ASYM_ROW(NK) PKV_ASYM(NK, 1) PKV_ASYM(NK, 2) PKV_ASYM(NK, 3) PKV_ASYM(NK, 4)
        PKV_ASYM_ROW(1)
        PKV_ASYM_ROW(2)
        PKV_ASYM_ROW(3)
        PKV_ASYM_ROW(4)
#undef PKV_ASYM_ROW
#undef PKV_ASYM
        default:
          return hipErrorInvalidValue;
      }
    }
  } else if (g.dtype == PKV_BF16 && !g.rope && g.P == kP && n8k != n8v && n8k <= 8 && n8v <= 8) {
    // unequal padded ranks with one above 32 (64-token pages; one launch per
    // cache in a batch, as above)
    if constexpr (kBatch) {
      return hipErrorNotSupported;
    } else {
      switch (n8k * 8 + n8v) {
#define PKV_ASYM_WIDE(NK, NV)                                                                             \
  case NK * 8 + NV:                                                                                       \
    if constexpr (NK != NV && (NK > 4 || NV > 4)) {                                                       \
      if constexpr (NV <= 4) {                                                                            \
        if (ev) {                                                                                         \
          hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Factors<NK, NV, true>, KA>), grid, dim3(256), 0,  \
                                stream, kev.start, kev.stop, 0, ka);                                      \
          break;                                                                                          \
        }                                                                                                 \
      }                                                                                                   \
      hipExtLaunchKernelGGL((decode_mfma_kernel<Bf16Factors<NK, NV>, KA>), grid, dim3(256), 0, stream,    \
                            kev.start, kev.stop, 0, ka);                                                  \
    }                                                                                                     \
    break;
#define PKV_ASYM_WIDE_ROW(NK)                                                                            \
  PKV_ASYM_WIDE(NK, 1) PKV_ASYM_WIDE(NK, 2) PKV_ASYM_WIDE(NK, 3) PKV_ASYM_WIDE(NK, 4) PKV_ASYM_WIDE(NK, 5) \
  PKV_ASYM_WIDE(NK, 6) PKV_ASYM_WIDE(NK, 7) PKV_ASYM_WIDE(NK, 8)
        PKV_ASYM_WIDE_ROW(1)
        PKV_ASYM_WIDE_ROW(2)
        PKV_ASYM_WIDE_ROW(3)
        PKV_ASYM_WIDE_ROW(4)
        PKV_ASYM_WIDE_ROW(5)
        PKV_ASYM_WIDE_ROW(6)
        PKV_ASYM_WIDE_ROW(7)
        PKV_ASYM_WIDE_ROW(8)
#undef PKV_ASYM_WIDE_ROW
#undef PKV_ASYM_WIDE
        default:
          return hipErrorInvalidValue;
      }
    }
  } else if (g.dtype == PKV_BF16 && g.rope && n8k != n8v && n8k <= kRopeOneStepMaxN8 && n8v <= kRopeOneStepMaxN8) {
    // pre-RoPE keys at unequal padded ranks up to 32 (one launch per cache
    // in a batch, as above)
    if constexpr (kBatch) {
      return hipErrorNotSupported;
    } else {
      switch ((g.P == kMinP ? 64 : 0) + n8k * 8 + n8v) {
#define PKV_ROPE_ASYM(NK, NV)                                                                              \
  case NK * 8 + NV:                                                                                        \
    if constexpr (NK != NV) {                                                                              \
      if (ev)                                                                                              \
        hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<NK, kP, true, NV>, KA>), grid, dim3(256), 0, \
                              stream, kev.start, kev.stop, 0, ka);                                         \
      else                                                                                                 \
        hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<NK, kP, false, NV>, KA>), grid, dim3(256), 0, \
                              stream, kev.start, kev.stop, 0, ka);                                         \
    }                                                                                                      \
    break;                                                                                                 \
  case 64 + NK * 8 + NV:                                                                                   \
    if constexpr (NK != NV) {                                                                              \
      if (ev)                                                                                              \
        hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<NK, kMinP, true, NV>, KA>), grid, dim3(256), \
                              0, stream, kev.start, kev.stop, 0, ka);                                      \
      else                                                                                                 \
        hipExtLaunchKernelGGL((decode_mfma_kernel<RopeFactors<NK, kMinP, false, NV>, KA>), grid, dim3(256), \
                              0, stream, kev.start, kev.stop, 0, ka);                                      \
    }                                                                                                      \
    break;
#define PKV_ROPE_ASYM_ROW(NK) PKV_ROPE_ASYM(NK, 1) PKV_ROPE_ASYM(NK, 2) PKV_ROPE_ASYM(NK, 3) PKV_ROPE_ASYM(NK, 4)
        PKV_ROPE_ASYM_ROW(1)
        PKV_ROPE_ASYM_ROW(2)
        PKV_ROPE_ASYM_ROW(3)
        PKV_ROPE_ASYM_ROW(4)
#undef PKV_ROPE_ASYM_ROW
#undef PKV_ROPE_ASYM
        default:
          return hipErrorInvalidValue;
      }
    }
  } else if constexpr (kBatch) {
    return hipErrorNotSupported;
  } else if (g.dtype == PKV_BF16) {
    if (g.rope)
      hipExtLaunchKernelGGL((decode_valu_kernel<uint16_t, true, KA>), grid, dim3(256), 0, stream, kev.start,
                            kev.stop, 0, ka);
    else
      hipExtLaunchKernelGGL((decode_valu_kernel<uint16_t, false, KA>), grid, dim3(256), 0, stream, kev.start,
                            kev.stop, 0, ka);
  } else {
    if (g.rope)
      hipExtLaunchKernelGGL((decode_valu_kernel<float, true, KA>), grid, dim3(256), 0, stream, kev.start,
                            kev.stop, 0, ka);
    else
      hipExtLaunchKernelGGL((decode_valu_kernel<float, false, KA>), grid, dim3(256), 0, stream, kev.start,
                            kev.stop, 0, ka);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partial(const CacheGeom& g, const AttnJob& job, hipStream_t stream) {
  return dispatch_partial(g, make_args(g, job), dim3(job.n_split, g.Hkv, g.B), stream);
}

hipError_t launch_partial_batch(const CacheGeom* gs, const int64_t* T, const int64_t* n_fact, const int* ns,
                                int n, const AttnJob& job, hipStream_t stream) {
  if (n < 1 || n > kMaxBatchCaches) return hipErrorInvalidValue;
  DecodeBatchArgs x;
  x.a = make_args(gs[0], job);
  x.n_seq = n;
  int cols = 0;
  for (int i = 0; i < n; ++i) {
    const CacheGeom& g = gs[i];
    if (ns[i] < 1 || ns[i] > job.n_split) return hipErrorInvalidValue;
    x.seq[i] = BatchSeq{g.base + g.lay.factors, g.base + g.lay.sink_k, g.base + g.lay.sink_v,
                        g.base + g.lay.win_k, g.base + g.lay.win_v,
                        (const int32_t*)(g.base + g.lay.page_table), T[i], n_fact[i], g.F_max, cols, ns[i]};
    cols += ns[i];
  }
  return dispatch_partial(gs[0], x, dim3(cols, gs[0].Hkv, 1), stream);
}

// Library-held decode workspace for callers that cannot allocate
// (pkv_decode_attn_noalloc).  In host code `scratch` names a host-side
// stand-in, not device memory: its address on each device comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.  Every call on a device shares the
// device's copy, so calls that overlap on one device race.
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pkv
