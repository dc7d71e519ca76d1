/*
 * pkv.h -- C-ABI of the MI355X (gfx950) PuzzleKV hot path.
 *
 * Method: "PuzzleKV: Page-Wise Low-Rank Decomposition for KV Cache
 * Compression" (arXiv 2608.23843).  Each completed P-token page of one layer's
 * KV head is stored as rank-r factors (Sec. 3.3, Eq. 2) obtained from the
 * page's P x P Gram matrix (Sec. 3.3, text after Eq. 3); a sink region and a
 * recent window stay dense (Sec. 3.3, steps (1)-(3)); decode attention runs
 * directly on dense and factorized pages with an online-softmax merge
 * (Sec. 3.3 (4), Eq. 4 and Eq. 5); new pages are factorized once as they
 * leave the window (Sec. 3.3 "Incremental Cache Update (5)").
 *
 * Conventions for every call
 *  - Return value: a pkv_status (0 = PKV_OK).  No call throws; when a call
 *    returns an error it has changed no state and enqueued no work.
 *  - Pointers named "device" point to GPU memory the caller owns (for example
 *    torch tensors).  The library never allocates or frees device memory and
 *    never synchronizes a stream, except pkv_read_page_table, which must
 *    return host data.  Host handles (pkv_cache) are allocated by
 *    pkv_cache_create and freed by pkv_cache_destroy.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work of a call is enqueued on it in order.
 *  - Calls on one cache must be serialized by the caller (they update the
 *    cache's host-side state); distinct caches are independent.
 *  - dtype: PKV_BF16 (bfloat16 storage, float32 arithmetic), PKV_F32, or
 *    PKV_BF16_INT4 (bfloat16 K, V, q and dense pages; factor pages held as
 *    the INT4 factors of Sec. 4.3).  K, V, q and the dense pages have the
 *    cache's element type (bf16 for PKV_BF16_INT4); attention output is
 *    float32.
 *  - Fixed in this version: head_dim d = 128, page length P = 64 or 32
 *    (other values return PKV_ERR_UNSUPPORTED); GQA group size
 *    G = H_q / H_kv <= 8.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,       /* bad size, null or misaligned pointer, bad combination */
  PKV_ERR_UNSUPPORTED = 2,       /* valid for the method, not implemented (d != 128, P not 64 or 32, G > 8) */
  PKV_ERR_CAPACITY = 3,          /* more tokens than max_tokens, workspace too small */
  PKV_ERR_NOT_ELIGIBLE = 4,      /* promotion requested with no page waiting */
  PKV_ERR_PROMOTION_PENDING = 5, /* append refused: a completed page must be promoted first */
  PKV_ERR_DEVICE = 6             /* a HIP runtime call or kernel launch failed */
} pkv_status;

/*
 * Storage formats.  PKV_BF16_INT4 (Sec. 4.3 "Quantization Compatibility"):
 * the singular values are split between the factors, Lt = U_r Sigma_r^(1/2)
 * (P x r) and Rt = Sigma_r^(1/2) W_r^T (r x d), and each factor is stored as
 * symmetric 4-bit codes c in -7..7 with one bfloat16 scale s per group:
 * per column of Lt_K, Rt_K and Rt_V, per row of Lt_V;
 * s = bf16_rne(max |x| / 7), c = clamp(rint(x / s), -7, 7) (c = 0 where
 * s = 0), x ~ c s.  Ranks up to 32; dense pages are bfloat16.
 */
typedef enum pkv_dtype { PKV_BF16 = 0, PKV_F32 = 1, PKV_BF16_INT4 = 2 } pkv_dtype;

/* Page classes reported by the page table (Sec. 3.3 (1)-(3), Sec. 4.1). */
typedef enum pkv_page_class {
  PKV_PAGE_UNUSED = 0, /* beyond the current length */
  PKV_PAGE_SINK = 1,   /* one of the first s/P pages; dense */
  PKV_PAGE_FACT = 2,   /* completed page stored as factors */
  PKV_PAGE_WIN = 3,    /* completed page in the dense recent window */
  PKV_PAGE_PART = 4    /* page still being filled; dense */
} pkv_page_class;

/* Factor part selector for pkv_pack_factors / pkv_unpack_factors.
 * PKV_KEYS_PRE_ROPE is the key part of a cache holding pre-RoPE keys
 * (pkv_cache_set_key_rope): the same elements as PKV_KEYS, with Rf_K stored
 * channel-major (in the order of the value part's Rf_V). */
typedef enum pkv_factor_kind { PKV_KEYS = 0, PKV_VALUES = 1, PKV_KEYS_PRE_ROPE = 2 } pkv_factor_kind;

/* Shape and parameters of one layer's hybrid cache (passed by pointer). */
typedef struct pkv_shape {
  int32_t batch;      /* B sequences; all have the same length T */
  int32_t n_q_heads;  /* H_q */
  int32_t n_kv_heads; /* H_kv, H_q % H_kv == 0; query head h reads KV head h / G */
  int32_t head_dim;   /* d (must be 128) */
  int32_t page_len;   /* P: 64, or 32 (Sec. 4.1 default) */
  int32_t rank_k;     /* r_K, 1 <= r_K <= min(P, d) */
  int32_t rank_v;     /* r_V, 1 <= r_V <= min(P, d) */
  int32_t sink;       /* s: dense sink tokens, a multiple of P (may be 0) */
  int32_t window;     /* w: dense window tokens (completed pages), a multiple of P */
  int32_t max_tokens; /* capacity T_max >= 1 */
  int32_t dtype;      /* pkv_dtype */
} pkv_shape;

/*
 * Device-buffer layout of a cache: the preallocated dense sink, the dense
 * window ring, the factor pool and the page table of Sec. 3.3 (1)-(3) and
 * (5).  Byte offsets from the caller's buffer, in this order, each region
 * starting at the previous one's end rounded up to 256 bytes.  With
 * n_s = s/P, n_w = w/P:
 *   sink_k  [B][H_kv][n_s][P][d]        keys, row-major
 *   sink_v  [B][H_kv][n_s][d][P]        values, transposed per page
 *   win_k   [B][H_kv][n_w+1][P][d]      ring of window/partial key pages
 *   win_v   [B][H_kv][n_w+1][d][P]      ring of value pages, transposed
 *   factors [B][H_kv][F_max][factor_page_bytes]   K part, then V part
 *   page_table [max_pages] int32: (class << 24) | slot
 * total_bytes is the page table's end rounded up to 256.
 * Factor parts (PKV_BF16, PKV_F32) use a fixed interleaved order matched to
 * the attention kernel's matrix-core register layout.  The Lf operands, and
 * Rf of key parts, pad the rank to r8 = 8 ceil(r / 8) (padding ranks hold
 * zeros); Rf of value parts keeps r2 = r rounded up to even when r8 <= 32
 * (r8 otherwise).  A key part holds r8 (P + d) elements, a value part
 * r8 P + r2 d, at either page length (the same count when 8 divides r).  A
 * P = 32 part is the P = 64 order with the operand rows of page rows 32..63
 * left out.
 * pkv_pack_factors and pkv_unpack_factors convert between a part and
 * row-major Lf (P x r), Rf (r x d).
 * PKV_BF16_INT4 parts hold codes and scales in their own interleaved order
 * (sizes at pkv_factor_part_bytes); pkv_pack_factors_int4 and
 * pkv_unpack_factors_int4 convert it.
 */
typedef struct pkv_layout {
  uint64_t sink_k, sink_v, win_k, win_v, factors, page_table;
  uint64_t total_bytes;
  int64_t n_sink_slots;      /* n_s */
  int64_t n_ring_slots;      /* n_w + 1 */
  int64_t max_fact_pages;    /* F_max = max(0, floor(T_max/P) - n_s - n_w) */
  int64_t max_pages;         /* ceil(T_max / P) */
  int64_t elem_bytes;        /* bytes of a dense element: 2 (bf16, bf16+int4) or 4 (f32) */
  int64_t dense_page_bytes;  /* P * d * elem_bytes */
  int64_t factor_k_elems;    /* packed elements (INT4: codes) of a K part: r8_K (P + d),
                                r8 = 8 ceil(r / 8), at P = 64 and P = 32 */
  int64_t factor_v_elems;    /* of a V part: r8_V P + r2_V d (INT4: codes, r8_V (P + d)) */
  int64_t factor_page_bytes; /* factor_k_bytes + factor_v_bytes */
  int64_t factor_k_bytes;    /* bytes of a K part (its offset in the page is 0): elems x
                                elem_bytes, or pkv_factor_part_bytes for INT4 */
  int64_t factor_v_bytes;    /* bytes of a V part (offset factor_k_bytes) */
} pkv_layout;

typedef struct pkv_cache pkv_cache; /* opaque host handle */

/* Human-readable name of a status code (static string). */
const char* pkv_status_string(int32_t status);
const char* pkv_version(void);

/* Eq. 3 (also App. D.1 Eq. 6): storage of a factorized K/V page pair over
 * its dense storage, (r_K + r_V)(P + d) / (2 P d).  Host only. */
double pkv_storage_ratio(int32_t P, int32_t r_k, int32_t r_v, int32_t d);

/*
 * Page classification of a T-token cache (Sec. 3.3 (1)-(3) and (5); Sec. 4.1
 * default dense region).  Host only, no GPU needed.
 *   n_fact < 0: steady state -- every completed non-sink page except the n_w
 *               most recent is FACT;
 *   n_fact >= 0: exactly the first n_fact such pages are FACT (the state
 *               between a page-completing append and its promotion).
 * Writes cls[p] (pkv_page_class) and slot[p] for p < n_pages; pages beyond
 * ceil(T/P) get UNUSED / 0.  Slots: SINK p; FACT p - n_s; WIN and PART
 * (p - n_s) mod (n_w + 1).  Errors: INVALID_ARG if s or w is not a multiple
 * of P, T < 0, or a pointer is null.
 */
int32_t pkv_classify(int64_t T, int32_t P, int32_t s, int32_t w, int64_t n_fact, int32_t* cls,
                     int32_t* slot, int64_t n_pages);

/* Packed elements of one factor part of `kind` (pkv_factor_kind) for rank r,
 * at P = 64 and at P = 32: r8 (P + d) for PKV_KEYS and PKV_KEYS_PRE_ROPE,
 * r8 P + r2 d for PKV_VALUES, with r8 = r rounded up to a multiple of 8 and
 * r2 = r rounded up to even (r2 = r8 when r8 > 32).  Errors: UNSUPPORTED
 * for other P or d != 128; INVALID_ARG for another kind or unless
 * 1 <= r <= P.  Host only. */
int32_t pkv_factor_part_elems(int32_t kind, int32_t P, int32_t d, int32_t r, int64_t* elems);

/*
 * Host-side conversion between row-major factors (float32 Lf [P][r] with
 * Lf = U_r Sigma_r, Rf [r][d] with Rf = W_r^T; Sec. 3.2 "Truncated SVD",
 * Sec. 3.3 Eq. 2) and one packed factor part.  `dtype` is the part's element
 * type (PKV_BF16 rounds nearest-even).  `packed` is host memory of
 * pkv_factor_part_elems elements.  Host only.
 */
int32_t pkv_pack_factors(int32_t kind, int32_t P, int32_t d, int32_t r, int32_t dtype,
                         const float* Lf, const float* Rf, void* packed);
int32_t pkv_unpack_factors(int32_t kind, int32_t P, int32_t d, int32_t r, int32_t dtype,
                           const void* packed, float* Lf, float* Rf);

/* Bytes of one factor part (kind: any pkv_factor_kind) of rank r in
 * storage format `dtype`.  PKV_BF16 / PKV_F32: pkv_factor_part_elems
 * elements of 2 / 4 bytes.  PKV_BF16_INT4 (the INT4 part of Sec. 4.3; K and V parts differ),
 * with A = r8 / 4 codes in a rank unit of ub = A / 2 bytes (a nibble per
 * code: 1, 2, 3 or 4 bytes; 3-byte units start at any byte), and h = 1 at
 * P = 64, 2 at P = 32:
 *   K part: roundup64(r8 d / 2 + (256 / h) ub + 2 d + 2 r8)
 *           (codes of Rt_K, codes of Lt_K in units of A, scales of Rt_K, Lt_K)
 *   V part: roundup64(r8 P / 2 + 4 d ub + 2 P + 2 d)
 *           (codes of Lt_V, codes of Rt_V in units of A, scales of Lt_V, Rt_V).
 * Host only. */
int32_t pkv_factor_part_bytes(int32_t kind, int32_t P, int32_t d, int32_t r, int32_t dtype,
                              int64_t* bytes);

/*
 * Host-side conversion between one PKV_BF16_INT4 factor part (host memory of
 * pkv_factor_part_bytes bytes) and its codes and scales (Sec. 4.3):
 *   Lq [P][r] int8 codes of Lt, Rq [r][d] int8 codes of Rt, values -7..7;
 *   Ls scales of Lt: [r] (keys, per column) or [P] (values, per row);
 *   Rs [d] scales of Rt (per column).
 * Scales are float32 here and bfloat16 in the part (packing rounds
 * nearest-even).  Packing sets padding ranks to code 0, scale 0.
 * Errors: INVALID_ARG (null pointer, bad kind, r < 1, r > min(P, d), a code
 * outside -7..7), UNSUPPORTED (P not 64 or 32, d != 128, r > 32).  Host only.
 */
int32_t pkv_pack_factors_int4(int32_t kind, int32_t P, int32_t d, int32_t r, const int8_t* Lq,
                              const float* Ls, const int8_t* Rq, const float* Rs, void* packed);
int32_t pkv_unpack_factors_int4(int32_t kind, int32_t P, int32_t d, int32_t r, const void* packed,
                                int8_t* Lq, float* Ls, int8_t* Rq, float* Rs);

/* Bytes and layout of the device buffer a cache of this shape needs: the
 * preallocated dense and factor storage of Sec. 3.3 (1)-(3) and (5), laid
 * out as described at pkv_layout.  Errors: as pkv_cache_create's shape
 * checks.  Host only. */
int32_t pkv_cache_layout(const pkv_shape* shape, pkv_layout* out);

/* Create a cache over a caller-owned device buffer of at least
 * pkv_cache_layout().total_bytes bytes, 256-byte aligned.  The buffer's
 * contents are set by pkv_prefill (call it, possibly with T = 0, before
 * pkv_append or pkv_decode_step).  Host only (no GPU work). */
int32_t pkv_cache_create(const pkv_shape* shape, void* device_buffer, uint64_t device_bytes,
                         pkv_cache** out);
void pkv_cache_destroy(pkv_cache* cache);

/* Host-side state: current length T, FACT pages stored, and whether a
 * completed page waits for pkv_promote_page. */
int32_t pkv_cache_state(const pkv_cache* cache, int64_t* T, int64_t* n_fact, int32_t* pending);

/*
 * Batched page decomposition (Sec. 3.3, text after Eq. 3): for each of
 * n_pages pages X (P x d, row-major, contiguous, `in_dtype`) form the Gram
 * matrix G = X X^T in float32 on the matrix cores, take its top-r
 * eigenvectors Q in float32, and write
 *   Lf = Q diag(sigma)  (P x r),   Rf = diag(1/sigma) Q^T X  (r x d),
 *   sigma_i = || (Q^T X)_i ||,
 * so Lf Rf is the rank-r truncated SVD of X (Sec. 3.2; Eckart-Young-Mirsky).
 * The eigen-solve, one page per wavefront: r <= 32 (every 32-token page):
 * Householder reduction of G to tridiagonal form, bisection for the r
 * largest eigenvalues, one eigenvector each from a twisted factorization,
 * back-transformation, then one Cholesky QR pass that makes the r columns
 * orthonormal (and, for eigenvalues the bisection cannot tell apart, such
 * as an exactly repeated singular value, refilled columns refined by
 * orthogonal iteration); a 32-token page is solved on its own 32 x 32 Gram
 * matrix.  r > 32: cyclic Jacobi rotations of G.
 * Outputs (device, row-major, `out_dtype`): Lf [n_pages][P][r],
 * Rf [n_pages][r][d]; sigma [n_pages][r] float32 (may be NULL).  Rows with
 * sigma = 0 are zero.  Errors: INVALID_ARG (null/misaligned pointers, bad
 * r), UNSUPPORTED (P not 64 or 32, or d != 128), DEVICE (launch failure).
 */
int32_t pkv_compress_pages(const void* X, int64_t n_pages, int32_t P, int32_t d, int32_t r,
                           int32_t in_dtype, int32_t out_dtype, void* Lf, void* Rf, float* sigma,
                           void* stream);

/*
 * Prefill (Sec. 3.3 (1)-(3)): from dense K, V (device, [B][H_kv][T][d], cache
 * dtype) build the hybrid cache: copy sink, window and partial pages into the
 * dense pools, factorize every FACT page of every (sequence, KV head, K/V)
 * with the kernel of pkv_compress_pages into the factor pool, and fill the
 * page table.  Resets the cache to length T (0 <= T <= max_tokens); T = 0
 * zero-fills the dense pools and empties the table (K, V may then be NULL).
 * A cache is first used after a prefill.
 */
int32_t pkv_prefill(pkv_cache* cache, const void* K, const void* V, int64_t T, void* stream);

/*
 * Chunked prefill (Sec. 3.3 (1)-(3) and (5) applied to C tokens at once):
 * K, V (device, [B][H_kv][C][d], cache element type) are the next C tokens
 * of every sequence.  The cache grows from T to T + C and ends in the steady
 * state: every page that leaves the recent window within the chunk is
 * factorized (from its ring slot, or straight from the chunk for pages that
 * never enter the window), the remaining rows go to the dense pools, and the
 * page table is refilled.  The factor pool, the page table and every valid
 * dense row end as after C calls of pkv_append and pkv_promote_page (rows of
 * a dense slot beyond its page's valid length are unspecified).  C = 0 does
 * nothing.  All pages the call factorizes on a stream go to one launch.
 * With an auxiliary stream set (pkv_cache_set_aux_stream), one launch there,
 * ordered after the work already on `stream`, decomposes the pages
 * factorized straight from the chunk and also the window's complete pages
 * (early factorization, as pkv_append does for one page): the call returns
 * with that work overlapping whatever the caller queues next.  The next
 * attention call (pkv_decode_attn, pkv_decode_partial, pkv_decode_step) or
 * pkv_prefill on a stream orders itself after the chunk's pages; a
 * promotion or a later chunk waits for the early pages it needs.  K and V must stay unchanged until the
 * auxiliary stream has passed the call's work.
 * Errors: INVALID_ARG (C < 0, null or misaligned K / V), CAPACITY
 * (T + C > max_tokens), PROMOTION_PENDING (a completed page waits for
 * pkv_promote_page).
 */
int32_t pkv_prefill_chunk(pkv_cache* cache, const void* K, const void* V, int64_t C, void* stream);

/*
 * Append one token (Sec. 3.3 "Incremental Cache Update (5)"): k_new, v_new
 * (device, [B][H_kv][d], cache dtype) go to row T mod P of page T / P, which
 * joins attention at once; T += 1.  If this append completes a page and the
 * oldest window page must leave the window, *promotion_pending (may be NULL)
 * is set to 1 and pkv_promote_page must run before the next append.
 * Errors: CAPACITY (T == max_tokens), PROMOTION_PENDING.
 */
int32_t pkv_append(pkv_cache* cache, const void* k_new, const void* v_new,
                   int32_t* promotion_pending, void* stream);

/* Factorize the page that left the window (once; factors go to the next
 * factor slot, its ring slot is released) and mark it FACT.  At most one page
 * per call (Sec. 3.3 (5)).  Errors: NOT_ELIGIBLE when nothing is waiting. */
int32_t pkv_promote_page(pkv_cache* cache, void* stream);

/*
 * Attention for a batch of sequences of different lengths (serving batches),
 * one cache per sequence -- each with its own pools and page table, so each
 * has its own length T_i and its own page classes; the method of Sec. 3.3 (4)
 * on every cache.  caches: host array of n handles (1 <= n <= 32) of batch 1
 * whose shapes agree except max_tokens (heads, d, P, ranks, sink, window,
 * dtype, pre-RoPE setting and frequencies); each holds T_i >= 1 tokens.
 * q: device [n][H_q][d] (cache dtype), 16-byte aligned; out: device float32
 * [n][H_q][d]; query row i attends over cache i.  One partial-attention
 * launch covers every (cache, KV head, split) for the matrix-core formats
 * whose K and V ranks pad to the same multiple of 8; other formats launch
 * once per cache.  Then one merge launch.  workspace: 256-byte aligned
 * device memory of pkv_decode_batch_workspace_bytes(caches, n, n_split)
 * bytes (which also takes empty caches).  n_split > 0: every cache's range
 * is cut into n_split parts, and row i equals pkv_decode_attn on cache i
 * with that n_split bit for bit.  n_split = 0: the library gives each cache
 * splits in proportion to its pages (the workgroups of one round of the GPU
 * shared out; formats without a batched kernel use one count), and rows
 * agree with per-cache calls to fp32 rounding.
 * Errors: INVALID_ARG (null or misaligned pointers, n out of range, shapes
 * that differ, an empty cache), CAPACITY (workspace too small).
 */
int32_t pkv_decode_attn_batch(const pkv_cache* const* caches, int32_t n, const void* q, float* out,
                              void* workspace, uint64_t workspace_bytes, int32_t n_split, void* stream);
int32_t pkv_decode_batch_workspace_bytes(const pkv_cache* const* caches, int32_t n, int32_t n_split,
                                         uint64_t* bytes);

/*
 * One decode step for a batch of sequences of different lengths, one cache of
 * batch 1 per sequence (Sec. 3.3 (5) then (4) on every cache): for cache i,
 * append (k_new[i], v_new[i]), promote the page leaving its window when due,
 * and attend q[i] over its tokens including the new one -- what
 * pkv_decode_step does on each cache, with one partial-attention launch and
 * one merge (which writes every new token) for the whole batch; a promotion
 * adds one decomposition launch for its cache.
 * caches: n (1..32) handles as for pkv_decode_attn_batch; lengths may be 0.
 * k_new, v_new: device [n][H_kv][d]; q: device [n][H_q][d] (cache dtype);
 * out: device float32 [n][H_q][d]; all 16-byte aligned.  workspace: as for
 * pkv_decode_attn_batch (pkv_decode_batch_workspace_bytes before the step).
 * Every cache ends as after pkv_decode_step, and with the same n_split the
 * outputs are bit-identical to it.  Caches without a recent window step one
 * by one (their promoted page is the new token's).
 * Errors: as pkv_decode_attn_batch, PROMOTION_PENDING, CAPACITY (a cache at
 * max_tokens or without a free factor slot); nothing changes then.
 */
int32_t pkv_decode_step_batch(pkv_cache* const* caches, int32_t n, const void* k_new, const void* v_new,
                              const void* q, float* out, void* workspace, uint64_t workspace_bytes,
                              int32_t n_split, void* stream);

/* Workspace bytes pkv_decode_attn needs for n_split splits per (sequence,
 * KV head): the split-K partial states that the Eq. 5 merge combines
 * (Sec. 3.3 (4)), rows = B H_q n_split, laid out as at pkv_decode_partial:
 * roundup256(rows d 4) + roundup256(rows 2 4).  n_split = 0 selects the
 * library's choice for the cache's current length; at most 512.  Host
 * only.  Errors: INVALID_ARG (null pointers, n_split out of range). */
int32_t pkv_decode_workspace_bytes(const pkv_cache* cache, int32_t n_split, uint64_t* bytes);

/*
 * Mixed decode attention (Sec. 3.3 (4), Eq. 4 and Eq. 5): for every query
 * head, softmax(q K^T / sqrt(d)) V over all T cached tokens, where factorized
 * pages are evaluated through their factors (scores (q Rf_K^T) Lf_K^T, output
 * (e^(s-m) Lf_V) Rf_V) without reconstructing them, dense pages directly, and
 * page-wise partial states are merged by online softmax within each split
 * and then across splits.  Equivalent to pkv_decode_partial followed by
 * pkv_decode_merge on the same stream.
 * q: device [B][H_q][d] (cache dtype), 16-byte aligned; out: device float32
 * [B][H_q][d], 16-byte aligned; workspace: device, 256-byte aligned, at least
 * pkv_decode_workspace_bytes(n_split) bytes (no initialization needed; calls
 * that share one workspace must not overlap).
 * Errors: INVALID_ARG (T == 0, null or misaligned pointers, n_split > 512),
 * CAPACITY (workspace too small).
 */
int32_t pkv_decode_attn(const pkv_cache* cache, const void* q, float* out, void* workspace,
                        uint64_t workspace_bytes, int32_t n_split, void* stream);

/*
 * First half of pkv_decode_attn: the page-wise states of Eq. 4, already
 * merged within each of n_split page ranges per (sequence, KV head).  Writes
 * to the workspace, per row = (b * H_q + h) * n_split + split:
 *   float o[row][d]        at byte 0 (unnormalized sum of e^(s-m) v),
 *   float (m, l)[row][2]   at byte align256(B * H_q * n_split * d * 4),
 * with m in log2 units (scores are scaled by log2(e)/sqrt(d)) and an empty
 * range reported as m = -inf, l = 0, o = 0.  These are the states a
 * context-parallel shard would exchange before the Eq. 5 merge.
 */
int32_t pkv_decode_partial(const pkv_cache* cache, const void* q, void* workspace,
                           uint64_t workspace_bytes, int32_t n_split, void* stream);

/* Second half: the Eq. 5 merge of the n_split partial states of every
 * (sequence, query head) in the workspace into the normalized float32
 * output out [B][H_q][d] (16-byte aligned). */
int32_t pkv_decode_merge(const pkv_cache* cache, const void* workspace, uint64_t workspace_bytes,
                         int32_t n_split, float* out, void* stream);

/* Copy the page table (the page classes and slots of Sec. 3.3 (1)-(3) and
 * (5), as pkv_classify describes them) to host: cls[p], slot[p] for p < n
 * (n <= max_pages).  Synchronizes `stream`.  Errors: INVALID_ARG (null
 * pointers, n < 0 or n > max_pages), DEVICE. */
int32_t pkv_read_page_table(const pkv_cache* cache, int32_t* cls, int32_t* slot, int64_t n,
                            void* stream);

/*
 * One decode step of a layer: PuzzleKV Sec. 3.3 (5) then (4) -- append the
 * new token's key and value (k_new, v_new: [B][H_kv][d] in the cache dtype,
 * 16-byte aligned), factorize the page that leaves the recent window when this
 * token completes a page (as pkv_promote_page), then the mixed attention of q
 * over all T + 1 tokens into out [B][H_q][d] float32, as pkv_decode_attn.
 * The cache afterwards is byte-identical to that of pkv_append +
 * pkv_promote_page (when due) + pkv_decode_attn; the output agrees with theirs
 * to float32 rounding.  The append costs no launch of its own: attention runs
 * over the T cached tokens, and the cross-split merge adds the new token's
 * state (score q.k_new / sqrt(d), weight 1, value v_new) beside the split
 * states (Eq. 5) and writes the token into its dense page.  With w = 0 the
 * completed page is factorized in the same step, so there the token is
 * appended by a launch of its own first.
 * workspace: at least pkv_decode_workspace_bytes for the length after the
 * append (any length up to max_tokens when sized for n_split = 512).  T
 * advances by one on success.
 * Errors: INVALID_ARG (null or misaligned pointers), CAPACITY (T ==
 * max_tokens, no free factor slot, workspace too small), PROMOTION_PENDING
 * (a promotion from pkv_append is still waiting); nothing is changed then.
 */
int32_t pkv_decode_step(pkv_cache* cache, const void* k_new, const void* v_new, const void* q,
                        float* out, void* workspace, uint64_t workspace_bytes, int32_t n_split,
                        void* stream);

/*
 * Early page factorization for pkv_decode_step (Sec. 3.3 (5): a page is
 * factorized once, when it leaves the recent window; its factors depend only
 * on the page's own tokens, which are final once the page is complete).
 * aux_stream: a second hipStream_t (as void*) of the caller, at default
 * priority, that outlives the cache's use of it.  When set, the step whose
 * token completes a window page enqueues that page's factorization on
 * aux_stream, ordered after the step's own work on its stream; the step at
 * which the page leaves the window (w / P pages later) makes its stream wait
 * for that factorization and flips the table entry.  The factorization thus
 * overlaps later decode steps instead of lengthening one.  Outputs and cache
 * contents are identical to those without it.  NULL (the default) turns it
 * off.  Creates and owns a few hipEvents (no device memory).
 * Errors: UNSUPPORTED (more than 64 window ring slots), PROMOTION_PENDING
 * (changing or clearing the stream while early factorizations are
 * outstanding), DEVICE.
 */
int32_t pkv_cache_set_aux_stream(pkv_cache* cache, void* aux_stream);

/*
 * Pre-RoPE keys (App. D.3 "RoPE Key Analysis" compares factorizing keys
 * before and after the rotary position embedding): from this call on, the
 * keys given to pkv_prefill, pkv_prefill_chunk, pkv_append and
 * pkv_decode_step are taken as pre-RoPE.  They are stored and factorized as
 * given, and the attention calls rotate every key, dense or reconstructed
 * from its factors, at its position t (its token index in the cache) before
 * the scores.  Channel pair (m, m + d/2) turns by the angle t * inv_freq[m]
 * (the pairing of the Llama and Qwen checkpoints); the angle is reduced in
 * double precision, so positions up to max_tokens keep full accuracy.  The
 * query is taken as already rotated at its own position.  Key parts then
 * use the PKV_KEYS_PRE_ROPE layout.
 * inv_freq: host, n_freq = d/2 finite float32 frequencies, copied; NULL
 * turns pre-RoPE keys off.  Only on an empty cache (length 0: after
 * pkv_cache_create or a pkv_prefill with T = 0).
 * Errors: INVALID_ARG (null cache, n_freq != d/2, a non-finite frequency, a
 * non-empty cache), UNSUPPORTED (PKV_BF16_INT4 caches).
 */
int32_t pkv_cache_set_key_rope(pkv_cache* cache, const float* inv_freq, int32_t n_freq);

/*
 * pkv_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as pkv_decode_attn (bit-identical output for the
 * same n_split), but the split partials go to a workspace the library holds:
 * one array of PKV_NOALLOC_WORKSPACE_BYTES per device, in the library's
 * device image, kept until the process ends.  The call allocates and frees
 * nothing, and the workspace needs no clearing (the partial kernel writes
 * every state the merge reads).  Every call on one device shares that
 * device's array, so calls that overlap on one device (two streams, two
 * host threads) race; calls in stream order do not.  The first call on a
 * device looks the array's address up once (hipGetSymbolAddress).
 * Errors: as pkv_decode_attn; CAPACITY when pkv_decode_workspace_bytes for
 * n_split exceeds PKV_NOALLOC_WORKSPACE_BYTES (checked before any device
 * call); DEVICE if the lookup fails.
 */
#define PKV_NOALLOC_WORKSPACE_BYTES (16ull << 20)
int32_t pkv_decode_attn_noalloc(const pkv_cache* cache, const void* q, float* out, int32_t n_split,
                                void* stream);

/* Kernel timing (measurement only; no passage of the method).
 *
 * start_event, stop_event: hipEvent_t handles (as void*) that the caller
 * created with timing enabled and owns.  The next launch, on this host thread,
 * of a decode-partial kernel (pkv_decode_partial, pkv_decode_attn) or of a
 * page-decomposition kernel (pkv_compress_pages, pkv_prefill,
 * pkv_promote_page) records start_event when that kernel begins executing
 * and stop_event when it ends, so hipEventElapsedTime gives the kernel's own
 * duration without the launch gaps around it.  The request is then cleared;
 * a call that launches no such kernel leaves it pending.  Both NULL clears a
 * pending request.  Not for use under stream capture.
 * Errors: PKV_ERR_INVALID_ARG if exactly one handle is NULL (nothing set). */
int32_t pkv_time_next_kernel(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
