// Host logic of the C-ABI under AddressSanitizer / UndefinedBehaviorSanitizer
// (test infrastructure): classification sweeps, every packed-part format's
// pack / unpack round trip, layouts, and the argument and state checks of
// every call that touches no device.  Exit status 0 when every check holds.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pkv.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static uint32_t rng_state = 12345u;
static float frand() {
  rng_state = rng_state * 1664525u + 1013904223u;
  return ((rng_state >> 8) & 0xffff) / 32768.f - 1.f;
}

int main() {
  const int P = 64, d = 128;
  for (int st = 0; st <= 7; ++st) CHECK(pkv_status_string(st) != nullptr);
  CHECK(pkv_version() != nullptr);

  // classification: every length up to 40 pages, a few sink / window sizes
  std::vector<int32_t> cls(4096), slot(4096);
  for (int s = 0; s <= 128; s += 64)
    for (int w = 0; w <= 192; w += 64)
      for (int64_t T = 0; T <= 64 * 40; T += 7) {
        const int64_t n = (T + P - 1) / P;
        CHECK(pkv_classify(T, P, s, w, -1, cls.data(), slot.data(), n) == 0);
      }
  CHECK(pkv_classify(100, P, 10, 64, -1, cls.data(), slot.data(), 2) != 0);  // s not a multiple of P

  // packed parts: every kind, element type and rank round-trips
  for (int r = 1; r <= 64; ++r) {
    std::vector<float> Lf(P * r), Rf(r * d), L2(P * r), R2(r * d);
    for (auto& x : Lf) x = frand();
    for (auto& x : Rf) x = frand();
    for (int kind = 0; kind <= 2; ++kind) {
      int64_t elems = 0;  // (value parts: Rf at the even-rounded rank)
      CHECK(pkv_factor_part_elems(kind, P, d, r, &elems) == 0);
      std::vector<float> packed(elems);
      CHECK(pkv_pack_factors(kind, P, d, r, PKV_F32, Lf.data(), Rf.data(), packed.data()) == 0);
      CHECK(pkv_unpack_factors(kind, P, d, r, PKV_F32, packed.data(), L2.data(), R2.data()) == 0);
      CHECK(std::memcmp(Lf.data(), L2.data(), Lf.size() * 4) == 0);
      CHECK(std::memcmp(Rf.data(), R2.data(), Rf.size() * 4) == 0);
      std::vector<uint16_t> pb(elems);
      CHECK(pkv_pack_factors(kind, P, d, r, PKV_BF16, Lf.data(), Rf.data(), pb.data()) == 0);
      CHECK(pkv_unpack_factors(kind, P, d, r, PKV_BF16, pb.data(), L2.data(), R2.data()) == 0);
      for (size_t i = 0; i < Lf.size(); ++i) CHECK(std::fabs(L2[i] - Lf[i]) <= std::fabs(Lf[i]) * 0.004f);
      int64_t bytes = 0;
      CHECK(pkv_factor_part_bytes(kind, P, d, r, PKV_BF16, &bytes) == 0 && bytes == elems * 2);
    }
    if (r <= 32) {
      for (int kind = 0; kind <= 1; ++kind) {
        int64_t qb = 0;
        CHECK(pkv_factor_part_bytes(kind, P, d, r, PKV_BF16_INT4, &qb) == 0);
        std::vector<int8_t> Lq(P * r), Rq(r * d), Lq2(P * r), Rq2(r * d);
        std::vector<float> Ls(kind == 0 ? r : P), Rs(d), Ls2(Ls.size()), Rs2(d);
        for (auto& c : Lq) c = (int8_t)((rng_state = rng_state * 1664525u + 1013904223u) % 15) - 7;
        for (auto& c : Rq) c = (int8_t)((rng_state = rng_state * 1664525u + 1013904223u) % 15) - 7;
        for (auto& x : Ls) x = 0.25f;
        for (auto& x : Rs) x = 0.5f;
        std::vector<uint8_t> part(qb);
        CHECK(pkv_pack_factors_int4(kind, P, d, r, Lq.data(), Ls.data(), Rq.data(), Rs.data(), part.data()) == 0);
        CHECK(pkv_unpack_factors_int4(kind, P, d, r, part.data(), Lq2.data(), Ls2.data(), Rq2.data(), Rs2.data()) ==
              0);
        CHECK(Lq == Lq2 && Rq == Rq2 && Ls == Ls2 && Rs == Rs2);
      }
      int64_t qb = 0;
      CHECK(pkv_factor_part_bytes(PKV_KEYS_PRE_ROPE, P, d, r, PKV_BF16_INT4, &qb) == PKV_ERR_UNSUPPORTED);
    }
  }

  // layouts and caches over a fake device address: every call below fails
  // its checks (or needs no device) before any launch
  for (int dtype = 0; dtype <= 2; ++dtype) {
    pkv_shape sh{};
    sh.batch = 2;
    sh.n_q_heads = 8;
    sh.n_kv_heads = 2;
    sh.head_dim = d;
    sh.page_len = P;
    sh.rank_k = 24;
    sh.rank_v = 16;
    sh.sink = 64;
    sh.window = 128;
    sh.max_tokens = 4096;
    sh.dtype = dtype;
    pkv_layout lay{};
    CHECK(pkv_cache_layout(&sh, &lay) == 0);
    void* fake = (void*)(uintptr_t)(256 * 1000);
    pkv_cache* c = nullptr;
    CHECK(pkv_cache_create(&sh, fake, lay.total_bytes - 1, &c) != 0);
    CHECK(pkv_cache_create(&sh, fake, lay.total_bytes, &c) == 0 && c);
    int64_t T = -1, nf = -1;
    int32_t pend = -1;
    CHECK(pkv_cache_state(c, &T, &nf, &pend) == 0 && T == 0 && nf == 0 && pend == 0);
    std::vector<float> f(d / 2, 0.01f);
    CHECK(pkv_cache_set_key_rope(c, f.data(), d / 2) == (dtype == PKV_BF16_INT4 ? PKV_ERR_UNSUPPORTED : 0));
    CHECK(pkv_cache_set_key_rope(c, nullptr, 0) == (dtype == PKV_BF16_INT4 ? PKV_ERR_UNSUPPORTED : 0));
    void* p16 = (void*)(uintptr_t)(256 * 5000);
    CHECK(pkv_prefill(c, p16, p16, 4097, nullptr) == PKV_ERR_CAPACITY);
    CHECK(pkv_prefill_chunk(c, p16, p16, -1, nullptr) == PKV_ERR_INVALID_ARG);
    CHECK(pkv_prefill_chunk(c, p16, p16, 4097, nullptr) == PKV_ERR_CAPACITY);
    CHECK(pkv_promote_page(c, nullptr) == PKV_ERR_NOT_ELIGIBLE);
    uint64_t wsb = 0;
    CHECK(pkv_decode_workspace_bytes(c, 600, &wsb) == PKV_ERR_INVALID_ARG);
    CHECK(pkv_decode_attn(c, p16, (float*)p16, p16, 1 << 20, 0, nullptr) == PKV_ERR_INVALID_ARG);  // empty
    const pkv_cache* cs[2] = {c, c};
    CHECK(pkv_decode_batch_workspace_bytes(cs, 2, 0, &wsb) == PKV_ERR_INVALID_ARG);  // batch 2 caches
    pkv_shape sh1 = sh;
    sh1.batch = 1;
    pkv_layout lay1{};
    pkv_cache* c1 = nullptr;
    CHECK(pkv_cache_layout(&sh1, &lay1) == 0 && pkv_cache_create(&sh1, fake, lay1.total_bytes, &c1) == 0);
    const pkv_cache* cs1[2] = {c1, c1};
    CHECK(pkv_decode_batch_workspace_bytes(cs1, 2, 0, &wsb) == 0 && wsb > 0);
    CHECK(pkv_decode_attn_batch(cs1, 2, p16, (float*)p16, p16, wsb, 0, nullptr) == PKV_ERR_INVALID_ARG);  // empty
    pkv_cache* ms1[2] = {c1, c1};
    CHECK(pkv_decode_step_batch(ms1, 2, p16, p16, p16, (float*)p16, p16, 16, 0, nullptr) == PKV_ERR_CAPACITY);
    pkv_cache_destroy(c1);
    CHECK(pkv_cache_set_aux_stream(c, nullptr) == 0);
    pkv_cache_destroy(c);
  }
  if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
  else std::printf("host driver: all checks passed\n");
  return failures ? 1 : 0;
}
