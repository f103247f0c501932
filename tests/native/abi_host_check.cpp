// Host-side exercise of libsparge's C ABI for a sanitizer build (AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code of api.cpp and noalloc.hip):
// every rejection path of every entry point with plausible and implausible
// arguments, the host helpers over many shapes (the token permutation writes
// into exactly-sized heap arrays, so an overrun is reported), and the status
// strings. No call here reaches a kernel launch. Exit status 0 = all as expected.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <memory>
#include <vector>

#include "../../include/sparge.h"

static int bad = 0;
#define EXPECT(expr, want)                                                              \
  do {                                                                                  \
    const long got_ = static_cast<long>(expr);                                          \
    if (got_ != static_cast<long>(want)) {                                              \
      std::fprintf(stderr, "line %d: %s = %ld, want %ld\n", __LINE__, #expr, got_, static_cast<long>(want)); \
      ++bad;                                                                            \
    }                                                                                   \
  } while (0)

int main() {
  // status strings: every code, and unknown ones
  for (int c = -12; c <= 2; ++c)
    if (!sparge_status_string(c)) ++bad;
  // top-k counts over many block counts and fractions
  int64_t k = 0;
  for (int64_t kb : {1, 2, 3, 10, 278, 512, 1182, 1861, 12288})
    for (int t = 1; t <= 1000; ++t) {
      EXPECT(sparge_topk_count(kb, t / 1000.0, &k), SPARGE_OK);
      if (k < 1 || k > kb) ++bad;
    }
  EXPECT(sparge_topk_count(10, std::nan(""), &k), SPARGE_ERR_TOPK);
  EXPECT(sparge_topk_count(10, 0.5, nullptr), SPARGE_ERR_NULL);
  EXPECT(sparge_topk_count(-1, 0.5, &k), SPARGE_ERR_ARG);
  // workspace sizes, including the overflow guards
  const int64_t big = int64_t(1) << 45;
  EXPECT(sparge_workspace_bytes(big, big, big, 128, 0.5), 0);
  EXPECT(sparge_workspace_bytes(1, 1, std::numeric_limits<int64_t>::max(), 128, 0.5), 0);
  EXPECT(sparge_workspace_bytes(1, 40, 75600, 128, 0.3) > 0, 1);
  EXPECT(sparge_workspace_bytes(1, 1, 100, 96, 0.3), 0);

  // token permutations into exactly-sized arrays
  const int64_t grids[][4] = {{0, 21, 45, 80}, {226, 13, 30, 45}, {256, 33, 45, 80}, {3, 1, 1, 1},
                              {0, 5, 9, 14}, {17, 4, 10, 12}, {0, 1, 1, 70000}};
  const int64_t cube[3] = {4, 4, 4}, odd[3] = {3, 5, 7};
  for (const auto& gr : grids)
    for (int layout : {SPARGE_LAYOUT_RASTER, SPARGE_LAYOUT_CUBE, SPARGE_LAYOUT_MORTON})
      for (const int64_t* c : {cube, odd}) {
        const int64_t n = gr[0] + gr[1] * gr[2] * gr[3];
        std::unique_ptr<int32_t[]> perm(new int32_t[n]);
        EXPECT(sparge_token_permutation(gr[0], gr[1], gr[2], gr[3], layout, c, perm.get()), SPARGE_OK);
        std::vector<char> seen(static_cast<size_t>(n), 0);
        for (int64_t i = 0; i < n; ++i) {
          if (perm[i] < 0 || perm[i] >= n || seen[perm[i]]) { ++bad; break; }
          seen[perm[i]] = 1;
        }
      }
  int32_t one = 0;
  EXPECT(sparge_token_permutation(-1, 1, 1, 1, SPARGE_LAYOUT_CUBE, cube, &one), SPARGE_ERR_ARG);
  EXPECT(sparge_token_permutation(0, 1, 1, 1, 7, cube, &one), SPARGE_ERR_ARG);
  EXPECT(sparge_token_permutation(0, 1, 1, 1, SPARGE_LAYOUT_CUBE, nullptr, &one), SPARGE_ERR_ARG);
  EXPECT(sparge_token_permutation(0, big, big, big, SPARGE_LAYOUT_RASTER, cube, &one), SPARGE_ERR_ARG);
  EXPECT(sparge_token_permutation(0, 1, 1, 1, SPARGE_LAYOUT_RASTER, cube, nullptr), SPARGE_ERR_NULL);

  // entry points: fake, well separated, aligned device addresses (never dereferenced:
  // every call below is rejected before any HIP call)
  auto P = [](uint64_t gib) { return reinterpret_cast<uint16_t*>(gib << 30); };
  uint16_t *q = P(1), *kk = P(2), *v = P(3), *o = P(4);
  void* ws = P(5);
  uint8_t* mask = reinterpret_cast<uint8_t*>(P(6));
  const int64_t H = 2, N = 256, D = 64;
  const int64_t st[3] = {H * N * D, N * D, D};
  const int64_t st_bad[3] = {H * N * D, N * D, 60};
  const int64_t st_neg[3] = {-8, N * D, D};
  const int64_t st_ovl[3] = {H * N * D, N * D, 32};
  const int64_t st_huge[3] = {H * N * D, N * D, (int64_t(1) << 24) + 8};
  for (int checked = 0; checked < 2; ++checked) {
    auto bsa = [&](const uint16_t* qq, uint16_t* oo, const int64_t* s, int64_t n, int64_t d, const uint8_t* m,
                   void* w, size_t wb, int causal) {
      return checked ? block_sparse_attn_checked(qq, kk, v, m, oo, 1, H, n, d, s, st, st, st, 0.f, causal, w, wb, nullptr)
                     : block_sparse_attn(qq, kk, v, m, oo, 1, H, n, d, s, st, st, st, 0.f, causal, w, wb, nullptr);
    };
    const size_t need = sparge_workspace_bytes(1, H, N, D, -1.0);
    EXPECT(bsa(nullptr, o, st, N, D, mask, ws, need, 0), SPARGE_ERR_NULL);
    EXPECT(bsa(q, o, st, 0, D, mask, ws, need, 0), SPARGE_ERR_SHAPE);
    EXPECT(bsa(q, o, st, N, 80, mask, ws, need, 0), SPARGE_ERR_SHAPE);
    EXPECT(bsa(q, o, st_bad, N, D, mask, ws, need, 0), SPARGE_ERR_STRIDE);
    EXPECT(bsa(q, o, st_neg, N, D, mask, ws, need, 0), SPARGE_ERR_STRIDE);
    EXPECT(bsa(q, o, st_huge, N, D, mask, ws, need, 0), SPARGE_ERR_STRIDE);
    EXPECT(bsa(q, o, st, N, D, mask, ws, need, 2), SPARGE_ERR_ARG);
    EXPECT(bsa(q, q + 64, st, N, D, mask, ws, need, 0), SPARGE_ERR_ALIAS);
    EXPECT(bsa(q, o, st, N, D, mask, nullptr, need, 0), SPARGE_ERR_WORKSPACE);
    EXPECT(bsa(q, o, st, N, D, mask, ws, need - 1, 0), SPARGE_ERR_WORKSPACE);
    EXPECT(bsa(q, o, st, N, D, reinterpret_cast<uint8_t*>(o) + 64, ws, need, 0), SPARGE_ERR_ALIAS);
  }
  EXPECT(sparge_attn_from_list(q, kk, v, reinterpret_cast<int32_t*>(ws), nullptr, 4, o, 1, H, N, D, st, st, st,
                               st, 0.f, 0, nullptr), SPARGE_ERR_NULL);
  EXPECT(sparge_attn_from_list(q, kk, v, nullptr, nullptr, 0, o, 1, H, N, D, st, st_ovl, st, st, 0.f, 0,
                               nullptr), SPARGE_ERR_STRIDE);
  EXPECT(sparge_attn_topk(q, kk, v, 0.5, o, 1, H, N, D, st, st, st, st, 0.f, 0, nullptr, ws, 16, nullptr),
         SPARGE_ERR_WORKSPACE);
  EXPECT(sparge_attn_topk(q, kk, v, 1.5, o, 1, H, N, D, st, st, st, st, 0.f, 0, nullptr, ws, 1 << 30, nullptr),
         SPARGE_ERR_TOPK);
  EXPECT(sparge_attn_cdf(q, kk, v, 0.0, o, 1, H, N, D, st, st, st, st, 0.f, 0, nullptr, ws, 1 << 30, nullptr),
         SPARGE_ERR_TOPK);
  EXPECT(sparge_attn_topk_noalloc(q, kk, v, 0.5, o, 1, H, N, D, st, st, st, st, 0.f, 0,
                                  reinterpret_cast<uint8_t*>(q) + 64, nullptr), SPARGE_ERR_ALIAS);
  const int64_t s40[3] = {40 * 75600 * 128, 75600 * 128, 128};
  EXPECT(sparge_attn_topk_noalloc(P(1), P(2), P(3), 0.95, P(4), 1, 40, 75600, 128, s40, s40, s40, s40, 0.f, 0,
                                  nullptr, nullptr), SPARGE_ERR_SCRATCH_LIMIT);
  EXPECT(sparge_pool_blocks(q, 1, H, N, D, st, 96, reinterpret_cast<float*>(o), nullptr), SPARGE_ERR_ARG);
  EXPECT(sparge_predict_mask(reinterpret_cast<float*>(q), reinterpret_cast<float*>(kk), 1, H, 786433, D, 0.5,
                             0.f, 0, nullptr, reinterpret_cast<int32_t*>(v), reinterpret_cast<int32_t*>(o),
                             nullptr), SPARGE_ERR_SHAPE);
  EXPECT(sparge_predict_mask_cdf(reinterpret_cast<float*>(q), reinterpret_cast<float*>(kk), 1, H, N, D, 0.5, 0.f,
                                 3, nullptr, reinterpret_cast<int32_t*>(v), reinterpret_cast<int32_t*>(o),
                                 nullptr), SPARGE_ERR_ARG);
  EXPECT(sparge_compact_mask(mask, 1, H, N, reinterpret_cast<int32_t*>(mask) + 1, reinterpret_cast<int32_t*>(o),
                             nullptr), SPARGE_ERR_ALIAS);
  EXPECT(sparge_check_mask(mask, 1, H, N, nullptr, 4096, nullptr), SPARGE_ERR_WORKSPACE);
  EXPECT(sparge_check_mask(mask, 1, H, N, mask, 4096, nullptr), SPARGE_ERR_ALIAS);
  EXPECT(sparge_permute_tokens(q, reinterpret_cast<int32_t*>(ws), o, 1, H, N, D, st, st, 5, nullptr),
         SPARGE_ERR_ARG);
  std::printf("abi host checks: %d unexpected results\n", bad);
  return bad ? 1 : 0;
}
