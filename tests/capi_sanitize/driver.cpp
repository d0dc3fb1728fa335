// Host-side driver for the sanitizer build of the C ABI: calls every entry
// point with arguments that its host validation must reject (or accept as
// empty) before anything reaches the device, so it runs without a GPU. Built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code of
// locks_capi.hip; any report, or a status other than the expected one,
// fails the run. Device pointers here are fake and never dereferenced.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "locks.h"

static int g_fail = 0;
#define EXPECT_EQ(a, b)                                                                    \
  do {                                                                                     \
    const long long va_ = (long long)(a), vb_ = (long long)(b);                            \
    if (va_ != vb_) {                                                                      \
      std::fprintf(stderr, "FAIL line %d: %s = %lld, expected %lld\n", __LINE__, #a, va_, vb_); \
      ++g_fail;                                                                            \
    }                                                                                      \
  } while (0)

int main() {
  void* fake = reinterpret_cast<void*>(uintptr_t{256});
  void* odd = reinterpret_cast<void*>(uintptr_t{264});  // 8-byte but not 16-byte aligned
  auto I = [&](void* p) { return static_cast<int32_t*>(p); };
  auto F = [&](void* p) { return static_cast<float*>(p); };
  locks_dims d{128, 16, 8, 8, 4};
  locks_dims bad_g{128, 16, 8, 8, 3};
  locks_dims bad_r{128, 16, 17, 8, 4};
  locks_dims bad_d{64, 16, 8, 8, 4};
  locks_dims zero_h{128, 16, 8, 0, 4};

  // sizes
  EXPECT_EQ(locks_summary_slot_bytes(&d), 818);
  EXPECT_EQ(locks_summary_slot_stride(&d), 896);
  EXPECT_EQ(locks_summary_slot_bytes(nullptr), 0);
  EXPECT_EQ(locks_summary_slot_bytes(&bad_r), 0);
  EXPECT_EQ(locks_summary_slot_stride(&bad_d), 0);
  EXPECT_EQ(locks_workspace_bytes(&d, 1, 8192, 1), 0);
  EXPECT_EQ(locks_workspace_bytes(&d, -1, 8192, 128), 0);
  EXPECT_EQ(locks_workspace_bytes(&d, 1, 1 << 17, 128), 0);
  EXPECT_EQ(locks_workspace_bytes(&zero_h, 1, 8192, 128), 0);
  // large but valid shapes: the size arithmetic must not overflow
  const size_t big = locks_workspace_bytes(&d, INT_MAX, 65536, 2048);
  if (big == 0 || big < (size_t)INT_MAX * 8 * 65536) {
    std::fprintf(stderr, "FAIL: workspace size for INT_MAX sequences: %zu\n", big);
    ++g_fail;
  }
  // per-head selection: the workspace of one query head per KV head-like row
  locks_dims dph{128, 16, 8, 8, 4, 0, LOCKS_MERGE_PER_HEAD};
  locks_dims dview{128, 16, 8, 32, 1, 0, LOCKS_MERGE_SHARE};
  locks_dims dbadrule{128, 16, 8, 8, 4, 0, LOCKS_MERGE_PER_HEAD + 1};
  locks_dims dhuge{128, 16, 8, INT_MAX / 2, 4, 0, LOCKS_MERGE_PER_HEAD};
  EXPECT_EQ(locks_workspace_bytes(&dph, 2, 2048, 64), locks_workspace_bytes(&dview, 2, 2048, 64));
  EXPECT_EQ(locks_workspace_bytes(&dbadrule, 2, 2048, 64), 0);
  EXPECT_EQ(locks_workspace_bytes(&dhuge, 1, 2048, 64), 0);
  for (int32_t s = -5; s <= 1; ++s)
    if (!locks_status_string(s) || !std::strlen(locks_status_string(s))) ++g_fail;
  if (std::strcmp(locks_status_string(INT_MIN), "unknown status") != 0) ++g_fail;

  // build / build_filled / append
  EXPECT_EQ(locks_build(&d, fake, 16, I(fake), -1, fake, nullptr), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_build(&d, nullptr, 16, I(fake), 4, fake, nullptr), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_build(&bad_g, fake, 16, I(fake), 4, fake, nullptr), LOCKS_ERR_UNSUPPORTED);
  EXPECT_EQ(locks_build(&d, fake, 0, I(fake), 4, fake, nullptr), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_build(&d, fake, 16, I(fake), 0, fake, nullptr), LOCKS_OK);
  EXPECT_EQ(locks_build(&d, odd, 16, I(fake), 4, fake, nullptr), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_build(nullptr, fake, 16, I(fake), 4, fake, nullptr), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_build_filled(&d, fake, 16, I(fake), I(fake), -2, 8, fake, nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_build_filled(&d, fake, 16, I(fake), I(fake), 0, 8, fake, nullptr), LOCKS_OK);
  EXPECT_EQ(locks_append_kv(&d, nullptr, fake, fake, fake, 16, I(fake), I(fake), 1, 8, nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_append_kv(&d, fake, fake, fake, fake, 16, I(fake), I(fake), 1, 0, nullptr),
            LOCKS_ERR_INVALID_ARG);

  // score / select / attention
  const size_t ws1 = locks_workspace_bytes(&d, 1, 8, 4);
  EXPECT_EQ(locks_score_select(&d, fake, fake, 16, I(fake), I(fake), I(fake), 1, 8, 1, I(fake),
                               I(fake), nullptr, fake, ws1, nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_score_select(&d, fake, fake, 16, I(fake), I(fake), I(fake), 1, 8, 4, nullptr,
                               I(fake), nullptr, fake, ws1, nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_score_select(&d, fake, fake, 16, I(fake), I(fake), I(fake), 1, 8, 4, I(fake),
                               I(fake), nullptr, fake, ws1 - 1, nullptr),
            LOCKS_ERR_WORKSPACE);
  EXPECT_EQ(locks_score_select(&d, fake, fake, 16, I(fake), I(fake), I(fake), 0, 8, 4, I(fake),
                               I(fake), nullptr, fake, ws1, nullptr),
            LOCKS_OK);
  EXPECT_EQ(locks_score_pages(&d, fake, fake, 16, I(fake), I(fake), 1, 70000, F(fake), nullptr),
            LOCKS_ERR_UNSUPPORTED);
  EXPECT_EQ(locks_score_pages(&d, odd, fake, 16, I(fake), I(fake), 1, 8, F(fake), nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_select_pages(&d, F(fake), I(fake), I(fake), 1, 8, 4, I(fake), I(fake), fake,
                               ws1 - 1, nullptr),
            LOCKS_ERR_WORKSPACE);
  EXPECT_EQ(locks_select_pages(&d, nullptr, I(fake), I(fake), 1, 8, 4, I(fake), I(fake), fake,
                               ws1, nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_sparse_attn(&d, fake, fake, fake, 16, I(fake), I(fake), I(fake), I(fake), 1, 8,
                              4, nullptr, nullptr, fake, ws1, nullptr),
            LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_sparse_attn(&d, fake, fake, fake, 16, I(fake), I(fake), I(fake), I(fake), 1, 8,
                              4, F(fake), nullptr, fake, 8, nullptr),
            LOCKS_ERR_WORKSPACE);

  // decode step: every rejection happens before a launch (a 17000-page table
  // takes the separate launches; a workspace one byte short is rejected)
  locks_dims d2{128, 16, 8, 2, 4};
  const int32_t host_lens[2] = {17000 * 16 - 3, 300};
  const size_t need = locks_workspace_bytes(&d2, 2, 17000, 64);
  auto step = [&](const void* k_new, float* out, int32_t* sel, int32_t* cnt, int32_t MP,
                  int32_t KB, uint32_t flags, void* ws, size_t wsb) {
    return locks_decode_step(&d2, fake, k_new, fake, fake, fake, fake, 40000, I(fake), I(fake),
                             host_lens, I(fake), 2, MP, KB, out, nullptr, sel, cnt, flags, ws, wsb,
                             nullptr);
  };
  EXPECT_EQ(step(fake, F(fake), nullptr, nullptr, 17000, 64, 0, fake, need - 1), LOCKS_ERR_WORKSPACE);
  EXPECT_EQ(step(fake, F(fake), nullptr, nullptr, 17000, 64, 0, nullptr, need), LOCKS_ERR_WORKSPACE);
  EXPECT_EQ(step(fake, F(fake), I(fake), nullptr, 17000, 64, 0, fake, need), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(step(fake, nullptr, nullptr, nullptr, 17000, 64, 0, fake, need), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(step(odd, F(fake), nullptr, nullptr, 17000, 64, 0, fake, need), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(step(fake, F(fake), nullptr, nullptr, 70000, 64, 0, fake, need), LOCKS_ERR_UNSUPPORTED);
  EXPECT_EQ(step(fake, F(fake), nullptr, nullptr, 17000, 1, 0, fake, need), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(step(fake, F(fake), nullptr, nullptr, 17000, 64, 2, fake, need), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_decode_step(&d2, fake, fake, fake, fake, fake, fake, 40000, I(fake), I(fake),
                              host_lens, I(fake), 0, 8, 4, F(fake), nullptr, nullptr, nullptr, 0,
                              nullptr, 0, nullptr),
            LOCKS_OK);
  // the no-allocation variant: a shape beyond its built-in scratch
  const int32_t host_lens8[8] = {16, 16, 16, 16, 16, 16, 16, 16};
  EXPECT_EQ(locks_decode_step_noalloc(&d2, fake, fake, fake, fake, fake, fake, 40000, I(fake),
                                      I(fake), host_lens8, I(fake), 8, 65536, 2048, F(fake),
                                      nullptr, nullptr, nullptr, 0, nullptr),
            LOCKS_ERR_WORKSPACE);
  EXPECT_EQ(locks_decode_step_noalloc(&d2, fake, fake, fake, fake, fake, fake, 40000, I(fake),
                                      I(fake), host_lens, I(fake), 2, 64, 8, F(fake), nullptr,
                                      nullptr, nullptr, 4, nullptr),
            LOCKS_ERR_INVALID_ARG);

  // host pool: argument errors only (no allocation without a device)
  void *hp = nullptr, *dp = nullptr;
  EXPECT_EQ(locks_host_pool_alloc(0, &hp, &dp), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_host_pool_alloc(4096, nullptr, &dp), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_host_pool_alloc(4096, &hp, nullptr), LOCKS_ERR_INVALID_ARG);
  EXPECT_EQ(locks_host_pool_free(nullptr), LOCKS_OK);

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("capi sanitizer driver: all checks passed\n");
  return 0;
}
