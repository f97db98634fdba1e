// Drives the C-ABI front end (api.cpp + plan.cpp, launchers stubbed) under
// host sanitizers: valid calls reach the launcher, invalid ones are rejected
// before it, extreme sizes do not overflow, and the error message is per
// thread (two threads failing with different messages at once).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <thread>

#include "../../include/crattn.h"

extern int g_launches;

static void *const FAKE = reinterpret_cast<void *>(uintptr_t(1) << 20);
static int failures = 0;

#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static int attn(int64_t cap, int64_t kv, int64_t pos0, int64_t L, int64_t Lq, int H, int D,
                void *ws, size_t wsb) {
  return chunk_causal_attn(FAKE, FAKE, FAKE, cap, kv, pos0, L, FAKE, nullptr, ws, wsb, 1, H, D,
                           Lq, 0.f, nullptr);
}

int main() {
  const float *T = static_cast<const float *>(FAKE);
  // valid calls reach the launcher
  int before = g_launches;
  EXPECT(rope_apply_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32760, 28080, T, 21, 30, 52, 1, 12,
                           128, 4680, 18, 0, 30, 52, CRATTN_BF16, nullptr) == CRATTN_OK);
  EXPECT(attn(32760, 32760, 28080, 4680, 4680, 12, 128, nullptr, 0) == CRATTN_OK);
  const size_t ws = chunk_causal_attn_workspace_bytes(1, 12, 585, 32760, 28080 + 2925, 4680, 128);
  EXPECT(ws > 0);
  EXPECT(attn(32760, 32760, 28080 + 2925, 4680, 585, 12, 128, FAKE, ws) == CRATTN_OK);
  EXPECT(chunk_causal_attn_noalloc(FAKE, FAKE, FAKE, 32760, 32760, 28080 + 2925, 4680, FAKE,
                                   nullptr, 1, 12, 128, 585, 0.f, nullptr) == CRATTN_OK);
  EXPECT(hsa_select(FAKE, FAKE, 32760, 32760, 1560, 3 * 4680, 4680, 6, 32,
                    static_cast<int32_t *>(FAKE), 1, 12, 128, 4680, nullptr) == CRATTN_OK);
  EXPECT(g_launches == before + 5);
  // invalid ones do not
  before = g_launches;
  EXPECT(attn(32760, 32759, 28080, 4680, 4680, 12, 128, nullptr, 0) == CRATTN_EINVAL);
  EXPECT(attn(32760, 32760, 28080 + 2925, 4680, 585, 12, 128, FAKE, 16) == CRATTN_EINVAL);
  EXPECT(attn(int64_t(1) << 40, int64_t(1) << 40, 0, 1, 1, 12, 128, nullptr, 0) == CRATTN_EINVAL);
  EXPECT(attn(INT64_MAX, INT64_MAX, INT64_MAX - 1, INT64_MAX, 1, 1, 64, nullptr, 0) ==
         CRATTN_EINVAL);
  EXPECT(attn(256, 256, 192, 64, INT64_MAX, 1, 64, nullptr, 0) == CRATTN_EINVAL);
  EXPECT(rope_apply_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, INT64_MAX, INT64_MAX - 5, T, 4, 8,
                           8, 1, 2, 64, 64, 3, 0, 8, 8, CRATTN_BF16, nullptr) == CRATTN_EINVAL);
  EXPECT(rope_apply_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 0, T, 4, 1 << 16, 1 << 16, 1,
                           2, 64, 64, 3, 0, 1 << 16, 1 << 16, CRATTN_BF16, nullptr) ==
         CRATTN_EINVAL);
  EXPECT(rope_apply_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 0, T, 4, 8, 8, 1, 2, 64,
                           INT64_MAX, 3, INT64_MAX, 8, 8, CRATTN_BF16, nullptr) == CRATTN_EINVAL);
  EXPECT(chunk_causal_attn_noalloc(FAKE, FAKE, FAKE, 65536, 65535, 61440, 4096, FAKE, nullptr, 1,
                                   4, 128, 4096, 0.f, nullptr) == CRATTN_EINVAL);
  EXPECT(hsa_select(FAKE, FAKE, 32760, 32761, 1560, 3 * 4680, 4680, 6, 32,
                    static_cast<int32_t *>(FAKE), 1, 12, 128, 4680, nullptr) == CRATTN_EINVAL);
  EXPECT(svg2_plan(T, static_cast<const int32_t *>(FAKE), T, static_cast<const int32_t *>(FAKE),
                   static_cast<const int32_t *>(FAKE), 1, 2, 64, 4, 8, 3, 2, INT64_MAX, 64, 0.9f,
                   0.f, static_cast<int32_t *>(FAKE), static_cast<int32_t *>(FAKE), 128,
                   static_cast<int32_t *>(FAKE), static_cast<int32_t *>(FAKE), 5,
                   nullptr) == CRATTN_EINVAL);
  EXPECT(hsa_pool_keys(FAKE, 32760, 1560, INT64_MAX, 1560, FAKE, 1, 12, 128, nullptr) ==
         CRATTN_EINVAL);
  EXPECT(hsa_pool_keys(FAKE, INT64_MAX, 0, 1560, 1560, FAKE, 1, 12, 128, nullptr) ==
         CRATTN_EINVAL);
  EXPECT(qkv_rope_append(FAKE, FAKE, FAKE, FAKE, FAKE, INT64_MAX, INT64_MAX - 3, T, 4, 8, 8, 1, 2,
                         64, 128, 64, 3, 0, 8, 8, nullptr) == CRATTN_EINVAL);
  EXPECT(qkv_rope_append(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 0, T, 4, 8, 8, 1, 2, 64, 128,
                         INT64_MAX, 3, INT64_MAX, 8, 8, nullptr) == CRATTN_EINVAL);
  EXPECT(hsa_attn(FAKE, FAKE, FAKE, INT64_MAX, INT64_MAX, INT64_MAX - 1, INT64_MAX, 1,
                  static_cast<const int32_t *>(FAKE), 4, FAKE, nullptr, 1, 2, 64, 64, 0.f,
                  nullptr) == CRATTN_EINVAL);
  EXPECT(svg2_attn(FAKE, FAKE, FAKE, INT64_MAX, static_cast<const int32_t *>(FAKE),
                   static_cast<const int32_t *>(FAKE), 5, static_cast<const int32_t *>(FAKE),
                   INT64_MAX, static_cast<const int32_t *>(FAKE), 4, 1, FAKE, nullptr, FAKE,
                   SIZE_MAX, 1, 2, 64, INT64_MAX, 0.f, nullptr) == CRATTN_EINVAL);
  EXPECT(g_launches == before);
  EXPECT(rope_table_bytes(128, 1 << 20, 1 << 20, 1 << 20) > 0);
  EXPECT(rope_table_bytes(128, (1 << 20) + 1, 1, 1) == 0);
  EXPECT(svg2_n_slots(INT64_MAX, 256) == 0);
  EXPECT(svg2_attn_workspace_bytes(1 << 20, 1 << 10, INT64_MAX / 2, 128, 1, 16) == 0);
  // the last error is per thread
  char msg_a[512] = "", msg_b[512] = "";
  std::thread ta([&] {
    for (int i = 0; i < 200; ++i) {
      attn(32760, 32759, 28080, 4680, 4680, 12, 128, nullptr, 0);
      strncpy(msg_a, crattn_last_error(), sizeof msg_a - 1);
    }
  });
  std::thread tb([&] {
    for (int i = 0; i < 200; ++i) {
      attn(256, 256, 192, 64, 64, 1, 96, nullptr, 0);
      strncpy(msg_b, crattn_last_error(), sizeof msg_b - 1);
    }
  });
  ta.join();
  tb.join();
  EXPECT(strstr(msg_a, "incomplete") != nullptr);
  EXPECT(strstr(msg_b, "head_dim") != nullptr);
  if (failures) return 1;
  puts("abi driver: ok");
  return 0;
}
