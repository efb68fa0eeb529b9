// Drives the host side of the C ABI without a GPU -- plan choice, the host scheduler, workspace sizes,
// status strings, and the argument checks of every entry point with arguments they must refuse before
// touching the device -- for a build whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.
// Exits 0 when every call returns what the header promises.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../include/sda.h"

static int bad = 0;
#define EXPECT(c)                                         \
  do {                                                    \
    if (!(c)) {                                           \
      fprintf(stderr, "line %d: %s\n", __LINE__, #c);     \
      ++bad;                                              \
    }                                                     \
  } while (0)

int main() {
  for (int s = -5; s <= 1; ++s) EXPECT(sda_status_string(s) != nullptr);
  for (int f = -1; f < 8; ++f) { (void)sda_record_bytes(f); (void)sda_format_dims(f); }
  sda_plan plan;
  const int Hs[4] = {16, 32, 64, 128};
  for (int H : Hs)
    for (int T : {1, 7, 64, 300, 5000}) {
      EXPECT(sda_make_plan(T, H, 512, 128, 512, 256, &plan) == SDA_OK);
      EXPECT(sda_make_plan(T, H, 576, 2048, 0, 0, &plan) == SDA_OK);
      EXPECT(sda_workspace_bytes(T, H, 512, &plan) > 0);
      EXPECT(sda_workspace_bytes_v41(T, H, &plan) >= sda_workspace_bytes(T, H, 512, &plan));
      (void)sda_workspace_lse_offset(T, H, 512, &plan);
      (void)sda_noalloc_workspace_bytes(T, H, 512, &plan);
    }
  EXPECT(sda_make_plan(4, 24, 512, 128, 0, 256, &plan) == SDA_ERR_UNSUPPORTED);
  EXPECT(sda_make_plan(0, 16, 512, 128, 0, 256, &plan) == SDA_ERR_INVALID_ARG);
  // plan choice and the host scheduler over lengths with every edge (negative, zero, past the width)
  for (int T : {1, 5, 64, 700}) {
    std::vector<int32_t> lens(T), xl(T);
    for (int t = 0; t < T; ++t) { lens[t] = (t * 37) % 200 - 20; xl[t] = (t * 91) % 2100 - 10; }
    for (int qpl : {0, 1, 3}) {
      const int nl = qpl > 1 ? (T + qpl - 1) / qpl : T;
      EXPECT(sda_choose_plan(T, 32, 512, SDA_FP8_528, lens.data(), 128, SDA_NVFP4_288, xl.data(), 2048, qpl, 0, 256,
                             &plan) == SDA_OK);
      EXPECT(sda_choose_plan(T, 128, 576, SDA_V32_656, nullptr, 2048, -1, nullptr, 0, qpl, 0, 0, &plan) == SDA_OK);
      EXPECT(sda_make_plan(T, 32, 512, 128, 2048, 256, &plan) == SDA_OK);
      for (int F : {0, 2, 7}) {
        plan.fixed_overhead = F;
        for (int P : {1, 3, 257}) {
          plan.num_parts = P;
          std::vector<int32_t> meta((size_t)P * SDA_META_INTS), ns(T + 1);
          EXPECT(sda_get_sched_meta_host(T, qpl, lens.data(), 128, xl.data(), 2048, &plan, meta.data(), ns.data()) ==
                 SDA_OK);
          EXPECT(ns[0] == 0 && ns[T] >= T);
        }
      }
      (void)nl;
    }
  }
  EXPECT(sda_choose_plan(4, 16, 512, 9, nullptr, 64, -1, nullptr, 0, 1, 0, 256, &plan) == SDA_ERR_UNSUPPORTED);
  // the entry points refuse bad arguments on the host (no pointer is dereferenced)
  void* fake = (void*)(uintptr_t)(1u << 20);
  sda_cache c{fake, 4, 64, SDA_FP8_528, 64 * 528, nullptr};
  sda_list l{(const int32_t*)fake, 128, 128, 1, nullptr};
  EXPECT(sda_make_plan(4, 16, 512, 128, 0, 256, &plan) == SDA_OK);
  EXPECT(sda_sparse_decode_attn(fake, 8192, 512, 4, 24, 512, 512, &c, &l, nullptr, nullptr, nullptr, 0.1f, &plan,
                                nullptr, nullptr, fake, 1 << 30, fake, 8192, 512, (float*)fake, 16,
                                nullptr) == SDA_ERR_UNSUPPORTED);
  EXPECT(sda_sparse_decode_attn(fake, 8192, 512, 4, 16, 512, 512, &c, &l, &c, nullptr, nullptr, 0.1f, &plan, nullptr,
                                nullptr, fake, 1 << 30, fake, 8192, 512, (float*)fake, 16,
                                nullptr) == SDA_ERR_INVALID_ARG);
  EXPECT(sda_sparse_decode_attn(fake, 8192, 512, 4, 16, 512, 512, &c, &l, nullptr, nullptr, nullptr, 0.1f, &plan,
                                nullptr, nullptr, fake, 16, fake, 8192, 512, (float*)fake, 16,
                                nullptr) == SDA_ERR_WORKSPACE);
  EXPECT(sda_decode_splits(fake, 8192, 512, 4, 16, 512, 512, &c, &l, nullptr, nullptr, nullptr, 0.1f, &plan, nullptr,
                           nullptr, fake, 1 << 30, fake, 8192, 512, (float*)fake, 16, nullptr) == SDA_ERR_INVALID_ARG);
  EXPECT(sda_combine_splits(4, 24, 512, (const float*)fake, (const float*)fake, (const int32_t*)fake, nullptr, fake,
                            8192, 512, (float*)fake, 16, nullptr) == SDA_ERR_UNSUPPORTED);
  sda_plan big;
  EXPECT(sda_make_plan(128, 128, 576, 2048, 0, 256, &big) == SDA_OK);
  sda_cache c5{fake, 2048, 64, SDA_V32_656, 64 * 656, nullptr};
  sda_list l5{(const int32_t*)fake, 2048, 2048, 1, nullptr};
  EXPECT(sda_sparse_decode_attn_noalloc(fake, 128 * 576, 576, 128, 128, 576, 512, &c5, &l5, nullptr, nullptr, nullptr,
                                        0.04f, &big, nullptr, nullptr, fake, 128 * 512, 512, (float*)fake, 128,
                                        nullptr) == SDA_ERR_WORKSPACE);
  sda_v41 v{};
  EXPECT(sda_sparse_decode_attn_v41(fake, 8192, 512, 4, 16, &c, &l, nullptr, nullptr, nullptr, 0.1f, &plan, nullptr,
                                    nullptr, fake, 1 << 30, &v, nullptr, 0, nullptr) == SDA_ERR_INVALID_ARG);
  EXPECT(sda_last_error() != nullptr);
  printf("api sanitizer check: %s\n", bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
