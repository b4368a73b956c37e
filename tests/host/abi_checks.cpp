// Host checks of libmla.so's C ABI, built with the library's host code and the launch stubs
// under ASan + UBSan (no GPU): every entry point's argument checks, calls that pass them
// (which end at a stub and report MLA_ERR_HIP), and a sweep of the split planner over
// shapes, lengths and CU counts.  Prints "ok" or the first failure.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "mla.h"

static int fails = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
      ++fails;                                                         \
    }                                                                  \
  } while (0)

int main() {
  void* F = (void*)0x1000;  // non-null, never dereferenced
  const float nan = std::nanf(""), inf = INFINITY;
  auto* u8 = (uint8_t*)F;
  auto* f32 = (float*)F;
  auto* i32 = (int32_t*)F;
  auto* u16 = (uint16_t*)F;

  for (int s = 0; s <= 5; ++s) EXPECT(mla_status_string((mla_status)s) != nullptr);
  EXPECT(mla_status_string((mla_status)77) != nullptr);
  EXPECT(mla_status_string((mla_status)-5) != nullptr);

  // quantize
  EXPECT(mla_quantize_fp8_sat(f32, u8, -1, 1.f, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_quantize_fp8_sat(f32, u8, 10, nan, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_quantize_fp8_sat(f32, u8, 10, -inf, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_quantize_fp8_sat(nullptr, u8, 10, 1.f, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_quantize_fp8_sat(nullptr, nullptr, 0, 1.f, nullptr) == MLA_OK);
  EXPECT(mla_quantize_fp8_sat(f32, u8, 10, 1.f, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_quantize_fp8_sat_dynamic(F, 0, u8, 10, f32, F, 4095, nullptr) == MLA_ERR_WORKSPACE);
  EXPECT(mla_quantize_fp8_sat_dynamic(F, 3, u8, 10, f32, F, 4096, nullptr) ==
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_quantize_fp8_sat_dynamic(F, 1, u8, 10, f32, F, 4096, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_kv_append_fp8_sat(F, 0, u8, 8, i32, i32, 2, 1, 64, 4, 1.f, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_kv_append_fp8_sat(F, 0, u8, 8, i32, i32, 1 << 16, 1 << 16, 64, 4, 1.f, nullptr) ==
         MLA_ERR_UNSUPPORTED);
  EXPECT(mla_kv_append_rope_fp8_sat(F, 0, u8, 8, i32, i32, 2, 1, 64, 4, 1.f, f32, f32, 100,
                                    nullptr) == MLA_ERR_HIP);
  EXPECT(mla_kv_append_rope_fp8_sat(F, 1, u8, 8, i32, i32, 2, 1, 64, 4, 1.f, nullptr, f32, 100,
                                    nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_kv_append_rope_fp8_sat(F, 0, u8, 8, i32, i32, 2, 1, 64, 4, 1.f, f32, f32, 0,
                                    nullptr) == MLA_ERR_INVALID_ARG);

  // decode: bad arguments, unsupported shapes, workspace, then calls that reach the launch
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1, 1, 16, 64, 4, 256, 1.f, 1.f, 0.07f, 4, 128,
                            u16, f32, 1 << 20, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1, 1, 16, 48, 4, 256, 1.f, 1.f, 0.07f, 4, 128,
                            u16, f32, 1 << 20, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1, 1, 16, 64, 4, 256, 1.f, 1.f, 0.07f, 4, 128,
                            u16, f32, 63, nullptr) == MLA_ERR_WORKSPACE);
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1, 1, 16, 64, 4, 256, 1.f, nan, 0.07f, 4, 128,
                            u16, f32, 1 << 20, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1, 2, 40000, 64, 4, 256, 1.f, 1.f, 0.07f, 4, 128,
                            u16, f32, 1 << 20, nullptr) == MLA_ERR_UNSUPPORTED);
  // the largest shapes the checks let through (row and grid bounds)
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 64, 16, 4096, 64, 1 << 20, 1 << 26, 1.f, 1.f,
                            0.07f, 2, 128, u16, f32, INT64_MAX, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1, 1, 128, 1 << 20, 2000, 1 << 26, 1.f, 1.f,
                            0.07f, 65535, 128, u16, f32, INT64_MAX, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_decode_splitkv(u8, u8, i32, i32, 1 << 20, 16, 4096, 64, 4, 256, 1.f, 1.f, 0.07f,
                            65535, 128, u16, f32, INT64_MAX, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_splitkv_ex(u8, u8, i32, i32, i32, i32, i32, 2, 8, 16, 64, 4, 256, 1.f, 1.f,
                               nullptr, nullptr, 0.07f, 4, 128, u16, f32, 1 << 20, nullptr) ==
         MLA_ERR_HIP);
  EXPECT(mla_decode_splitkv_dev_scales(u8, u8, i32, i32, 2, 8, 16, 64, 4, 256, f32, f32, 0.07f,
                                       4, 128, u16, f32, 1 << 20, nullptr) == MLA_ERR_HIP);

  // combine
  EXPECT(mla_splitkv_combine(u16, f32, 1, 4, 1, 16, 1.f, u16, nullptr, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_splitkv_combine(u16, f32, 1, 4097, 1, 16, 1.f, u16, nullptr, nullptr) ==
         MLA_ERR_UNSUPPORTED);
  EXPECT(mla_splitkv_combine_partial(u16, f32, 1, 4, 1, 16, u16, f32, 15, nullptr) ==
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_splitkv_combine_partial(u16, f32, 3, 4, 2, 16, u16, f32, 64, nullptr) ==
         MLA_ERR_HIP);
  EXPECT(mla_splitkv_combine_dev_scale(u16, f32, 1, 4, 1, 16, f32, u16, f32, nullptr) ==
         MLA_ERR_HIP);
  EXPECT(mla_hbm_read_probe(F, 32768, (uint32_t*)F, 1, nullptr) == MLA_ERR_HIP);

  // the decode without allocation: argument checks, partials that do not fit, and calls
  // that pass (they end where the array's address is looked up: no device here)
  const int64_t kRows = (MLA_NOALLOC_SCRATCH_BYTES - 256) / 1028;
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, 1, 1, 16, 64, 4, 256, 1.f, 1.f, 0.07f, 4, nullptr,
                            nullptr, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode_noalloc(nullptr, u8, i32, i32, 1, 1, 16, 64, 4, 256, 1.f, 1.f, 0.07f, 4, u16,
                            nullptr, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, 1, 1, 16, 64, 4, 256, nan, 1.f, 0.07f, 4, u16,
                            nullptr, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, 1, 1, 16, 48, 4, 256, 1.f, 1.f, 0.07f, 4, u16,
                            nullptr, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_noalloc(nullptr, nullptr, nullptr, nullptr, 0, 1, 16, 64, 4, 256, 1.f, 1.f,
                            0.07f, 4, nullptr, nullptr, nullptr) == MLA_OK);
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, 1, 1, 128, 64, 4, 256, 1.f, 1.f, 0.07f,
                            (int)(kRows / 128) + 1, u16, f32, nullptr) == MLA_ERR_WORKSPACE);
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, 1, 1, 128, 64, 4, 256, 1.f, 1.f, 0.07f,
                            (int)(kRows / 128), u16, f32, nullptr) == MLA_ERR_HIP);
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, (int)(kRows / 128) + 1, 1, 128, 64, 4, 256, 1.f,
                            1.f, 0.07f, 0, u16, f32, nullptr) == MLA_ERR_WORKSPACE);
  EXPECT(mla_decode_noalloc(u8, u8, i32, i32, 16, 1, 128, 64, 4, 256, 1.f, 1.f, 0.07f, 0, u16,
                            f32, nullptr) == MLA_ERR_HIP);

  // planner: every shape gets a split count within [1, max(1, tiles / 2)] (and at most 4096),
  // 128 rows per group and partial_rows = B * S * Sq * H
  const int batches[] = {1, 2, 3, 16, 32, 64, 1024};
  const int qts[] = {1, 2, 8, 16};
  const int heads[] = {1, 16, 64, 128, 4096};
  const int lens[] = {1, 31, 64, 65, 1000, 4096, 131072, 1048576, 1 << 26};
  const int cus[] = {1, 80, 256, 304, 1024};
  long n = 0;
  for (int B : batches)
    for (int Sq : qts)
      for (int H : heads)
        for (int L : lens)
          for (int cu : cus) {
            int S = -1, r = -1;
            int64_t rows = -1;
            const mla_status st = mla_splitkv_plan(B, Sq, H, L, 0, cu, &S, &r, &rows);
            if ((int64_t)Sq * H > 65536) {
              EXPECT(st == MLA_ERR_UNSUPPORTED);
              continue;
            }
            EXPECT(st == MLA_OK);
            const int64_t tiles = ((int64_t)L + 31) / 32;
            const int64_t smax = tiles / 2 > 0 ? tiles / 2 : 1;
            EXPECT(S >= 1 && S <= smax && S <= 4096);
            EXPECT(r == 128);
            EXPECT(rows == (int64_t)B * S * Sq * H);
            const int64_t total = (int64_t)B * L / 2 + 1;  // mixed lengths
            EXPECT(mla_splitkv_plan(B, Sq, H, L, total, cu, &S, nullptr, nullptr) == MLA_OK);
            EXPECT(S >= 1 && S <= smax);
            ++n;
          }
  EXPECT(n > 1000);
  EXPECT(mla_splitkv_plan(1, 1, 128, 1000, 0, 0, nullptr, nullptr, nullptr) == MLA_ERR_HIP);

  if (fails == 0) std::printf("ok\n");
  return fails == 0 ? 0 : 1;
}
