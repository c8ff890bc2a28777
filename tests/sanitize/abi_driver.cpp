// Drives every C-ABI entry point through its argument validation: NULL and misaligned pointers,
// negative, zero and extreme sizes (products that would overflow int64), bad enums and
// hyperparameters, and well-formed calls (which return FP8MP_ERR_NO_DEVICE without a GPU, or reach
// the launch stubs on one). Built with host address and undefined-behaviour sanitizers; any
// sanitizer report or unexpected status fails the run. Pointers are fake addresses that the
// validation never dereferences.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fp8mp.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                                    \
  do {                                                                                        \
    const int got_ = (int)(call);                                                             \
    if (got_ != (int)(want)) {                                                                \
      std::fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
      ++g_fail;                                                                               \
    }                                                                                         \
  } while (0)
// a well-formed call: no device here (or the launch stub on a GPU machine)
#define EXPECT_VALID(call)                                                                    \
  do {                                                                                        \
    const int got_ = (int)(call);                                                             \
    if (got_ != FP8MP_ERR_NO_DEVICE && got_ != FP8MP_OK && got_ != FP8MP_ERR_WRONG_ARCH) {    \
      std::fprintf(stderr, "line %d: %s -> %d, want a valid call\n", __LINE__, #call, got_);  \
      ++g_fail;                                                                               \
    }                                                                                         \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const int64_t BIG = INT64_MAX, HALF = INT64_MAX / 2;
constexpr fp8mp_status INV = FP8MP_ERR_INVALID_ARG, UNS = FP8MP_ERR_UNSUPPORTED;

int main() {
  uint8_t* q = (uint8_t*)P(1 << 20);
  float* f = (float*)P(1 << 21);
  uint16_t* h = (uint16_t*)P(1 << 22);
  const void* x = P(1 << 23);
  const fp8mp_dtype BF = FP8MP_BF16, F32 = FP8MP_F32;
  const fp8mp_format E4 = FP8MP_E4M3, E5 = FP8MP_E5M2;

  // fp8_amax_cast
  EXPECT(fp8_amax_cast(nullptr, BF, 4, 4, 4, E4, f, q, 4, nullptr, 0, f, nullptr), INV);
  EXPECT(fp8_amax_cast(x, (fp8mp_dtype)7, 4, 4, 4, E4, f, q, 4, nullptr, 0, f, nullptr), INV);
  EXPECT(fp8_amax_cast(x, BF, -1, 4, 4, E4, f, q, 4, nullptr, 0, f, nullptr), INV);
  EXPECT(fp8_amax_cast(x, BF, 4, 4, 4, E4, nullptr, q, 4, nullptr, 0, f, nullptr), INV);
  EXPECT(fp8_amax_cast(P(4104), BF, 4, 4, 4, E4, f, q, 4, nullptr, 0, f, nullptr), INV);
  EXPECT(fp8_amax_cast(x, BF, 4, 4, 12, E4, f, q, 16, nullptr, 0, f, nullptr), INV);
  EXPECT(fp8_amax_cast(x, F32, 4, 4, 8, E4, f, q, 16, nullptr, 0, f, nullptr), UNS);
  EXPECT(fp8_amax_cast(x, BF, BIG, BIG, BIG, E4, f, q, BIG, nullptr, 0, f, nullptr), UNS);
  EXPECT(fp8_amax_cast(x, BF, HALF, 16, 16, E4, f, nullptr, 0, q, BIG - 15, f, nullptr), UNS);
  EXPECT(fp8_amax_cast(x, BF, 0, BIG, BIG, E4, f, q, BIG, nullptr, 0, f, nullptr), FP8MP_OK);
  EXPECT_VALID(fp8_amax_cast(x, BF, 4, 4, 4, E4, f, q, 4, nullptr, 0, f, nullptr));
  EXPECT_VALID(fp8_amax_cast(x, BF, 300, 200, 208, E5, f, q, 208, q, 304, f, nullptr));
  EXPECT_VALID(fp8_amax_cast(x, F32, 1, 17, 1000, E4, f, q, 17, nullptr, 0, nullptr, nullptr));
  EXPECT(fp8_amax_cast(x, F32, 1, 17, 1000, E4, f, q, 3, nullptr, 0, nullptr, nullptr), INV);   // ld_q < cols

  // fp8_amax_cast_batched
  fp8mp_cast_item items[3];
  for (auto& it : items) it = fp8mp_cast_item{x, BF, 64, E4, f, q, f};
  EXPECT(fp8_amax_cast_batched(-1, items, nullptr), INV);
  EXPECT(fp8_amax_cast_batched(3, nullptr, nullptr), INV);
  items[2].q = (uint8_t*)P(4100);
  EXPECT(fp8_amax_cast_batched(3, items, nullptr), INV);
  items[2].q = q;
  items[1].numel = -5;
  EXPECT(fp8_amax_cast_batched(3, items, nullptr), INV);
  items[1].numel = BIG;
  EXPECT_VALID(fp8_amax_cast_batched(3, items, nullptr));
  EXPECT(fp8_amax_cast_batched(0, nullptr, nullptr), FP8MP_OK);

  // fp8_scale_update (+ batched)
  EXPECT(fp8_scale_update(nullptr, 4, E4, 0, f, f, nullptr), INV);
  EXPECT(fp8_scale_update(f, 0, E4, 0, f, f, nullptr), INV);
  EXPECT(fp8_scale_update(f, 4, E4, -1, f, f, nullptr), INV);
  EXPECT(fp8_scale_update(f, 4, (fp8mp_format)9, 0, f, f, nullptr), INV);
  EXPECT_VALID(fp8_scale_update(f, INT32_MAX, FP8MP_FP16, INT32_MAX, f, f, nullptr));
  float* hs[2] = {f, f + 8};
  int32_t lens[2] = {4, 1024}, margins[2] = {0, 3};
  fp8mp_format fmts[2] = {E4, E5};
  EXPECT(fp8_scale_update_batched(-1, hs, lens, fmts, margins, hs, hs, nullptr), INV);
  EXPECT(fp8_scale_update_batched(2, hs, nullptr, fmts, margins, hs, hs, nullptr), INV);
  lens[1] = 0;
  EXPECT(fp8_scale_update_batched(2, hs, lens, fmts, margins, hs, hs, nullptr), INV);
  lens[1] = 1024;
  EXPECT_VALID(fp8_scale_update_batched(2, hs, lens, fmts, margins, hs, hs, nullptr));

  // fp8_scaled_gemm and its forms
  EXPECT(fp8_scaled_gemm(q, E4, 32, q, E4, 32, -1, 8, 32, f, f, h, 8, nullptr), INV);
  EXPECT(fp8_scaled_gemm(q, E4, 32, q, E4, 32, 4, 8, 24, f, f, h, 8, nullptr), UNS);
  EXPECT(fp8_scaled_gemm(q, E4, 40, q, E4, 32, 4, 8, 32, f, f, h, 8, nullptr), INV);
  EXPECT(fp8_scaled_gemm(q, E4, 32, q, E4, 32, 4, 8, 32, f, f, (uint16_t*)P(4098), 8, nullptr), INV);
  EXPECT(fp8_scaled_gemm(q, E4, 32, q, E4, 32, 4, 8, 32, f, f, h, 12, nullptr), INV);
  EXPECT(fp8_scaled_gemm(q, E4, 32, q, E4, 32, BIG, int64_t(1) << 40, 32, f, f, h, int64_t(1) << 40, nullptr), UNS);
  EXPECT(fp8_scaled_gemm(q, E4, 32, q, E4, 32, 4, BIG, 32, f, f, h, BIG - 7, nullptr), INV);     // ldc < n
  EXPECT(fp8_scaled_gemm(q, E4, 1 << 23, q, E4, 32, 4, 8, 32, f, f, h, 8, nullptr), UNS);
  EXPECT_VALID(fp8_scaled_gemm(q, E4, 32, q, E5, 32, 4, 8, 32, f, f, h, 8, nullptr));
  EXPECT_VALID(fp8_scaled_gemm(q, E4, 0, q, E4, 0, 4, 8, 0, f, f, h, 8, nullptr));
  EXPECT_VALID(fp8_scaled_gemm_fast_accum(q, E5, 4096, q, E4, 4096, 4096, 11008, 4096, f, f, h, 11008, nullptr));
  // k == 0 leaves lda and ldb unused; with no C the output count must still not overflow
  EXPECT(fp8_scaled_gemm_amax_cast(q, E4, 0, q, E4, 0, BIG, BIG, 0, f, f, nullptr, 0, E4, f, nullptr, 0, f, nullptr),
         UNS);
  EXPECT(fp8_scaled_gemm_amax_cast(q, E4, 32, q, E4, 32, 4, 8, 32, f, f, h, 8, E4, f, (uint8_t*)P(4104), 16, f,
                                   nullptr), INV);
  EXPECT(fp8_scaled_gemm_amax_cast(q, E4, 32, q, E4, 32, 4, 8, 32, f, f, h, 8, E4, nullptr, q, 16, f, nullptr), INV);
  EXPECT_VALID(fp8_scaled_gemm_amax_cast(q, E4, 32, q, E4, 32, 4, 8, 32, f, f, nullptr, 0, E5, f, q, 16, f, nullptr));
  EXPECT_VALID(fp8_scaled_gemm_amax_cast_fast_accum(q, E4, 32, q, E4, 32, 4, 8, 32, f, f, h, 8, E4, f, q, 16, f,
                                                    nullptr));

  // fp8_layernorm_amax_cast
  EXPECT(fp8_layernorm_amax_cast(x, BF, 4, 0, 8, f, f, 1e-5f, h, 8, E4, f, q, 8, f, f, f, nullptr), INV);
  EXPECT(fp8_layernorm_amax_cast(x, BF, 4, 8, 8, f, f, -1.0f, h, 8, E4, f, q, 8, f, f, f, nullptr), INV);
  EXPECT(fp8_layernorm_amax_cast(x, BF, BIG, 8, BIG, f, f, 1e-5f, h, BIG, E4, f, q, BIG, f, f, f, nullptr), UNS);
  EXPECT_VALID(fp8_layernorm_amax_cast(x, BF, 4, 8, 8, f, nullptr, 1e-5f, h, 8, E4, f, q, 8, f, nullptr, nullptr,
                                       nullptr));

  // fp8_reduce_shared_scale
  EXPECT(fp8_reduce_shared_scale(q, E5, 0, 64, 64, f, h, BF, nullptr), INV);
  EXPECT(fp8_reduce_shared_scale(q, E5, 4, 64, 63, f, h, BF, nullptr), INV);
  EXPECT(fp8_reduce_shared_scale(q, E5, INT32_MAX, BIG, BIG, f, h, F32, nullptr), UNS);
  EXPECT_VALID(fp8_reduce_shared_scale(q, E5, 8, 1000, 1024, f, h, BF, nullptr));

  // fp8_adam_step (+ weight cast)
  EXPECT(fp8_adam_step(64, x, BF, q, f, f + 1, f, f, nullptr, h, h, f + 2, f + 3, f, f, nullptr, 1e-3f, 0.9f, 0.999f,
                       1e-8f, 0.0f, 0, nullptr), INV);
  EXPECT(fp8_adam_step(64, x, BF, q, f, f + 1, f, f, nullptr, h, h, f + 2, f + 3, f, f, nullptr, 1e-3f, 1.0f, 0.999f,
                       1e-8f, 0.0f, 3, nullptr), INV);
  EXPECT(fp8_adam_step(64, x, BF, q, f, f, f, f, nullptr, h, h, f + 2, f + 3, f, f, nullptr, 1e-3f, 0.9f, 0.999f,
                       1e-8f, 0.0f, 3, nullptr), INV);
  EXPECT_VALID(fp8_adam_step(64, x, BF, q, f, f + 1, f, f, nullptr, h, h, f + 2, f + 3, f, f, nullptr, 1e-3f, 0.9f,
                             0.999f, 1e-8f, 0.1f, BIG, nullptr));
  EXPECT(fp8_adam_step_weight_cast(64, x, BF, q, f, f + 1, f, f, nullptr, h, h, f + 2, f + 3, f, f, nullptr, 1e-3f,
                                   0.9f, 0.999f, 1e-8f, 0.0f, 2, FP8MP_FP16, f, q, f, nullptr), INV);
  EXPECT_VALID(fp8_adam_step_weight_cast(64, x, BF, q, f, f + 1, f, f, nullptr, h, h, f + 2, f + 3, f, f, nullptr,
                                         1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 2, E4, f, q, f, nullptr));

  // status strings and device info
  for (int s = -3; s < 12; ++s)
    if (fp8mp_status_string((fp8mp_status)s) == nullptr) ++g_fail;
  char buf[8];
  const int di = (int)fp8mp_device_info(buf, sizeof buf);
  if (di != FP8MP_ERR_NO_DEVICE && di != FP8MP_OK && di != FP8MP_ERR_WRONG_ARCH) ++g_fail;
  if (std::strlen(buf) >= sizeof buf) ++g_fail;
  EXPECT(fp8mp_device_info(nullptr, 16), INV);

  std::printf("abi driver: %d failures\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
