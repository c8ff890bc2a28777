// Entry points of the scaled FP8 GEMM: C = (A . B^T) * sa_inv * sb_inv with
// FP32 accumulation and a BF16 output, optionally with the amax and FP8 cast
// of that output fused into the epilogue. The kernels are in gemm_kernels.h;
// this file picks the instantiation unit by accumulation mode and formats.
//
// [MPT] §横断的知見 "FP8 への拡張": only the GEMMs run in FP8; §"HPC ソルバーとの目的の分岐":
// the matrix units accumulate in FP32.
#include "common.h"
#include "gemm_parts.h"

namespace fp8mp {
namespace {

constexpr int kNoOutputCast = -1;

hipError_t dispatch(const GemmArgs& g, fp8mp_format a_fmt, fp8mp_format b_fmt, int y_fmt, bool fast, int num_cus,
                    hipStream_t stream) {
  if (fast) return launch_gemm_fast(g, a_fmt, b_fmt, y_fmt, num_cus, stream);
  return a_fmt == FP8MP_E4M3 ? launch_gemm_exact_a_e4m3(g, b_fmt, y_fmt, num_cus, stream)
                             : launch_gemm_exact_a_e5m2(g, b_fmt, y_fmt, num_cus, stream);
}

}  // namespace

hipError_t launch_scaled_gemm(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                              fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                              const float* a_scale_inv, const float* b_scale_inv, uint16_t* c,
                              int64_t ldc, bool fast_accum, int num_cus, hipStream_t stream) {
  const GemmArgs g{a, lda, b, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc, nullptr, nullptr, 0, nullptr};
  return dispatch(g, a_fmt, b_fmt, kNoOutputCast, fast_accum, num_cus, stream);
}

hipError_t launch_scaled_gemm_amax_cast(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                                        fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                        const float* a_scale_inv, const float* b_scale_inv, uint16_t* c,
                                        int64_t ldc, fp8mp_format y_fmt, const float* y_scale, uint8_t* y_q,
                                        int64_t ld_yq, float* y_amax, bool fast_accum, int num_cus,
                                        hipStream_t stream) {
  const GemmArgs g{a, lda, b, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc, y_scale, y_q, ld_yq, y_amax};
  return dispatch(g, a_fmt, b_fmt, y_fmt, fast_accum, num_cus, stream);
}

}  // namespace fp8mp
