// Launch entry points of the GEMM instantiation units (gemm_exact_a4.hip,
// gemm_exact_a5.hip, gemm_fast.hip), called by gemm.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "fp8mp.h"

namespace fp8mp {

// Everything a launch needs besides the format templates.
struct GemmArgs {
  const uint8_t* a; int64_t lda;
  const uint8_t* b; int64_t ldb;
  int64_t m, n, k;
  const float* sa; const float* sb;
  uint16_t* c; int64_t ldc;
  const float* y_scale; uint8_t* y_q; int64_t ld_yq; float* y_amax;
};

// y_fmt: an fp8mp_format for the fused output cast, or -1 for none.
// FP32-accumulation GEMM with A in E4M3 (resp. E5M2), B in b_fmt.
hipError_t launch_gemm_exact_a_e4m3(const GemmArgs& g, fp8mp_format b_fmt, int y_fmt, int num_cus,
                                    hipStream_t stream);
hipError_t launch_gemm_exact_a_e5m2(const GemmArgs& g, fp8mp_format b_fmt, int y_fmt, int num_cus,
                                    hipStream_t stream);
// Fast-accumulation GEMM (FP8 MFMA), any format pair.
hipError_t launch_gemm_fast(const GemmArgs& g, fp8mp_format a_fmt, fp8mp_format b_fmt, int y_fmt, int num_cus,
                            hipStream_t stream);

}  // namespace fp8mp
