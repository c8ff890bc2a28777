// Instantiates the FP32-accumulation GEMM with an E5M2 A operand (the kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8mp {

hipError_t launch_gemm_exact_a_e5m2(const GemmArgs& g, fp8mp_format b_fmt, int y_fmt, int num_cus,
                                    hipStream_t stream) {
  return b_fmt == FP8MP_E4M3 ? launch_y<FP8MP_E5M2, FP8MP_E4M3, kAccExact>(g, y_fmt, num_cus, stream)
                             : launch_y<FP8MP_E5M2, FP8MP_E5M2, kAccExact>(g, y_fmt, num_cus, stream);
}

}  // namespace fp8mp
