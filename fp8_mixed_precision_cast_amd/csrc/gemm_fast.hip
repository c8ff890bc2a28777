// Instantiates the fast-accumulation GEMM (FP8 MFMA) (the kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8mp {

hipError_t launch_gemm_fast(const GemmArgs& g, fp8mp_format a_fmt, fp8mp_format b_fmt, int y_fmt, int num_cus,
                            hipStream_t stream) {
  if (a_fmt == FP8MP_E4M3 && b_fmt == FP8MP_E4M3)
    return launch_y<FP8MP_E4M3, FP8MP_E4M3, kAccFast>(g, y_fmt, num_cus, stream);
  if (a_fmt == FP8MP_E5M2 && b_fmt == FP8MP_E4M3)
    return launch_y<FP8MP_E5M2, FP8MP_E4M3, kAccFast>(g, y_fmt, num_cus, stream);
  if (a_fmt == FP8MP_E4M3 && b_fmt == FP8MP_E5M2)
    return launch_y<FP8MP_E4M3, FP8MP_E5M2, kAccFast>(g, y_fmt, num_cus, stream);
  return launch_y<FP8MP_E5M2, FP8MP_E5M2, kAccFast>(g, y_fmt, num_cus, stream);
}

}  // namespace fp8mp
