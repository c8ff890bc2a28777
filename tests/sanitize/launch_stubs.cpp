// Host-only stand-ins for the kernel launchers, so the C-ABI front end (argument validation and
// dispatch) can be built and run under host sanitizers without device code. Each stub counts its
// calls and launches nothing.
#include "common.h"

namespace fp8mp {
int g_launches = 0;
hipError_t launch_amax_cast_batched(CastBatch&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_amax_cast(const void*, fp8mp_dtype, int64_t, int64_t, int64_t, fp8mp_format, const float*, uint8_t*,
                            int64_t, uint8_t*, int64_t, float*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scale_update(float*, int32_t, fp8mp_format, int32_t, float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_scale_update_batched(const ScaleUpdateBatch&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scaled_gemm(const uint8_t*, fp8mp_format, int64_t, const uint8_t*, fp8mp_format, int64_t, int64_t,
                              int64_t, int64_t, const float*, const float*, uint16_t*, int64_t, bool, int,
                              hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scaled_gemm_amax_cast(const uint8_t*, fp8mp_format, int64_t, const uint8_t*, fp8mp_format, int64_t,
                                        int64_t, int64_t, int64_t, const float*, const float*, uint16_t*, int64_t,
                                        fp8mp_format, const float*, uint8_t*, int64_t, float*, bool, int,
                                        hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_layernorm_amax_cast(const void*, fp8mp_dtype, int64_t, int64_t, int64_t, const float*, const float*,
                                      float, uint16_t*, int64_t, fp8mp_format, const float*, uint8_t*, int64_t, float*,
                                      float*, float*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_adam_step(int64_t, const void*, fp8mp_dtype, uint8_t*, const float*, float*, const float*,
                            const float*, float*, uint16_t*, uint16_t*, const float*, float*, const float*,
                            const float*, float*, float, float, float, float, float, float, float, int, const float*,
                            uint8_t*, float*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_reduce_shared_scale(const uint8_t*, fp8mp_format, int32_t, int64_t, int64_t, const float*, void*,
                                      fp8mp_dtype, int, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace fp8mp
