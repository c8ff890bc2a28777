// Sum of N ranks' FP8 gradient shards that share one scale, dequantised once:
//   out[i] = round_out( (sum_r dec(q_r[i])) * scale_inv ),
// the sum taken in FP32 in rank order, starting from rank 0's value.
//
// [MPT] §横断的知見 "テンソルスケーリングが FP8 実用化の鍵": an FP8 all-reduce uses one scale
// shared by all GPUs, the smallest of the ranks' scales, so that the ranks'
// codes can be summed directly. This is the arithmetic a rank applies to the
// shards it receives (the collective itself moves the bytes). HBM-bound:
// N bytes read and 2 (BF16) or 4 (FP32) bytes written per element.
#include "common.h"

namespace fp8mp {
namespace {

constexpr int kRedBlock = 256;

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Four codes (one dword) -> four floats, exactly (every FP8 value is an fp32).
template <int FMT>
__device__ __forceinline__ void dec4(uint32_t w, float& a, float& b, float& c, float& d) {
  v2f lo, hi;
  if constexpr (FMT == FP8MP_E4M3) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  }
  a = lo[0];
  b = lo[1];
  c = hi[0];
  d = hi[1];
}

template <int FMT>
__device__ __forceinline__ float dec1(uint8_t code) {
  float a, b, c, d;
  dec4<FMT>(code, a, b, c, d);
  return a;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

template <int FMT, int OUT>
__global__ __launch_bounds__(kRedBlock) void reduce_shared_kernel(const uint8_t* __restrict__ q, int n_ranks,
                                                                  int64_t numel, int64_t rank_stride,
                                                                  const float* __restrict__ scale_inv,
                                                                  void* __restrict__ out, int vec) {
  const float si = *scale_inv;
  const int64_t tid = (int64_t)blockIdx.x * kRedBlock + threadIdx.x, nthreads = (int64_t)gridDim.x * kRedBlock;
  int64_t start = 0;
  if (vec) {
    // 16 codes per thread and iteration: one 16-byte load per rank.
    const int64_t nchunk = numel / 16;
    for (int64_t c = tid; c < nchunk; c += nthreads) {
      // The running sum starts from rank 0's value (not from +0, which would
      // turn a lone -0 into +0), then adds ranks 1 .. n-1 in order.
      float acc[16];
      {
        const uint4 v = *reinterpret_cast<const uint4*>(q + 16 * c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) dec4<FMT>(w[k], acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]);
      }
      for (int r = 1; r < n_ranks; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(q + r * rank_stride + 16 * c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float a, b, cc, d;
          dec4<FMT>(w[k], a, b, cc, d);
          acc[4 * k] += a;
          acc[4 * k + 1] += b;
          acc[4 * k + 2] += cc;
          acc[4 * k + 3] += d;
        }
      }
      if constexpr (OUT == FP8MP_BF16) {
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + 16 * c);
        o[0] = uint4{pack_bf16(acc[0] * si, acc[1] * si), pack_bf16(acc[2] * si, acc[3] * si),
                     pack_bf16(acc[4] * si, acc[5] * si), pack_bf16(acc[6] * si, acc[7] * si)};
        o[1] = uint4{pack_bf16(acc[8] * si, acc[9] * si), pack_bf16(acc[10] * si, acc[11] * si),
                     pack_bf16(acc[12] * si, acc[13] * si), pack_bf16(acc[14] * si, acc[15] * si)};
      } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + 16 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = float4{acc[4 * k] * si, acc[4 * k + 1] * si, acc[4 * k + 2] * si, acc[4 * k + 3] * si};
      }
    }
    start = nchunk * 16;
  }
  // The rest (or everything, when the layout allows no 16-byte access).
  for (int64_t i = start + tid; i < numel; i += nthreads) {
    float acc = dec1<FMT>(q[i]);
    for (int r = 1; r < n_ranks; ++r) acc += dec1<FMT>(q[r * rank_stride + i]);
    const float yv = acc * si;
    if constexpr (OUT == FP8MP_BF16) static_cast<uint16_t*>(out)[i] = (uint16_t)(pack_bf16(yv, 0.f) & 0xFFFFu);
    else static_cast<float*>(out)[i] = yv;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int FMT>
hipError_t launch_out(const uint8_t* q, int n_ranks, int64_t numel, int64_t rank_stride, const float* scale_inv,
                      void* out, fp8mp_dtype out_dtype, int num_cus, hipStream_t stream) {
  const int vec = aligned(q, 16) && rank_stride % 16 == 0 && aligned(out, 16);
  const int64_t work = vec ? (numel + 15) / 16 : numel;
  const int64_t need = (work + kRedBlock - 1) / kRedBlock;
  const int64_t cap = (int64_t)num_cus * 4;
  const int grid = (int)(need < cap ? (need > 0 ? need : 1) : cap);
  if (out_dtype == FP8MP_BF16)
    hipLaunchKernelGGL((reduce_shared_kernel<FMT, FP8MP_BF16>), dim3(grid), dim3(kRedBlock), 0, stream, q, n_ranks,
                       numel, rank_stride, scale_inv, out, vec);
  else
    hipLaunchKernelGGL((reduce_shared_kernel<FMT, FP8MP_F32>), dim3(grid), dim3(kRedBlock), 0, stream, q, n_ranks,
                       numel, rank_stride, scale_inv, out, vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_shared_scale(const uint8_t* q, fp8mp_format fmt, int32_t n_ranks, int64_t numel,
                                      int64_t rank_stride, const float* scale_inv, void* out,
                                      fp8mp_dtype out_dtype, int num_cus, hipStream_t stream) {
  if (fmt == FP8MP_E4M3)
    return launch_out<FP8MP_E4M3>(q, n_ranks, numel, rank_stride, scale_inv, out, out_dtype, num_cus, stream);
  return launch_out<FP8MP_E5M2>(q, n_ranks, numel, rank_stride, scale_inv, out, out_dtype, num_cus, stream);
}

}  // namespace fp8mp
