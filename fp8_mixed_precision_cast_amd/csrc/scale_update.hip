// Delayed-scaling update: scale from the amax history, then roll the history.
//
// [TE] §動的スケーリングとFP8レシピの設定: the DelayedScaling recipe takes a margin
// (default 0) and an amax history length (default 1024) that the scale is
// computed from. [MPT] §横断的知見 on tensor scaling names delayed per-tensor
// scaling. The update is latency-bound: one workgroup reads at most a few KB.
#include "common.h"

namespace fp8mp {
namespace {

constexpr int kBlock = 256;
constexpr int kLdsEntries = 8192;   // histories up to this long are rolled through LDS in one pass

template <int FMT>
__device__ __forceinline__ void update_scale_from(uint32_t a, int32_t margin, float* __restrict__ scale,
                                                  float* __restrict__ scale_inv) {
  // finite and positive: 0 < bits < +Inf
  if (a != 0u && a < 0x7F800000u) {
    const float ratio = Fp8Traits<FMT>::kMax / __uint_as_float(a);  // IEEE binary32 division
    const float s = __builtin_ldexpf(ratio, -margin);               // exact 2^-margin, one rounding
    const float inv = 1.0f / s;
    const uint32_t sb = __float_as_uint(s), ib = __float_as_uint(inv);
    if (sb != 0u && sb < 0x7F800000u && ib < 0x7F800000u) {
      *scale = s;
      *scale_inv = inv;
    }
  }
}

__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t a = red[0];
#pragma unroll
  for (int w = 1; w < kBlock / 64; ++w) a = a > red[w] ? a : red[w];
  return a;
}

// One tensor's update, run by one whole workgroup (`stage` and `red` are its
// LDS).
template <int FMT>
__device__ __forceinline__ void update_one(float* __restrict__ hist, int32_t len, int32_t margin,
                                           float* __restrict__ scale, float* __restrict__ scale_inv,
                                           uint32_t* stage, uint32_t* red) {
  uint32_t* h = reinterpret_cast<uint32_t*>(hist);

  // Max over every entry. History entries are amaxes: non-negative floats or
  // the canonical NaN, so the unsigned max of the bit patterns (sign masked)
  // is the NaN-propagating float max.
  if (len <= kLdsEntries) {
    // One pass: every entry is read once into LDS, then written back shifted.
    uint32_t m = 0;
    for (int32_t i = threadIdx.x; i < len; i += kBlock) {
      const uint32_t v = h[i];
      stage[i] = v;
      const uint32_t a = v & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
    const uint32_t a = block_max(m, red);   // also orders the LDS writes before the reads below
    if (threadIdx.x == 0) update_scale_from<FMT>(a, margin, scale, scale_inv);
    for (int32_t i = threadIdx.x; i < len; i += kBlock) h[i] = i == 0 ? 0u : stage[i - 1];
    return;
  }

  uint32_t m = 0;
  for (int32_t i = threadIdx.x; i < len; i += kBlock) {
    const uint32_t v = h[i] & 0x7FFFFFFFu;
    m = m > v ? m : v;
  }
  const uint32_t a = block_max(m, red);
  if (threadIdx.x == 0) update_scale_from<FMT>(a, margin, scale, scale_inv);

  // Long histories roll in place by chunks moved from the top down, each read
  // fully before any of it is written; a chunk's writes never reach entries a
  // lower chunk still has to read.
  for (int32_t top = len; top > 0; top -= kBlock) {
    const int32_t i = top - kBlock + (int32_t)threadIdx.x;   // destination index
    __syncthreads();
    uint32_t v = 0;
    const bool dst = i >= 0 && i < len;
    if (dst && i >= 1) v = h[i - 1];
    __syncthreads();
    if (dst) h[i] = v;
  }
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void scale_update_kernel(float* __restrict__ hist, int32_t len,
                                                              int32_t margin, float* __restrict__ scale,
                                                              float* __restrict__ scale_inv) {
  __shared__ uint32_t red[kBlock / 64];
  __shared__ uint32_t stage[kLdsEntries];
  update_one<FMT>(hist, len, margin, scale, scale_inv, stage, red);
}

// Several tensors in one launch: workgroup b updates tensor b.
__global__ __launch_bounds__(kBlock) void scale_update_batched_kernel(ScaleUpdateBatch batch) {
  __shared__ uint32_t red[kBlock / 64];
  __shared__ uint32_t stage[kLdsEntries];
  const int t = blockIdx.x;
  float* h = batch.history[t];
  const int32_t len = batch.len[t], margin = batch.margin[t];
  float *s = batch.scale[t], *si = batch.scale_inv[t];
  if (batch.fmt[t] == FP8MP_E4M3) update_one<FP8MP_E4M3>(h, len, margin, s, si, stage, red);
  else if (batch.fmt[t] == FP8MP_E5M2) update_one<FP8MP_E5M2>(h, len, margin, s, si, stage, red);
  else update_one<FP8MP_FP16>(h, len, margin, s, si, stage, red);
}

}  // namespace

hipError_t launch_scale_update_batched(const ScaleUpdateBatch& batch, int n, hipStream_t stream) {
  hipLaunchKernelGGL(scale_update_batched_kernel, dim3(n), dim3(kBlock), 0, stream, batch);
  return hipGetLastError();
}

hipError_t launch_scale_update(float* history, int32_t len, fp8mp_format fmt, int32_t margin,
                               float* scale, float* scale_inv, hipStream_t stream) {
  if (fmt == FP8MP_E4M3)
    hipLaunchKernelGGL((scale_update_kernel<FP8MP_E4M3>), dim3(1), dim3(kBlock), 0, stream, history, len,
                       margin, scale, scale_inv);
  else if (fmt == FP8MP_FP16)
    hipLaunchKernelGGL((scale_update_kernel<FP8MP_FP16>), dim3(1), dim3(kBlock), 0, stream, history, len,
                       margin, scale, scale_inv);
  else
    hipLaunchKernelGGL((scale_update_kernel<FP8MP_E5M2>), dim3(1), dim3(kBlock), 0, stream, history, len,
                       margin, scale, scale_inv);
  return hipGetLastError();
}

}  // namespace fp8mp
