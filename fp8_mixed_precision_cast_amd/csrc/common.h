// Shared pieces of the HIP kernels: FP8 format constants, the saturating
// round-to-nearest-even conversion, and amax helpers. gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8mp.h"

namespace fp8mp {

// Largest finite value and its code per format. [MPT] §定義 precision table:
// E4M3 tops out at 448, E5M2 at 57344.
template <int FMT> struct Fp8Traits;
template <> struct Fp8Traits<FP8MP_E4M3> {
  static constexpr float kMax = 448.0f;
  static constexpr uint32_t kMaxBits = 0x43E00000u;   // 448.0f
};
template <> struct Fp8Traits<FP8MP_E5M2> {
  static constexpr float kMax = 57344.0f;
  static constexpr uint32_t kMaxBits = 0x47600000u;   // 57344.0f
};
// Tensor-scaled FP16 storage (scale updates only): [MPT] §定義 table, 65504.
template <> struct Fp8Traits<FP8MP_FP16> {
  static constexpr float kMax = 65504.0f;
  static constexpr uint32_t kMaxBits = 0x477FE000u;   // 65504.0f
};

// Clamp to [-fmax, fmax] so the hardware conversion never overflows (it is
// not saturating: 512 would become the E4M3 NaN code). Infinities clamp to
// +-fmax, which is the saturating reading for them. A NaN input comes out of
// fmed3 as one of the bounds; enc4 replaces its code afterwards.
template <int FMT>
__device__ __forceinline__ float sat_clamp(float p) {
  constexpr float m = Fp8Traits<FMT>::kMax;
  return __builtin_amdgcn_fmed3f(p, -m, m);
}

// Four clamped fp32 values -> four FP8 codes, byte i from argument i. gfx950's
// v_cvt_pk_{fp8,bf8}_f32 produce OCP codes and round to nearest even (the MODE
// register's default rounding).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r = 0;
  if constexpr (FMT == FP8MP_E4M3) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, r, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, r, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  }
  return static_cast<uint32_t>(r);
}

// The code of a NaN product x * s: 0x7F with the sign the product would have,
// sign(x) xor sign(s). (The hardware conversion always writes 0xFF / 0xFE.)
__device__ __forceinline__ uint32_t nan_code(float x, float s) {
  return 0x7Fu | (((__float_as_uint(x) ^ __float_as_uint(s)) >> 24) & 0x80u);
}

// q = enc(x * s) for four fp32 sources. NaN products are rare, so they are
// detected per group of four and patched on a side path.
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float x0, float x1, float x2, float x3, float s) {
  const float p0 = x0 * s, p1 = x1 * s, p2 = x2 * s, p3 = x3 * s;
  uint32_t r = cvt4<FMT>(sat_clamp<FMT>(p0), sat_clamp<FMT>(p1), sat_clamp<FMT>(p2), sat_clamp<FMT>(p3));
  const bool n0 = p0 != p0, n1 = p1 != p1, n2 = p2 != p2, n3 = p3 != p3;
  if (__builtin_expect(n0 | n1 | n2 | n3, 0)) {
    if (n0) r = (r & 0xFFFFFF00u) | nan_code(x0, s);
    if (n1) r = (r & 0xFFFF00FFu) | (nan_code(x1, s) << 8);
    if (n2) r = (r & 0xFF00FFFFu) | (nan_code(x2, s) << 16);
    if (n3) r = (r & 0x00FFFFFFu) | (nan_code(x3, s) << 24);
  }
  return r;
}

// enc4 without the side path: NaN bytes are patched with selects, so the
// code is straight-line (for epilogues that convert many groups in a row).
template <int FMT>
__device__ __forceinline__ uint32_t enc4_sel(float x0, float x1, float x2, float x3, float s) {
  const float p0 = x0 * s, p1 = x1 * s, p2 = x2 * s, p3 = x3 * s;
  uint32_t r = cvt4<FMT>(sat_clamp<FMT>(p0), sat_clamp<FMT>(p1), sat_clamp<FMT>(p2), sat_clamp<FMT>(p3));
  r = p0 != p0 ? (r & 0xFFFFFF00u) | nan_code(x0, s) : r;
  r = p1 != p1 ? (r & 0xFFFF00FFu) | (nan_code(x1, s) << 8) : r;
  r = p2 != p2 ? (r & 0xFF00FFFFu) | (nan_code(x2, s) << 16) : r;
  r = p3 != p3 ? (r & 0x00FFFFFFu) | (nan_code(x3, s) << 24) : r;
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two BF16 words (four values) -> four codes.
template <int FMT>
__device__ __forceinline__ uint32_t enc4_bf16(uint32_t w0, uint32_t w1, float s) {
  return enc4<FMT>(bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1), s);
}

template <int FMT>
__device__ __forceinline__ uint32_t enc4_bf16_sel(uint32_t w0, uint32_t w1, float s) {
  return enc4_sel<FMT>(bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1), s);
}

// Four BF16 values -> four codes when no product can be NaN (no NaN source,
// and s finite and nonzero, so neither 0 * Inf nor Inf * 0 occurs).
template <int FMT>
__device__ __forceinline__ uint32_t enc4_bf16_nonan(uint32_t w0, uint32_t w1, float s) {
  return cvt4<FMT>(sat_clamp<FMT>(bf16_lo(w0) * s), sat_clamp<FMT>(bf16_hi(w0) * s), sat_clamp<FMT>(bf16_lo(w1) * s),
                   sat_clamp<FMT>(bf16_hi(w1) * s));
}

// One source value -> one code (edge paths).
template <int FMT>
__device__ __forceinline__ uint8_t enc1(float x, float s) {
  return static_cast<uint8_t>(enc4<FMT>(x, 0.f, 0.f, 0.f, s) & 0xFFu);
}

// amax is kept as the unsigned bit pattern of |x|: for non-negative floats the
// unsigned order is the numeric order, +Inf sits above every finite value and
// every NaN pattern sits above +Inf, so an unsigned max propagates NaN.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running max over packed BF16 magnitudes (two lanes of 16 bits).
__device__ __forceinline__ uint32_t amax_bf16x2(uint32_t acc, uint32_t w) {
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t bf16x2_acc_to_f32_bits(uint32_t acc) {
  uint32_t lo = acc & 0xFFFFu, hi = acc >> 16;
  return (lo > hi ? lo : hi) << 16;
}

__device__ __forceinline__ uint32_t amax_f32(uint32_t acc, float x) {
  uint32_t b = __float_as_uint(x) & 0x7FFFFFFFu;
  return acc > b ? acc : b;
}

__device__ __forceinline__ uint32_t canonical_nan(uint32_t m) {
  return m > 0x7F800000u ? 0x7FC00000u : m;
}

// Block-wide unsigned max, then at most one atomic per block into *amax.
template <int BLOCK>
__device__ __forceinline__ void block_amax_commit(uint32_t m, float* amax) {
  __shared__ uint32_t red[BLOCK / 64];
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < BLOCK / 64; ++w) r = r > red[w] ? r : red[w];
    r = canonical_nan(r);
    // amax only grows, so a block whose max does not exceed the value already
    // there has nothing to add: the atomic is skipped. Same-address atomics
    // serialize in L2, and most blocks end up skipping once a large value
    // has landed.
    unsigned int* a = reinterpret_cast<unsigned int*>(amax);
    if (r != 0u && r > __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(a, r);
  }
}

// Up to kMaxCastBatch contiguous BF16 tensors cast in one launch.
constexpr int kMaxCastBatch = 8;
struct CastBatch {
  const void* x[kMaxCastBatch];
  void* q[kMaxCastBatch];
  const float* scale[kMaxCastBatch];
  float* amax[kMaxCastBatch];
  int64_t numel[kMaxCastBatch];
  int32_t fmt[kMaxCastBatch];
  int32_t block_start[kMaxCastBatch + 1];
  int32_t n;
};
hipError_t launch_amax_cast_batched(CastBatch& batch, int num_cus, hipStream_t stream);

// Largest GEMM leading dimension in bytes: a 256-row tile then spans less
// than 2^30 bytes, so its copies use 32-bit buffer offsets.
constexpr int64_t kGemmMaxLd = int64_t(1) << 22;

// Launchers (host side), one translation unit each.
hipError_t launch_amax_cast(const void* x, fp8mp_dtype dt, int64_t rows, int64_t cols, int64_t ld_x,
                            fp8mp_format fmt, const float* scale, uint8_t* q, int64_t ld_q,
                            uint8_t* q_t, int64_t ld_qt, float* amax, int num_cus,
                            hipStream_t stream);
hipError_t launch_scale_update(float* history, int32_t len, fp8mp_format fmt, int32_t margin,
                               float* scale, float* scale_inv, hipStream_t stream);
// Up to kMaxBatch tensors' recipe state, passed by value to one launch.
constexpr int kMaxBatch = 16;
struct ScaleUpdateBatch {
  float* history[kMaxBatch];
  float* scale[kMaxBatch];
  float* scale_inv[kMaxBatch];
  int32_t len[kMaxBatch];
  int32_t margin[kMaxBatch];
  int32_t fmt[kMaxBatch];
};
hipError_t launch_scale_update_batched(const ScaleUpdateBatch& batch, int n, hipStream_t stream);
hipError_t launch_scaled_gemm(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                              fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                              const float* a_scale_inv, const float* b_scale_inv, uint16_t* c,
                              int64_t ldc, bool fast_accum, int num_cus, hipStream_t stream);
hipError_t launch_scaled_gemm_amax_cast(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                                        fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                        const float* a_scale_inv, const float* b_scale_inv, uint16_t* c,
                                        int64_t ldc, fp8mp_format y_fmt, const float* y_scale, uint8_t* y_q,
                                        int64_t ld_yq, float* y_amax, bool fast_accum, int num_cus,
                                        hipStream_t stream);
hipError_t launch_layernorm_amax_cast(const void* x, fp8mp_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                      const float* gamma, const float* beta, float eps, uint16_t* y, int64_t ld_y,
                                      fp8mp_format fmt, const float* scale, uint8_t* q, int64_t ld_q, float* amax,
                                      float* mean, float* rstd, int num_cus, hipStream_t stream);
hipError_t launch_adam_step(int64_t n, const void* grad, fp8mp_dtype grad_dtype, uint8_t* m_q, const float* m_dq_in,
                            float* m_dq_out, const float* m_scale, const float* m_scale_inv, float* m_amax,
                            uint16_t* v, uint16_t* w, const float* w_dq_in, float* w_dq_out, const float* w_scale,
                            const float* w_scale_inv, float* w_amax, float lr, float beta1, float beta2, float eps,
                            float weight_decay, float bias_c1, float bias_c2, int wq_fmt, const float* wq_scale,
                            uint8_t* wq, float* wq_amax, int num_cus, hipStream_t stream);
hipError_t launch_reduce_shared_scale(const uint8_t* q, fp8mp_format fmt, int32_t n_ranks, int64_t numel,
                                      int64_t rank_stride, const float* scale_inv, void* out,
                                      fp8mp_dtype out_dtype, int num_cus, hipStream_t stream);

}  // namespace fp8mp
