// One Adam step over decoupled-precision optimizer state, in one pass:
// the first moment m as E4M3 codes with a per-tensor scale, the second moment
// v as FP16, the master weights w as FP16 values of w * s_w (tensor scaling).
//
// [MPT] §定義 (precision sensitivity of training variables) and §横断的知見
// "精度分離 (Precision Decoupling)": master weights and the second moment need
// high precision, the first moment tolerates FP8; FP8-LM keeps m in FP8, v in
// FP16 and w in FP16 with tensor scaling (6 bytes per parameter instead of
// 16). Both scales follow the delayed recipe: the step writes with the
// current scale and records the new tensor's amax for the next update.
//
// Per element, in binary32, in this order (contraction off):
//   g = grad; m = dec(m_q) * m_dq; v = float(v); w = float(w) * w_dq
//   m = beta1 * m + (1 - beta1) * g
//   v = beta2 * v + (1 - beta2) * (g * g)
//   u = (m * c1) / (sqrt(v * c2) + eps)
//   w = w - lr * (u + wd * w)
//   m_q = enc_e4m3(m * m_scale); v = fp16(v); w = fp16(w * w_scale)
// FP16 stores round to nearest even and saturate at +-65504. HBM traffic per
// parameter: grad 2 (BF16) or 4, m 1 + 1, v 2 + 2, w 2 + 2 bytes.
//
// With WQF (a format) the same pass also writes the next forward's weight
// codes from the master weights as stored: W = fp32(fp16 w) * w_scale_inv
// (what the next step reads back), wq = enc_WQF(W * wq_scale), and records
// max |W| for that tensor's own delayed scale: one more byte per parameter
// instead of a separate pass that reads the 2-byte master weights again.
#include "common.h"

namespace fp8mp {
namespace {

constexpr int kAdamBlock = 256;
constexpr float kFp16Max = 65504.0f;

typedef float v2f __attribute__((ext_vector_type(2)));

struct AdamHp {
  float lr, beta1, beta2, eps, wd, c1, c2;
};

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Round to nearest even, saturating: clamp first (every value beyond 65504
// rounds to 65504 or overflows), NaN passes through.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float x) {
  const float c = x != x ? x : __builtin_amdgcn_fmed3f(x, -kFp16Max, kFp16Max);
  return __builtin_bit_cast(uint16_t, (_Float16)c);
}

// The step for one element; returns m and w (binary32) for the amaxes.
__device__ __forceinline__ void adam_elem(float g, float& m, float& v, float& w, const AdamHp& hp) {
  m = hp.beta1 * m + (1.0f - hp.beta1) * g;
  v = hp.beta2 * v + (1.0f - hp.beta2) * (g * g);
  const float u = (m * hp.c1) / (sqrtf(v * hp.c2) + hp.eps);
  w = w - hp.lr * (u + hp.wd * w);
}

template <int GD>
__device__ __forceinline__ float load_grad(const void* grad, int64_t i) {
  if constexpr (GD == FP8MP_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(grad)[i] << 16);
  return static_cast<const float*>(grad)[i];
}

// No forward weight codes (WQF of the plain step).
constexpr int kNoWq = -1;

// The forward weight codes' outputs.
struct WqOut {
  const float* scale;   // the forward weight's scale in force (read)
  uint8_t* q;           // n codes or NULL
  float* amax;          // max |W| accumulated, or NULL
};

template <int GD, int WQF>
__global__ __launch_bounds__(kAdamBlock) void adam_kernel(
    int64_t n, const void* __restrict__ grad, uint8_t* __restrict__ m_q, const float* __restrict__ m_dq_in,
    float* __restrict__ m_dq_out, const float* __restrict__ m_scale, const float* __restrict__ m_scale_inv,
    float* __restrict__ m_amax, uint16_t* __restrict__ v16, uint16_t* __restrict__ w16,
    const float* __restrict__ w_dq_in, float* __restrict__ w_dq_out, const float* __restrict__ w_scale,
    const float* __restrict__ w_scale_inv, float* __restrict__ w_amax, AdamHp hp, int vec, WqOut wqo) {
  const float mdq = *m_dq_in, wdq = *w_dq_in, ms = *m_scale, ws = *w_scale;
  float wsi = 0.f, qs = 0.f;
  if constexpr (WQF != kNoWq) {
    wsi = *w_scale_inv;
    qs = wqo.q != nullptr ? *wqo.scale : 0.f;
  }
  const int64_t tid = (int64_t)blockIdx.x * kAdamBlock + threadIdx.x, nthreads = (int64_t)gridDim.x * kAdamBlock;
  uint32_t am_m = 0, am_w = 0, am_q = 0;
  int64_t start = 0;
  if (vec) {
    // Eight parameters per thread and iteration: 16 B of BF16 gradient (32 B
    // of FP32), 8 B of m codes, 16 B each of v and w.
    const int64_t n8 = n / 8;
    for (int64_t c = tid; c < n8; c += nthreads) {
      float g[8];
      if constexpr (GD == FP8MP_BF16) {
        const uint4 gw = reinterpret_cast<const uint4*>(grad)[c];
        const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          g[2 * k] = bf16_lo(gg[k]);
          g[2 * k + 1] = bf16_hi(gg[k]);
        }
      } else {
        const float4 g0 = reinterpret_cast<const float4*>(grad)[2 * c];
        const float4 g1 = reinterpret_cast<const float4*>(grad)[2 * c + 1];
        g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
        g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
      }
      const uint2 mq = reinterpret_cast<const uint2*>(m_q)[c];
      const uint4 vv = reinterpret_cast<const uint4*>(v16)[c];
      const uint4 wv = reinterpret_cast<const uint4*>(w16)[c];
      const uint32_t mw[2] = {mq.x, mq.y}, vw[4] = {vv.x, vv.y, vv.z, vv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
      float m[8], v[8], w[8];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)mw[k], false);
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)mw[k], true);
        m[4 * k] = lo[0] * mdq;
        m[4 * k + 1] = lo[1] * mdq;
        m[4 * k + 2] = hi[0] * mdq;
        m[4 * k + 3] = hi[1] * mdq;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = f16_to_f32((uint16_t)(vw[k] & 0xFFFFu));
        v[2 * k + 1] = f16_to_f32((uint16_t)(vw[k] >> 16));
        w[2 * k] = f16_to_f32((uint16_t)(ww[k] & 0xFFFFu)) * wdq;
        w[2 * k + 1] = f16_to_f32((uint16_t)(ww[k] >> 16)) * wdq;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        adam_elem(g[e], m[e], v[e], w[e], hp);
        am_m = amax_f32(am_m, m[e]);
        am_w = amax_f32(am_w, w[e]);
      }
      reinterpret_cast<uint2*>(m_q)[c] =
          uint2{enc4<FP8MP_E4M3>(m[0], m[1], m[2], m[3], ms), enc4<FP8MP_E4M3>(m[4], m[5], m[6], m[7], ms)};
      uint32_t vo[4], wo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vo[k] = (uint32_t)f32_to_f16_sat(v[2 * k]) | ((uint32_t)f32_to_f16_sat(v[2 * k + 1]) << 16);
        wo[k] = (uint32_t)f32_to_f16_sat(w[2 * k] * ws) | ((uint32_t)f32_to_f16_sat(w[2 * k + 1] * ws) << 16);
      }
      reinterpret_cast<uint4*>(v16)[c] = uint4{vo[0], vo[1], vo[2], vo[3]};
      reinterpret_cast<uint4*>(w16)[c] = uint4{wo[0], wo[1], wo[2], wo[3]};
      if constexpr (WQF != kNoWq) {
        float W[8];   // the master weights as stored, read back
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          W[2 * k] = f16_to_f32((uint16_t)(wo[k] & 0xFFFFu)) * wsi;
          W[2 * k + 1] = f16_to_f32((uint16_t)(wo[k] >> 16)) * wsi;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) am_q = amax_f32(am_q, W[e]);
        if (wqo.q != nullptr)
          reinterpret_cast<uint2*>(wqo.q)[c] =
              uint2{enc4<WQF>(W[0], W[1], W[2], W[3], qs), enc4<WQF>(W[4], W[5], W[6], W[7], qs)};
      }
    }
    start = n8 * 8;
  }
  for (int64_t i = start + tid; i < n; i += nthreads) {
    const float g = load_grad<GD>(grad, i);
    float m = __builtin_amdgcn_cvt_pk_f32_fp8((int)m_q[i], false)[0] * mdq;
    float v = f16_to_f32(v16[i]);
    float w = f16_to_f32(w16[i]) * wdq;
    adam_elem(g, m, v, w, hp);
    am_m = amax_f32(am_m, m);
    am_w = amax_f32(am_w, w);
    m_q[i] = enc1<FP8MP_E4M3>(m, ms);
    v16[i] = f32_to_f16_sat(v);
    const uint16_t wh = f32_to_f16_sat(w * ws);
    w16[i] = wh;
    if constexpr (WQF != kNoWq) {
      const float W = f16_to_f32(wh) * wsi;
      am_q = amax_f32(am_q, W);
      if (wqo.q != nullptr) wqo.q[i] = enc1<WQF>(W, qs);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // the inverses of the scales this step wrote with, for the next step's reads
    *m_dq_out = *m_scale_inv;
    *w_dq_out = *w_scale_inv;
  }
  if (m_amax != nullptr) block_amax_commit<kAdamBlock>(am_m, m_amax);
  if (w_amax != nullptr) {
    __syncthreads();   // the block reduction's shared slots are reused
    block_amax_commit<kAdamBlock>(am_w, w_amax);
  }
  if constexpr (WQF != kNoWq) {
    if (wqo.amax != nullptr) {
      __syncthreads();
      block_amax_commit<kAdamBlock>(am_q, wqo.amax);
    }
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int GD, int WQF>
void launch_kernel(int grid, hipStream_t stream, int64_t n, const void* grad, uint8_t* m_q, const float* m_dq_in,
                   float* m_dq_out, const float* m_scale, const float* m_scale_inv, float* m_amax, uint16_t* v,
                   uint16_t* w, const float* w_dq_in, float* w_dq_out, const float* w_scale, const float* w_scale_inv,
                   float* w_amax, const AdamHp& hp, int vec, const WqOut& wqo) {
  hipLaunchKernelGGL((adam_kernel<GD, WQF>), dim3(grid), dim3(kAdamBlock), 0, stream, n, grad, m_q, m_dq_in, m_dq_out,
                     m_scale, m_scale_inv, m_amax, v, w, w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, hp, vec,
                     wqo);
}

template <int WQF>
hipError_t launch_fmt(int64_t n, const void* grad, fp8mp_dtype grad_dtype, uint8_t* m_q, const float* m_dq_in,
                      float* m_dq_out, const float* m_scale, const float* m_scale_inv, float* m_amax, uint16_t* v,
                      uint16_t* w, const float* w_dq_in, float* w_dq_out, const float* w_scale,
                      const float* w_scale_inv, float* w_amax, const AdamHp& hp, const WqOut& wqo, int num_cus,
                      hipStream_t stream) {
  const int vec = aligned(grad, 16) && aligned(m_q, 8) && aligned(v, 16) && aligned(w, 16) &&
                  (wqo.q == nullptr || aligned(wqo.q, 8));
  const int64_t work = vec ? (n + 7) / 8 : n;
  const int64_t need = (work + kAdamBlock - 1) / kAdamBlock;
  const int64_t cap = (int64_t)num_cus * 4;
  const int grid = (int)(need < cap ? (need > 0 ? need : 1) : cap);
  if (grad_dtype == FP8MP_BF16)
    launch_kernel<FP8MP_BF16, WQF>(grid, stream, n, grad, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, v, w,
                                   w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, hp, vec, wqo);
  else
    launch_kernel<FP8MP_F32, WQF>(grid, stream, n, grad, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, v, w,
                                  w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, hp, vec, wqo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_adam_step(int64_t n, const void* grad, fp8mp_dtype grad_dtype, uint8_t* m_q, const float* m_dq_in,
                            float* m_dq_out, const float* m_scale, const float* m_scale_inv, float* m_amax,
                            uint16_t* v, uint16_t* w, const float* w_dq_in, float* w_dq_out, const float* w_scale,
                            const float* w_scale_inv, float* w_amax, float lr, float beta1, float beta2, float eps,
                            float weight_decay, float bias_c1, float bias_c2, int wq_fmt, const float* wq_scale,
                            uint8_t* wq, float* wq_amax, int num_cus, hipStream_t stream) {
  const AdamHp hp{lr, beta1, beta2, eps, weight_decay, bias_c1, bias_c2};
  const WqOut wqo{wq_scale, wq, wq_amax};
  const bool with_wq = wq != nullptr || wq_amax != nullptr;
#define FP8MP_ADAM(WQF)                                                                                              \
  launch_fmt<WQF>(n, grad, grad_dtype, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, v, w, w_dq_in, w_dq_out, \
                  w_scale, w_scale_inv, w_amax, hp, wqo, num_cus, stream)
  if (!with_wq) return FP8MP_ADAM(kNoWq);
  if (wq_fmt == FP8MP_E5M2) return FP8MP_ADAM(FP8MP_E5M2);
  return FP8MP_ADAM(FP8MP_E4M3);
#undef FP8MP_ADAM
}

}  // namespace fp8mp
