// C-ABI front end: argument validation, the gfx950 check and dispatch.
//
// Validation runs on the host before anything touches the device, so a bad
// argument returns FP8MP_ERR_INVALID_ARG even on a machine without a GPU.
// The only device query is the per-device arch check, cached after its first
// success. [TE] §FP8非対応GPUでのフォールバック実装 checks the device's capability at
// run time and falls back to 16-bit; here there is no fallback path: a device
// other than gfx950 gets FP8MP_ERR_WRONG_ARCH.
#include <atomic>
#include <cstdio>
#include <cstring>

#include <cmath>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unchecked, 1 = gfx950, 2 = another arch. CU count cached alongside.
std::atomic<int> g_arch_state[kMaxDevices];
std::atomic<int> g_num_cus[kMaxDevices];

// A C caller may pass any int where the header names an enum, and in C++ reading
// an out-of-range value as the enum type is undefined: the enum arguments are
// read through their object representation, as int, and checked as such.
template <class E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}
template <class E>
bool valid_format(const E& f) { return raw(f) == FP8MP_E4M3 || raw(f) == FP8MP_E5M2; }
template <class E>
bool valid_dtype(const E& d) { return raw(d) == FP8MP_F32 || raw(d) == FP8MP_BF16; }

fp8mp_status query_device(int* dev_out, hipDeviceProp_t* props_out) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return FP8MP_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8MP_ERR_HIP;
  *dev_out = dev;
  if (props_out && hipGetDeviceProperties(props_out, dev) != hipSuccess) return FP8MP_ERR_HIP;
  return FP8MP_OK;
}

// Ensures the current device is gfx950; returns its CU count through *cus.
fp8mp_status check_device(int* cus) {
  int dev = 0;
  fp8mp_status st = query_device(&dev, nullptr);
  if (st != FP8MP_OK) return st;
  if (dev >= 0 && dev < kMaxDevices) {
    const int s = g_arch_state[dev].load(std::memory_order_acquire);
    if (s == 1) {
      *cus = g_num_cus[dev].load(std::memory_order_relaxed);
      return FP8MP_OK;
    }
    if (s == 2) return FP8MP_ERR_WRONG_ARCH;
  }
  hipDeviceProp_t props;
  if (hipGetDeviceProperties(&props, dev) != hipSuccess) return FP8MP_ERR_HIP;
  const bool ok = std::strncmp(props.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < kMaxDevices) {
    g_num_cus[dev].store(props.multiProcessorCount, std::memory_order_relaxed);
    g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  }
  *cus = props.multiProcessorCount;
  return ok ? FP8MP_OK : FP8MP_ERR_WRONG_ARCH;
}

fp8mp_status from_hip(hipError_t e) { return e == hipSuccess ? FP8MP_OK : FP8MP_ERR_HIP; }

bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Host-side checks shared by the GEMM entry points (no device access).
fp8mp_status check_gemm(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b, fp8mp_format b_fmt,
                        int64_t ldb, int64_t m, int64_t n, int64_t k, const float* a_scale_inv,
                        const float* b_scale_inv, const uint16_t* c, int64_t ldc, bool c_optional = false) {
  if (!valid_format(a_fmt) || !valid_format(b_fmt)) return FP8MP_ERR_INVALID_ARG;
  if (m < 0 || n < 0 || k < 0) return FP8MP_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return FP8MP_OK;
  if ((c == nullptr && !c_optional) || a_scale_inv == nullptr || b_scale_inv == nullptr) return FP8MP_ERR_INVALID_ARG;
  if (k > 0 && (a == nullptr || b == nullptr)) return FP8MP_ERR_INVALID_ARG;
  if (lda < k || ldb < k || (c != nullptr && ldc < n)) return FP8MP_ERR_INVALID_ARG;
  if (!is_aligned(a_scale_inv, 4) || !is_aligned(b_scale_inv, 4)) return FP8MP_ERR_INVALID_ARG;
  if (k % 16 != 0) return FP8MP_ERR_UNSUPPORTED;
  // 16-byte copies of the operands and 16-byte stores of the output rows
  if (k > 0 && (lda % 16 != 0 || ldb % 16 != 0 || !is_aligned(a, 16) || !is_aligned(b, 16)))
    return FP8MP_ERR_INVALID_ARG;
  if (c != nullptr && (!is_aligned(c, 16) || ldc % 8 != 0)) return FP8MP_ERR_INVALID_ARG;
  // tile copies address at most 256 rows with 32-bit offsets
  if (k > 0 && (lda > fp8mp::kGemmMaxLd || ldb > fp8mp::kGemmMaxLd)) return FP8MP_ERR_UNSUPPORTED;
  // every row index product must stay inside int64 (lda, ldb may be 0 when k == 0)
  if ((lda > 0 && m > (INT64_MAX / 8) / lda) || (ldb > 0 && n > (INT64_MAX / 8) / ldb) ||
      (c != nullptr && m > (INT64_MAX / 8) / ldc))
    return FP8MP_ERR_UNSUPPORTED;
  // the launch's tile count must fit an int (each factor is checked first, so the product cannot overflow)
  const int64_t tiles_m = m / 128 + (m % 128 != 0), tiles_n = n / 128 + (n % 128 != 0);
  if (tiles_m > 0x7FFFFFFF || tiles_n > 0x7FFFFFFF || tiles_m * tiles_n > 0x7FFFFFFF) return FP8MP_ERR_UNSUPPORTED;
  return FP8MP_OK;
}

}  // namespace

extern "C" {

fp8mp_status fp8_amax_cast(const void* x, fp8mp_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           fp8mp_format fmt, const float* scale, uint8_t* q, int64_t ld_q, uint8_t* q_t,
                           int64_t ld_qt, float* amax, hipStream_t stream) {
  if (!valid_dtype(x_dtype) || !valid_format(fmt)) return FP8MP_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0) return FP8MP_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8MP_OK;
  if (x == nullptr || ld_x < cols) return FP8MP_ERR_INVALID_ARG;
  if ((q || q_t) && scale == nullptr) return FP8MP_ERR_INVALID_ARG;
  if (q && ld_q < cols) return FP8MP_ERR_INVALID_ARG;
  if (q_t && ld_qt < rows) return FP8MP_ERR_INVALID_ARG;
  if (amax && !is_aligned(amax, 4)) return FP8MP_ERR_INVALID_ARG;
  if (scale && !is_aligned(scale, 4)) return FP8MP_ERR_INVALID_ARG;
  // The kernels move 16-byte vectors: every data pointer is 16-byte aligned.
  if (!is_aligned(x, 16) || (q && !is_aligned(q, 16)) || (q_t && !is_aligned(q_t, 16))) return FP8MP_ERR_INVALID_ARG;
  // One contiguous run (flat kernels) or 16-byte aligned BF16 rows (tile kernel).
  const bool flat = (rows == 1 || (ld_x == cols && (!q || ld_q == cols))) && !q_t;
  if (!flat) {
    if (x_dtype != FP8MP_BF16) return FP8MP_ERR_UNSUPPORTED;   // fp32 sources: contiguous, no transposed copy
    if ((ld_x * 2) % 16 != 0 || (q && ld_q % 16 != 0) || (q_t && ld_qt % 16 != 0)) return FP8MP_ERR_INVALID_ARG;
  }
  // every row/column index product must stay inside int64
  if (rows > (INT64_MAX / 8) / ld_x) return FP8MP_ERR_UNSUPPORTED;
  if (q_t && cols > (INT64_MAX / 8) / ld_qt) return FP8MP_ERR_UNSUPPORTED;
  if (!q && !q_t && !amax) return FP8MP_OK;
  int cus = 0;
  fp8mp_status st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_amax_cast(x, x_dtype, rows, cols, ld_x, fmt, scale, q, ld_q, q_t, ld_qt,
                                          amax, cus, stream));
}

fp8mp_status fp8_amax_cast_batched(int32_t n_items, const fp8mp_cast_item* items, hipStream_t stream) {
  if (n_items < 0) return FP8MP_ERR_INVALID_ARG;
  if (n_items == 0) return FP8MP_OK;
  if (items == nullptr) return FP8MP_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_items; ++i) {
    const fp8mp_cast_item& it = items[i];
    if (!valid_dtype(it.x_dtype) || !valid_format(it.fmt) || it.numel < 0) return FP8MP_ERR_INVALID_ARG;
    if (it.numel == 0) continue;
    if (it.x == nullptr || (it.q && it.scale == nullptr)) return FP8MP_ERR_INVALID_ARG;
    if (!is_aligned(it.x, 16) || (it.q && !is_aligned(it.q, 16))) return FP8MP_ERR_INVALID_ARG;
    if ((it.amax && !is_aligned(it.amax, 4)) || (it.scale && !is_aligned(it.scale, 4))) return FP8MP_ERR_INVALID_ARG;
  }
  int cus = 0;
  fp8mp_status st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  fp8mp::CastBatch b{};
  auto flush = [&]() -> fp8mp_status {
    if (b.n == 0) return FP8MP_OK;
    fp8mp_status r = from_hip(fp8mp::launch_amax_cast_batched(b, cus, stream));
    b = fp8mp::CastBatch{};
    return r;
  };
  for (int32_t i = 0; i < n_items; ++i) {
    const fp8mp_cast_item& it = items[i];
    if (it.numel == 0 || (!it.q && !it.amax)) continue;
    if (it.x_dtype != FP8MP_BF16) {   // fp32 sources: their own flat kernel
      st = from_hip(fp8mp::launch_amax_cast(it.x, it.x_dtype, 1, it.numel, it.numel, it.fmt, it.scale, it.q,
                                            it.numel, nullptr, 0, it.amax, cus, stream));
      if (st != FP8MP_OK) return st;
      continue;
    }
    b.x[b.n] = it.x;
    b.q[b.n] = it.q;
    b.scale[b.n] = it.scale;
    b.amax[b.n] = it.amax;
    b.numel[b.n] = it.numel;
    b.fmt[b.n] = it.fmt;
    if (++b.n == fp8mp::kMaxCastBatch && (st = flush()) != FP8MP_OK) return st;
  }
  return flush();
}

fp8mp_status fp8_scale_update(float* amax_history, int32_t history_len, fp8mp_format fmt, int32_t margin,
                              float* scale, float* scale_inv, hipStream_t stream) {
  if (!valid_format(fmt) && raw(fmt) != FP8MP_FP16) return FP8MP_ERR_INVALID_ARG;
  if (amax_history == nullptr || scale == nullptr || scale_inv == nullptr) return FP8MP_ERR_INVALID_ARG;
  if (history_len < 1 || margin < 0) return FP8MP_ERR_INVALID_ARG;
  if (!is_aligned(amax_history, 4) || !is_aligned(scale, 4) || !is_aligned(scale_inv, 4))
    return FP8MP_ERR_INVALID_ARG;
  int cus = 0;
  fp8mp_status st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_scale_update(amax_history, history_len, fmt, margin, scale, scale_inv,
                                             stream));
}

fp8mp_status fp8_scale_update_batched(int32_t n_tensors, float* const* amax_histories, const int32_t* history_lens,
                                      const fp8mp_format* fmts, const int32_t* margins, float* const* scales,
                                      float* const* scale_invs, hipStream_t stream) {
  if (n_tensors < 0) return FP8MP_ERR_INVALID_ARG;
  if (n_tensors == 0) return FP8MP_OK;
  if (!amax_histories || !history_lens || !fmts || !margins || !scales || !scale_invs) return FP8MP_ERR_INVALID_ARG;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (!valid_format(fmts[t]) && raw(fmts[t]) != FP8MP_FP16) return FP8MP_ERR_INVALID_ARG;
    if (!amax_histories[t] || !scales[t] || !scale_invs[t]) return FP8MP_ERR_INVALID_ARG;
    if (history_lens[t] < 1 || margins[t] < 0) return FP8MP_ERR_INVALID_ARG;
    if (!is_aligned(amax_histories[t], 4) || !is_aligned(scales[t], 4) || !is_aligned(scale_invs[t], 4))
      return FP8MP_ERR_INVALID_ARG;
  }
  int cus = 0;
  fp8mp_status st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  for (int32_t t0 = 0; t0 < n_tensors; t0 += fp8mp::kMaxBatch) {
    const int n = n_tensors - t0 < fp8mp::kMaxBatch ? n_tensors - t0 : fp8mp::kMaxBatch;
    fp8mp::ScaleUpdateBatch b{};
    for (int i = 0; i < n; ++i) {
      b.history[i] = amax_histories[t0 + i];
      b.scale[i] = scales[t0 + i];
      b.scale_inv[i] = scale_invs[t0 + i];
      b.len[i] = history_lens[t0 + i];
      b.margin[i] = margins[t0 + i];
      b.fmt[i] = fmts[t0 + i];
    }
    st = from_hip(fp8mp::launch_scale_update_batched(b, n, stream));
    if (st != FP8MP_OK) return st;
  }
  return FP8MP_OK;
}

}  // extern "C"

namespace {

fp8mp_status scaled_gemm(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b, fp8mp_format b_fmt,
                         int64_t ldb, int64_t m, int64_t n, int64_t k, const float* a_scale_inv,
                         const float* b_scale_inv, uint16_t* c, int64_t ldc, bool fast_accum, hipStream_t stream) {
  fp8mp_status st = check_gemm(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc);
  if (st != FP8MP_OK || m == 0 || n == 0) return st;
  int cus = 0;
  st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_scaled_gemm(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv,
                                            c, ldc, fast_accum, cus, stream));
}

fp8mp_status scaled_gemm_amax_cast(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                                   fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                   const float* a_scale_inv, const float* b_scale_inv, uint16_t* c, int64_t ldc,
                                   fp8mp_format y_fmt, const float* y_scale, uint8_t* y_q, int64_t ld_yq,
                                   float* y_amax, bool fast_accum, hipStream_t stream) {
  fp8mp_status st = check_gemm(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc,
                               /*c_optional=*/y_q != nullptr || y_amax != nullptr);
  if (st != FP8MP_OK) return st;
  if (!valid_format(y_fmt)) return FP8MP_ERR_INVALID_ARG;
  if (y_q && (y_scale == nullptr || ld_yq < n)) return FP8MP_ERR_INVALID_ARG;
  if (y_q && (!is_aligned(y_q, 16) || ld_yq % 16 != 0)) return FP8MP_ERR_INVALID_ARG;
  if (y_scale && !is_aligned(y_scale, 4)) return FP8MP_ERR_INVALID_ARG;
  if (y_amax && !is_aligned(y_amax, 4)) return FP8MP_ERR_INVALID_ARG;
  if (y_q && m > (INT64_MAX / 8) / ld_yq) return FP8MP_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return FP8MP_OK;
  int cus = 0;
  st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_scaled_gemm_amax_cast(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv,
                                                      b_scale_inv, c, ldc, y_fmt, y_scale, y_q, ld_yq, y_amax,
                                                      fast_accum, cus, stream));
}

}  // namespace

extern "C" {

fp8mp_status fp8_scaled_gemm(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                             fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                             const float* a_scale_inv, const float* b_scale_inv, uint16_t* c, int64_t ldc,
                             hipStream_t stream) {
  return scaled_gemm(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc, false, stream);
}

fp8mp_status fp8_scaled_gemm_fast_accum(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                                        fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                        const float* a_scale_inv, const float* b_scale_inv, uint16_t* c,
                                        int64_t ldc, hipStream_t stream) {
  return scaled_gemm(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc, true, stream);
}

fp8mp_status fp8_scaled_gemm_amax_cast(const uint8_t* a, fp8mp_format a_fmt, int64_t lda, const uint8_t* b,
                                       fp8mp_format b_fmt, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                       const float* a_scale_inv, const float* b_scale_inv, uint16_t* c,
                                       int64_t ldc, fp8mp_format y_fmt, const float* y_scale, uint8_t* y_q,
                                       int64_t ld_yq, float* y_amax, hipStream_t stream) {
  return scaled_gemm_amax_cast(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc, y_fmt,
                               y_scale, y_q, ld_yq, y_amax, false, stream);
}

fp8mp_status fp8_scaled_gemm_amax_cast_fast_accum(const uint8_t* a, fp8mp_format a_fmt, int64_t lda,
                                                  const uint8_t* b, fp8mp_format b_fmt, int64_t ldb, int64_t m,
                                                  int64_t n, int64_t k, const float* a_scale_inv,
                                                  const float* b_scale_inv, uint16_t* c, int64_t ldc,
                                                  fp8mp_format y_fmt, const float* y_scale, uint8_t* y_q,
                                                  int64_t ld_yq, float* y_amax, hipStream_t stream) {
  return scaled_gemm_amax_cast(a, a_fmt, lda, b, b_fmt, ldb, m, n, k, a_scale_inv, b_scale_inv, c, ldc, y_fmt,
                               y_scale, y_q, ld_yq, y_amax, true, stream);
}

fp8mp_status fp8_layernorm_amax_cast(const void* x, fp8mp_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                     const float* gamma, const float* beta, float eps, uint16_t* y, int64_t ld_y,
                                     fp8mp_format fmt, const float* scale, uint8_t* q, int64_t ld_q, float* amax,
                                     float* mean, float* rstd, hipStream_t stream) {
  if (!valid_dtype(x_dtype) || !valid_format(fmt)) return FP8MP_ERR_INVALID_ARG;
  if (rows < 0 || cols <= 0 || cols > INT32_MAX) return FP8MP_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps == INFINITY) return FP8MP_ERR_INVALID_ARG;   // also rejects NaN
  if (rows == 0) return FP8MP_OK;
  if (x == nullptr || gamma == nullptr || ld_x < cols) return FP8MP_ERR_INVALID_ARG;
  if (y && ld_y < cols) return FP8MP_ERR_INVALID_ARG;
  if (q && (scale == nullptr || ld_q < cols)) return FP8MP_ERR_INVALID_ARG;
  if (!is_aligned(x, x_dtype == FP8MP_BF16 ? 2 : 4) || !is_aligned(gamma, 4) || (beta && !is_aligned(beta, 4)))
    return FP8MP_ERR_INVALID_ARG;
  if ((y && !is_aligned(y, 2)) || (scale && !is_aligned(scale, 4)) || (amax && !is_aligned(amax, 4)) ||
      (mean && !is_aligned(mean, 4)) || (rstd && !is_aligned(rstd, 4)))
    return FP8MP_ERR_INVALID_ARG;
  if (rows > (INT64_MAX / 8) / ld_x || (y && rows > (INT64_MAX / 8) / ld_y) || (q && rows > (INT64_MAX / 8) / ld_q))
    return FP8MP_ERR_UNSUPPORTED;
  if (!y && !q && !amax && !mean && !rstd) return FP8MP_OK;
  int cus = 0;
  fp8mp_status st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_layernorm_amax_cast(x, x_dtype, rows, cols, ld_x, gamma, beta, eps, y, ld_y, fmt,
                                                    scale, q, ld_q, amax, mean, rstd, cus, stream));
}

fp8mp_status fp8_reduce_shared_scale(const uint8_t* q, fp8mp_format fmt, int32_t n_ranks, int64_t numel,
                                     int64_t rank_stride, const float* scale_inv, void* out, fp8mp_dtype out_dtype,
                                     hipStream_t stream) {
  if (!valid_format(fmt) || !valid_dtype(out_dtype)) return FP8MP_ERR_INVALID_ARG;
  if (n_ranks < 1 || numel < 0 || rank_stride < numel) return FP8MP_ERR_INVALID_ARG;
  if (numel == 0) return FP8MP_OK;
  if (q == nullptr || scale_inv == nullptr || out == nullptr) return FP8MP_ERR_INVALID_ARG;
  if (!is_aligned(scale_inv, 4) || !is_aligned(out, out_dtype == FP8MP_BF16 ? 2 : 4)) return FP8MP_ERR_INVALID_ARG;
  if (n_ranks > 1 && rank_stride > (INT64_MAX / 2) / (n_ranks - 1)) return FP8MP_ERR_UNSUPPORTED;
  int cus = 0;
  fp8mp_status st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_reduce_shared_scale(q, fmt, n_ranks, numel, rank_stride, scale_inv, out, out_dtype,
                                                    cus, stream));
}

namespace {

// Validation shared by both Adam entry points (no device access).
fp8mp_status check_adam(int64_t n, const void* grad, fp8mp_dtype grad_dtype, uint8_t* m_q, const float* m_dq_in,
                        float* m_dq_out, const float* m_scale, const float* m_scale_inv, float* m_amax, uint16_t* v,
                        uint16_t* w, const float* w_dq_in, float* w_dq_out, const float* w_scale,
                        const float* w_scale_inv, float* w_amax, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int64_t step) {
  if (!valid_dtype(grad_dtype) || n < 0) return FP8MP_ERR_INVALID_ARG;
  if (step < 1 || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f)) return FP8MP_ERR_INVALID_ARG;
  const void* required[] = {grad, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, v, w, w_dq_in, w_dq_out,
                            w_scale, w_scale_inv};
  for (const void* p : required)
    if (p == nullptr) return FP8MP_ERR_INVALID_ARG;
  if (m_dq_out == m_dq_in || w_dq_out == w_dq_in || m_dq_out == w_dq_out) return FP8MP_ERR_INVALID_ARG;
  const float* scalars[] = {m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, w_dq_in, w_dq_out, w_scale, w_scale_inv,
                            w_amax};
  for (const float* p : scalars)
    if (p != nullptr && !is_aligned(p, 4)) return FP8MP_ERR_INVALID_ARG;
  if (!is_aligned(grad, grad_dtype == FP8MP_BF16 ? 2 : 4) || !is_aligned(v, 2) || !is_aligned(w, 2))
    return FP8MP_ERR_INVALID_ARG;
  const float hp[] = {lr, beta1, beta2, eps, weight_decay};
  for (float x : hp)
    if (!std::isfinite(x)) return FP8MP_ERR_INVALID_ARG;
  return FP8MP_OK;
}

// Adam's bias correction 1 / (1 - beta^t), formed in binary64 from the binary32
// beta and rounded once to binary32 (finite for 0 <= beta < 1 and t >= 1).
float bias_correction(float beta, int64_t step) {
  return (float)(1.0 / (1.0 - std::pow((double)beta, (double)step)));
}

}  // namespace

fp8mp_status fp8_adam_step(int64_t n, const void* grad, fp8mp_dtype grad_dtype, uint8_t* m_q, const float* m_dq_in,
                           float* m_dq_out, const float* m_scale, const float* m_scale_inv, float* m_amax,
                           uint16_t* v, uint16_t* w, const float* w_dq_in, float* w_dq_out, const float* w_scale,
                           const float* w_scale_inv, float* w_amax, float lr, float beta1, float beta2, float eps,
                           float weight_decay, int64_t step, hipStream_t stream) {
  fp8mp_status st = check_adam(n, grad, grad_dtype, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, v, w,
                               w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, lr, beta1, beta2, eps, weight_decay,
                               step);
  if (st != FP8MP_OK || n == 0) return st;
  int cus = 0;
  st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_adam_step(n, grad, grad_dtype, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax,
                                          v, w, w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, lr, beta1, beta2,
                                          eps, weight_decay, bias_correction(beta1, step),
                                          bias_correction(beta2, step), -1, nullptr, nullptr, nullptr, cus,
                                          stream));
}

fp8mp_status fp8_adam_step_weight_cast(int64_t n, const void* grad, fp8mp_dtype grad_dtype, uint8_t* m_q,
                                       const float* m_dq_in, float* m_dq_out, const float* m_scale,
                                       const float* m_scale_inv, float* m_amax, uint16_t* v, uint16_t* w,
                                       const float* w_dq_in, float* w_dq_out, const float* w_scale,
                                       const float* w_scale_inv, float* w_amax, float lr, float beta1, float beta2,
                                       float eps, float weight_decay, int64_t step, fp8mp_format wq_fmt, const float* wq_scale, uint8_t* wq, float* wq_amax,
                                       hipStream_t stream) {
  fp8mp_status st = check_adam(n, grad, grad_dtype, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, v, w,
                               w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, lr, beta1, beta2, eps, weight_decay,
                               step);
  if (st != FP8MP_OK) return st;
  if (!valid_format(wq_fmt) || (wq == nullptr && wq_amax == nullptr) || (wq != nullptr && wq_scale == nullptr))
    return FP8MP_ERR_INVALID_ARG;
  if ((wq_scale != nullptr && !is_aligned(wq_scale, 4)) || (wq_amax != nullptr && !is_aligned(wq_amax, 4)))
    return FP8MP_ERR_INVALID_ARG;
  if (n == 0) return FP8MP_OK;
  int cus = 0;
  st = check_device(&cus);
  if (st != FP8MP_OK) return st;
  return from_hip(fp8mp::launch_adam_step(n, grad, grad_dtype, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax,
                                          v, w, w_dq_in, w_dq_out, w_scale, w_scale_inv, w_amax, lr, beta1, beta2,
                                          eps, weight_decay, bias_correction(beta1, step),
                                          bias_correction(beta2, step), wq_fmt, wq_scale, wq, wq_amax, cus,
                                          stream));
}

const char* fp8mp_status_string(fp8mp_status status) {
  switch (raw(status)) {
    case FP8MP_OK: return "ok";
    case FP8MP_ERR_INVALID_ARG: return "invalid argument";
    case FP8MP_ERR_UNSUPPORTED: return "unsupported shape, layout or alignment";
    case FP8MP_ERR_NO_DEVICE: return "no HIP device";
    case FP8MP_ERR_WRONG_ARCH: return "device is not gfx950";
    case FP8MP_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

fp8mp_status fp8mp_device_info(char* buf, size_t len) {
  if (buf == nullptr || len == 0) return FP8MP_ERR_INVALID_ARG;
  buf[0] = '\0';
  int dev = 0;
  hipDeviceProp_t props;
  fp8mp_status st = query_device(&dev, &props);
  if (st != FP8MP_OK) return st;
  std::snprintf(buf, len, "arch=%s cus=%d formats=e4m3:448,e5m2:57344", props.gcnArchName,
                props.multiProcessorCount);
  return std::strncmp(props.gcnArchName, "gfx950", 6) == 0 ? FP8MP_OK : FP8MP_ERR_WRONG_ARCH;
}

}  // extern "C"
