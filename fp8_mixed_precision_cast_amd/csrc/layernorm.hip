// LayerNorm over the rows of x, with the amax and the FP8 cast of its BF16
// output in the same pass.
//
// [TE] §基本的なFP8トレーニングコードの構成: the LayerNorm module is swapped for its
// FP8-aware counterpart along with the linear layer it feeds. The textbook
// LayerNorm over the contiguous (last) dimension:
//   mu = mean(x), var = mean((x - mu)^2), rstd = 1 / sqrt(var + eps),
//   y = (x - mu) * rstd * gamma + beta,
// evaluated in FP32 and rounded to BF16. The cast then applies to that BF16
// output exactly what fp8_amax_cast applies to a BF16 tensor: amax = max |y|
// and q = enc(y * scale) ([TE] §動的スケーリングとFP8レシピの設定: the next layer's
// operand is cast with its delayed scale, its amax goes into its history).
//
// Register path (BF16 rows, 16-byte aligned, cols a multiple of 8 and at most
// 16384): one, two or four waves per row, at most eight 16-byte chunks per
// thread, held in registers, so the row is read from HBM once; the two row
// sums (mean, then squared deviations) are per-thread runs followed by a
// butterfly whose result every lane shares (and, across waves, an LDS sum). HBM traffic is 2 B read + 2 B (y) + 1 B (q)
// per element. Anything else (fp32 rows, odd strides, longer rows) takes the
// generic path: one workgroup per row, three strided passes over the row.
#include "common.h"

namespace fp8mp {
namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kLnBlock = 256;
constexpr int kLnRows = kLnBlock / 64;   // rows per workgroup on the register path
constexpr int kNoQ = -1;                 // neither codes nor amax
constexpr int kMaxChunksPerThread = 8;   // register path: cols <= 4 waves * 64 * 8 chunks * 8

__device__ __forceinline__ float wave_sum(float v) {
  // Butterfly: at every level lane l adds lane l ^ off's partial; addition is
  // commutative, so all lanes end with the same sum.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// An empty asm that claims to rewrite the packed row: each phase then widens
// the BF16 values again from the packed words (one shift or mask each) rather
// than keeping 8 floats per chunk alive across phases, which would not fit.
template <int U>
__device__ __forceinline__ void keep_packed(uint4 (&v)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) asm volatile("" : "+v"(v[u].x), "+v"(v[u].y), "+v"(v[u].z), "+v"(v[u].w));
}

__device__ __forceinline__ float ln_out(float x, float mu, float rstd, float g, float b) {
  return ((x - mu) * rstd) * g + b;
}

// Partial sums each thread keeps for one row: with two waves per row a thread
// plays two of the 256 virtual lanes below, otherwise one.
template <int WPR>
constexpr int kParts = WPR == 2 ? 2 : 1;

// Row sum. One wave per row: the wave's butterfly. Two or four waves per row:
// one order for both, so the result does not depend on which of those launch
// shapes a width gets. The row's 16-byte chunks are dealt to 256 virtual
// lanes (chunk c to lane c % 256); each lane adds its chunks in order (the
// caller's partials); each virtual wave of 64 lanes reduces by the butterfly;
// the four wave sums are added as (w0 + w1) + (w2 + w3). Thread t of a row with
// T = 64 WPR threads holds virtual lanes t + T p, p < kParts. Every thread of
// the workgroup must call it the same number of times.
template <int WPR>
__device__ __forceinline__ float row_sum(float (&part)[kParts<WPR>], float* red) {
  if constexpr (WPR == 1) {
    return wave_sum(part[0]);
  } else {
    const int wave = threadIdx.x >> 6;
    const int rg = wave / WPR, wr = wave % WPR;   // row group of the workgroup, wave within the row
#pragma unroll
    for (int p = 0; p < kParts<WPR>; ++p) {
      const float w = wave_sum(part[p]);
      if ((threadIdx.x & 63) == 0) red[rg * 4 + wr + WPR * p] = w;   // virtual wave (t + T p) / 64
    }
    __syncthreads();
    const float t = (red[rg * 4] + red[rg * 4 + 1]) + (red[rg * 4 + 2] + red[rg * 4 + 3]);
    __syncthreads();   // red is reused by the next sum
    return t;
  }
}

// Register path. WPR waves share a row (rows per workgroup = 4 / WPR); thread
// t of a row holds the row's 16-byte chunks t, t + T, t + 2T, ... (T = 64 WPR
// threads, at most U of them), so the row is read from HBM once. PF: the next
// row group's chunks are loaded while this one is normalised (twice the bytes
// in flight per thread, for 4U more registers).
template <int U, int WPR, int YF, bool PF>
__global__ __launch_bounds__(kLnBlock) void ln_rows_bf16(
    const uint16_t* __restrict__ x, int64_t rows, int cols, int64_t ld_x, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, uint16_t* __restrict__ y, int64_t ld_y,
    const float* __restrict__ scale, uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ amax,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
  constexpr int kRowsPerBlock = kLnBlock / 64 / WPR;
  constexpr int T = 64 * WPR;
  constexpr int P = kParts<WPR>;
  static_assert(WPR == 1 || T * P == 256, "two or four waves per row deal chunks to 256 virtual lanes");
  __shared__ float red[kLnBlock / 64 * 2];
  const int t = threadIdx.x % T, rg = threadIdx.x / T;
  const int nch = cols >> 3;
  uint32_t am = 0;   // packed BF16 magnitudes of this thread's outputs
  // Grid-stride over groups of rows. The loop bounds are the same for the
  // whole workgroup (row_sum's barriers need it); a row past the end only
  // takes part in the sums. A bounded grid keeps the amax to one atomic per
  // workgroup.
  uint4 vn[PF ? U : 1];   // PF: the next row group's chunks, in flight
  if constexpr (PF) {
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + rg;
    const bool live = row < rows;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (live ? row : 0) * ld_x);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = t + T * u;
      vn[u] = (live && c < nch) ? xr[c] : uint4{0u, 0u, 0u, 0u};
    }
  }
  for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock; r0 < rows; r0 += (int64_t)gridDim.x * kRowsPerBlock) {
    const int64_t row = r0 + rg;
    const bool live = row < rows;
    uint4 v[U];
    if constexpr (PF) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = vn[u];
      const int64_t nrow = row + (int64_t)gridDim.x * kRowsPerBlock;
      const bool nlive = nrow < rows;
      const uint4* xn = reinterpret_cast<const uint4*>(x + (nlive ? nrow : 0) * ld_x);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = t + T * u;
        vn[u] = (nlive && c < nch) ? xn[c] : uint4{0u, 0u, 0u, 0u};
      }
    } else {
      const uint4* xr = reinterpret_cast<const uint4*>(x + (live ? row : 0) * ld_x);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = t + T * u;
        v[u] = (live && c < nch) ? xr[c] : uint4{0u, 0u, 0u, 0u};
      }
    }
    // chunk u of this thread is chunk t + T u of the row, virtual lane t + T (u % P)
    float s[P];
#pragma unroll
    for (int p = 0; p < P; ++p) s[p] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + T * u < nch) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[u % P] += bf16_lo(w[e]);
          s[u % P] += bf16_hi(w[e]);
        }
      }
    }
    const float n = (float)cols;
    const float mu = row_sum<WPR>(s, red) / n;
    keep_packed<U>(v);
    float ss[P];
#pragma unroll
    for (int p = 0; p < P; ++p) ss[p] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + T * u < nch) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d0 = bf16_lo(w[e]) - mu, d1 = bf16_hi(w[e]) - mu;
          ss[u % P] += d0 * d0;
          ss[u % P] += d1 * d1;
        }
      }
    }
    const float var = row_sum<WPR>(ss, red) / n;
    const float rstd = 1.0f / sqrtf(var + eps);
    keep_packed<U>(v);
    if (!live) continue;

    // The outputs replace the source chunks in registers.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = t + T * u;
      if (c < nch) {
        const float4 g0 = reinterpret_cast<const float4*>(gamma)[2 * c];
        const float4 g1 = reinterpret_cast<const float4*>(gamma)[2 * c + 1];
        float4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
        if (beta != nullptr) {
          b0 = reinterpret_cast<const float4*>(beta)[2 * c];
          b1 = reinterpret_cast<const float4*>(beta)[2 * c + 1];
        }
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16(ln_out(bf16_lo(w[e]), mu, rstd, gv[2 * e], bv[2 * e]),
                           ln_out(bf16_hi(w[e]), mu, rstd, gv[2 * e + 1], bv[2 * e + 1]));
        v[u] = uint4{o[0], o[1], o[2], o[3]};
      }
    }
    if (y != nullptr) {
      uint4* yr = reinterpret_cast<uint4*>(y + row * ld_y);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t + T * u < nch) yr[t + T * u] = v[u];
    }
    if constexpr (YF != kNoQ) {
      uint32_t m = 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t + T * u < nch)
          m = amax_bf16x2(amax_bf16x2(amax_bf16x2(amax_bf16x2(m, v[u].x), v[u].y), v[u].z), v[u].w);
      am = amax_bf16x2(am, m);
      if (q != nullptr) {
        const float sc = *scale;
        const uint32_t sb = __float_as_uint(sc) & 0x7FFFFFFFu;
        // No NaN product can occur without a NaN output or a zero or infinite
        // scale; the choice is made for the whole wave so only one loop runs.
        const bool no_nan = (m & 0xFFFFu) <= 0x7F80u && (m >> 16) <= 0x7F80u && sb != 0u && sb < 0x7F800000u;
        uint2* qr = reinterpret_cast<uint2*>(q + row * ld_q);
        if (__all(no_nan)) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (t + T * u < nch)
              qr[t + T * u] = uint2{enc4_bf16_nonan<YF>(v[u].x, v[u].y, sc), enc4_bf16_nonan<YF>(v[u].z, v[u].w, sc)};
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (t + T * u < nch)
              qr[t + T * u] = uint2{enc4_bf16_sel<YF>(v[u].x, v[u].y, sc), enc4_bf16_sel<YF>(v[u].z, v[u].w, sc)};
        }
      }
    }
    if (t == 0) {
      if (mean_out != nullptr) mean_out[row] = mu;
      if (rstd_out != nullptr) rstd_out[row] = rstd;
    }
  }
  if constexpr (YF != kNoQ) {
    if (amax != nullptr) block_amax_commit<kLnBlock>(bf16x2_acc_to_f32_bits(am), amax);
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < kLnBlock / 64; ++w) t += red[w];
  __syncthreads();   // red is reused by the next sum
  return t;
}

template <int DT>
__device__ __forceinline__ float load_src(const void* x, int64_t i) {
  if constexpr (DT == FP8MP_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[i] << 16);
  return static_cast<const float*>(x)[i];
}

// Generic path: one workgroup per row (grid-stride), three strided passes.
template <int YF, int DT>
__global__ __launch_bounds__(kLnBlock) void ln_rows_generic(
    const void* __restrict__ x, int64_t rows, int cols, int64_t ld_x, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, uint16_t* __restrict__ y, int64_t ld_y,
    const float* __restrict__ scale, uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ amax,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
  __shared__ float red[kLnBlock / 64];
  const float n = (float)cols;
  const float sc = (YF != kNoQ && q != nullptr) ? *scale : 0.f;
  uint32_t am = 0;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * ld_x;
    float s = 0.f;
    for (int j = threadIdx.x; j < cols; j += kLnBlock) s += load_src<DT>(x, base + j);
    const float mu = block_sum(s, red) / n;
    float ss = 0.f;
    for (int j = threadIdx.x; j < cols; j += kLnBlock) {
      const float d = load_src<DT>(x, base + j) - mu;
      ss += d * d;
    }
    const float var = block_sum(ss, red) / n;
    const float rstd = 1.0f / sqrtf(var + eps);
    for (int j = threadIdx.x; j < cols; j += kLnBlock) {
      const float o = ln_out(load_src<DT>(x, base + j), mu, rstd, gamma[j], beta != nullptr ? beta[j] : 0.f);
      const uint32_t h = pack_bf16(o, 0.f) & 0xFFFFu;
      if (y != nullptr) y[row * ld_y + j] = (uint16_t)h;
      if constexpr (YF != kNoQ) {
        am = amax_bf16x2(am, h);
        if (q != nullptr) q[row * ld_q + j] = enc1<YF>(__uint_as_float(h << 16), sc);
      }
    }
    if (threadIdx.x == 0) {
      if (mean_out != nullptr) mean_out[row] = mu;
      if (rstd_out != nullptr) rstd_out[row] = rstd;
    }
  }
  if constexpr (YF != kNoQ) {
    if (amax != nullptr) block_amax_commit<kLnBlock>(bf16x2_acc_to_f32_bits(am), amax);
  }
}

struct LnArgs {
  const void* x; int64_t rows; int cols; int64_t ld_x;
  const float* gamma; const float* beta; float eps;
  uint16_t* y; int64_t ld_y;
  const float* scale; uint8_t* q; int64_t ld_q; float* amax;
  float* mean; float* rstd;
};

// Workgroups of one register-path kernel that fit on a CU at once (at least
// 1; computed once per instantiation). The grid-stride kernels launch exactly
// that many per CU, so every workgroup is resident from the start and there
// is no second round.
template <int U, int WPR, int YF, bool PF>
int resident_blocks() {
  static const int n = []() {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, ln_rows_bf16<U, WPR, YF, PF>, kLnBlock, 0) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  return n;
}

template <int U, int WPR, int YF, bool PF>
hipError_t launch_reg_pf(const LnArgs& a, int num_cus, hipStream_t stream) {
  constexpr int kRowsPerBlock = kLnBlock / 64 / WPR;
  const int64_t need = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t slots = (int64_t)num_cus * resident_blocks<U, WPR, YF, PF>();
  const int64_t grid = need < slots ? need : slots;
  hipLaunchKernelGGL((ln_rows_bf16<U, WPR, YF, PF>), dim3((unsigned)grid), dim3(kLnBlock), 0, stream,
                     static_cast<const uint16_t*>(a.x), a.rows, a.cols, a.ld_x, a.gamma, a.beta, a.eps, a.y, a.ld_y,
                     a.scale, a.q, a.ld_q, a.amax, a.mean, a.rstd);
  return hipGetLastError();
}

// Row prefetch where it measured faster (6-10%): four waves per row with codes,
// at 6145-8192 columns (four chunks per thread, nearly all used) and, beyond
// 8192, when both y and the codes are written. Elsewhere its registers cost
// more occupancy than the extra bytes in flight win (up to 7% slower at
// 5120-6144 columns).
template <int U, int WPR, int YF>
hipError_t launch_reg(const LnArgs& a, int num_cus, hipStream_t stream) {
  if constexpr (WPR == 4 && YF != kNoQ && (U == 4 || U == 8)) {
    const bool pf = U == 4 ? a.cols > 6144 : (a.y != nullptr && a.q != nullptr);
    if (pf) return launch_reg_pf<U, WPR, YF, true>(a, num_cus, stream);
  }
  return launch_reg_pf<U, WPR, YF, false>(a, num_cus, stream);
}

// Chunks per thread and waves per row, measured per width: rows up to 2048
// columns take one wave. Wider rows take two or four; with codes (more
// registers live, so fewer waves fit) the wider split keeps more rows in
// flight per CU. At most kMaxChunksPerThread chunks per thread.
template <int YF>
hipError_t launch_reg_u(const LnArgs& a, int num_cus, hipStream_t stream) {
  const int nch = a.cols / 8;
  if (nch <= 64 * 1) return launch_reg<1, 1, YF>(a, num_cus, stream);
  if (nch <= 64 * 2) return launch_reg<2, 1, YF>(a, num_cus, stream);
  if (nch <= 64 * 4) return launch_reg<4, 1, YF>(a, num_cus, stream);
  if constexpr (YF == kNoQ) {
    if (nch <= 128 * 4) return launch_reg<4, 2, YF>(a, num_cus, stream);
    if (nch <= 128 * 8) return launch_reg<8, 2, YF>(a, num_cus, stream);
  } else {
    if (nch <= 256 * 2) return launch_reg<2, 4, YF>(a, num_cus, stream);
    if (nch <= 256 * 4) return launch_reg<4, 4, YF>(a, num_cus, stream);
  }
  return launch_reg<kMaxChunksPerThread, 4, YF>(a, num_cus, stream);
}

template <int YF>
hipError_t launch_generic(const LnArgs& a, fp8mp_dtype dt, int num_cus, hipStream_t stream) {
  const int64_t grid = a.rows < (int64_t)num_cus * 8 ? a.rows : (int64_t)num_cus * 8;
  if (dt == FP8MP_BF16)
    hipLaunchKernelGGL((ln_rows_generic<YF, FP8MP_BF16>), dim3((unsigned)grid), dim3(kLnBlock), 0, stream, a.x,
                       a.rows, a.cols, a.ld_x, a.gamma, a.beta, a.eps, a.y, a.ld_y, a.scale, a.q, a.ld_q, a.amax,
                       a.mean, a.rstd);
  else
    hipLaunchKernelGGL((ln_rows_generic<YF, FP8MP_F32>), dim3((unsigned)grid), dim3(kLnBlock), 0, stream, a.x,
                       a.rows, a.cols, a.ld_x, a.gamma, a.beta, a.eps, a.y, a.ld_y, a.scale, a.q, a.ld_q, a.amax,
                       a.mean, a.rstd);
  return hipGetLastError();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

hipError_t launch_layernorm_amax_cast(const void* x, fp8mp_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                      const float* gamma, const float* beta, float eps, uint16_t* y, int64_t ld_y,
                                      fp8mp_format fmt, const float* scale, uint8_t* q, int64_t ld_q, float* amax,
                                      float* mean, float* rstd, int num_cus, hipStream_t stream) {
  const LnArgs a{x, rows, (int)cols, ld_x, gamma, beta, eps, y, ld_y, scale, q, ld_q, amax, mean, rstd};
  const bool reg = x_dtype == FP8MP_BF16 && cols % 8 == 0 && cols <= 4 * 64 * 8 * kMaxChunksPerThread &&
                   aligned(x, 16) && ld_x % 8 == 0 && aligned(gamma, 16) && (beta == nullptr || aligned(beta, 16)) &&
                   (y == nullptr || (aligned(y, 16) && ld_y % 8 == 0)) &&
                   (q == nullptr || (aligned(q, 8) && ld_q % 8 == 0));
  const bool cast = q != nullptr || amax != nullptr;
  if (reg) {
    if (!cast) return launch_reg_u<kNoQ>(a, num_cus, stream);
    return fmt == FP8MP_E4M3 ? launch_reg_u<FP8MP_E4M3>(a, num_cus, stream)
                             : launch_reg_u<FP8MP_E5M2>(a, num_cus, stream);
  }
  if (!cast) return launch_generic<kNoQ>(a, x_dtype, num_cus, stream);
  return fmt == FP8MP_E4M3 ? launch_generic<FP8MP_E4M3>(a, x_dtype, num_cus, stream)
                           : launch_generic<FP8MP_E5M2>(a, x_dtype, num_cus, stream);
}

}  // namespace fp8mp
