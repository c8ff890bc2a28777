// Fused amax + scaled saturating FP8 cast (+ transposed copy) for gfx950.
//
// [TE] §NVIDIA Transformer EngineとFP8混合精度とは: the scaling factor follows each
// tensor's observed value range. Delayed scaling lets the range (amax) of step
// t be recorded in the same pass that casts step t with the scale of step t-1,
// so one read of the source suffices.
//
// The work is HBM-bound: per element it reads the source (2 B BF16, 4 B fp32)
// and writes one code (plus one for the transposed copy). Every kernel streams
// 16-byte vectors, reduces amax in registers as unsigned bit patterns of |x|,
// and commits one atomic per workgroup. Sources are read once and stream past
// the caches (non-temporal loads). The codes are stored normally, so they stay
// in the 256 MB MALL for the GEMM that reads them next: measured on the 7B MLP
// step, the fast-accumulation GEMM after the cast took 177 us instead of 201 us
// with non-temporal code stores (the cast itself 48 us either way; alone and
// cold it is about 5% slower).
#include "common.h"

namespace fp8mp {
namespace {

constexpr int kFlatBlock = 512;
constexpr int kFlatUnroll = 4;   // 16-element chunks per thread per iteration
constexpr int kTileBlock = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // for the non-temporal loads
constexpr int kTileRows = 128;   // 32 row groups of 4
constexpr int kTileCols = 128;   // 8 column groups of 16

// The last numel % 16 elements of a flat cast, one per thread of block 0
// (at most 15; the 16-byte chunks before them go through the vector body).
template <int FMT, int DT, bool HAS_Q>
__device__ __forceinline__ uint32_t flat_tail(const void* __restrict__ x, uint8_t* __restrict__ q, int64_t numel,
                                              float s, uint32_t m) {
  const int64_t e = (numel & ~int64_t(15)) + threadIdx.x;
  if (e < numel) {
    const float v = DT == FP8MP_BF16 ? __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[e] << 16)
                                     : static_cast<const float*>(x)[e];
    m = amax_f32(m, v);
    if constexpr (HAS_Q) q[e] = enc1<FMT>(v, s);
  }
  return m;
}

// ---------------------------------------------------------------------------
// Contiguous BF16 source: each thread converts kFlatUnroll chunks of 16
// elements per iteration (two 16-byte loads -> one 16-byte store per chunk);
// all loads of an iteration are issued before any conversion. The source is
// read non-temporally; the codes are cached for the GEMM that follows. The
// magnitude max of an iteration's sources also tells whether any is NaN: when
// no lane of the wave has one (and s is finite and nonzero), no product can
// be NaN and the codes skip the NaN checks.
template <int FMT, bool HAS_Q>
__device__ __forceinline__ uint32_t flat_bf16_body(const uint4* __restrict__ x, uint4* __restrict__ q,
                                                   int64_t nchunk, float s, int64_t block, int64_t nblocks) {
  uint32_t acc = 0;
  // no product x * s can be NaN when no source is NaN and s is finite and nonzero
  const uint32_t sbits = __float_as_uint(s) & 0x7FFFFFFFu;
  const bool s_ok = sbits != 0u && sbits < 0x7F800000u;
  const int64_t stride = nblocks * kFlatBlock;
  for (int64_t base = block * kFlatBlock + threadIdx.x; base < nchunk; base += kFlatUnroll * stride) {
    u32x4 a[kFlatUnroll], b[kFlatUnroll];
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i < nchunk) {
        if constexpr (HAS_Q) {
          a[u] = __builtin_nontemporal_load(xv + 2 * i);
          b[u] = __builtin_nontemporal_load(xv + 2 * i + 1);
        } else {
          // an amax-only pass is followed by the cast of the same source
          // (just-in-time scaling): ordinary loads leave it in the MALL
          a[u] = xv[2 * i];
          b[u] = xv[2 * i + 1];
        }
      } else {
        a[u] = u32x4{0, 0, 0, 0};
        b[u] = a[u];
      }
    }
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
      m = amax_bf16x2(m, a[u].x); m = amax_bf16x2(m, a[u].y);
      m = amax_bf16x2(m, a[u].z); m = amax_bf16x2(m, a[u].w);
      m = amax_bf16x2(m, b[u].x); m = amax_bf16x2(m, b[u].y);
      m = amax_bf16x2(m, b[u].z); m = amax_bf16x2(m, b[u].w);
    }
    acc = amax_bf16x2(acc, m);
    if constexpr (HAS_Q) {
      if (__all(s_ok && (m & 0xFFFFu) <= 0x7F80u && (m >> 16) <= 0x7F80u)) {
#pragma unroll
        for (int u = 0; u < kFlatUnroll; ++u) {
          const int64_t i = base + u * stride;
          if (i < nchunk) {
            u32x4 o;
            o.x = enc4_bf16_nonan<FMT>(a[u].x, a[u].y, s); o.y = enc4_bf16_nonan<FMT>(a[u].z, a[u].w, s);
            o.z = enc4_bf16_nonan<FMT>(b[u].x, b[u].y, s); o.w = enc4_bf16_nonan<FMT>(b[u].z, b[u].w, s);
            *(reinterpret_cast<u32x4*>(q) + i) = o;
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < kFlatUnroll; ++u) {
          const int64_t i = base + u * stride;
          if (i < nchunk) {
            u32x4 o;
            o.x = enc4_bf16<FMT>(a[u].x, a[u].y, s); o.y = enc4_bf16<FMT>(a[u].z, a[u].w, s);
            o.z = enc4_bf16<FMT>(b[u].x, b[u].y, s); o.w = enc4_bf16<FMT>(b[u].z, b[u].w, s);
            *(reinterpret_cast<u32x4*>(q) + i) = o;
          }
        }
      }
    }
  }
  return bf16x2_acc_to_f32_bits(acc);
}

template <int FMT, bool HAS_Q>
__global__ __launch_bounds__(kFlatBlock) void cast_flat_bf16(const uint4* __restrict__ x,
                                                             uint4* __restrict__ q, int64_t numel,
                                                             const float* __restrict__ scale,
                                                             float* __restrict__ amax) {
  const float s = HAS_Q ? *scale : 1.0f;
  uint32_t m = flat_bf16_body<FMT, HAS_Q>(x, q, numel / 16, s, blockIdx.x, gridDim.x);
  if (blockIdx.x == 0) m = flat_tail<FMT, FP8MP_BF16, HAS_Q>(x, reinterpret_cast<uint8_t*>(q), numel, s, m);
  if (amax) block_amax_commit<kFlatBlock>(m, amax);
}

// Several contiguous BF16 tensors in one launch: blocks [start[t], start[t+1])
// run tensor t's flat cast; the first of them also converts its last
// numel % 16 elements.
template <bool HAS_Q_UNUSED>
__global__ __launch_bounds__(kFlatBlock) void cast_flat_bf16_batched(CastBatch batch) {
  int t = 0;
  while (t + 1 < batch.n && (int)blockIdx.x >= batch.block_start[t + 1]) ++t;
  const int64_t block = (int64_t)blockIdx.x - batch.block_start[t];
  const int64_t nblocks = (int64_t)batch.block_start[t + 1] - batch.block_start[t];
  const bool has_q = batch.q[t] != nullptr;
  const float s = has_q ? *batch.scale[t] : 1.0f;
  const int64_t nchunk = batch.numel[t] / 16;
  const uint4* x = static_cast<const uint4*>(batch.x[t]);
  uint4* q = static_cast<uint4*>(batch.q[t]);
  uint32_t m;
  if (batch.fmt[t] == FP8MP_E4M3)
    m = has_q ? flat_bf16_body<FP8MP_E4M3, true>(x, q, nchunk, s, block, nblocks)
              : flat_bf16_body<FP8MP_E4M3, false>(x, q, nchunk, s, block, nblocks);
  else
    m = has_q ? flat_bf16_body<FP8MP_E5M2, true>(x, q, nchunk, s, block, nblocks)
              : flat_bf16_body<FP8MP_E5M2, false>(x, q, nchunk, s, block, nblocks);
  if (block == 0) {
    uint8_t* qb = static_cast<uint8_t*>(batch.q[t]);
    if (batch.fmt[t] == FP8MP_E4M3)
      m = has_q ? flat_tail<FP8MP_E4M3, FP8MP_BF16, true>(batch.x[t], qb, batch.numel[t], s, m)
                : flat_tail<FP8MP_E4M3, FP8MP_BF16, false>(batch.x[t], qb, batch.numel[t], s, m);
    else
      m = has_q ? flat_tail<FP8MP_E5M2, FP8MP_BF16, true>(batch.x[t], qb, batch.numel[t], s, m)
                : flat_tail<FP8MP_E5M2, FP8MP_BF16, false>(batch.x[t], qb, batch.numel[t], s, m);
  }
  if (batch.amax[t] != nullptr) block_amax_commit<kFlatBlock>(canonical_nan(m), batch.amax[t]);
}

// Contiguous fp32 source, 16 elements (four 16-byte loads) -> one 16-byte store.
template <int FMT, bool HAS_Q>
__global__ __launch_bounds__(kFlatBlock) void cast_flat_f32(const float4* __restrict__ x,
                                                            uint4* __restrict__ q, int64_t numel,
                                                            const float* __restrict__ scale,
                                                            float* __restrict__ amax) {
  const float s = HAS_Q ? *scale : 1.0f;
  const int64_t nchunk = numel / 16;
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kFlatBlock;
  for (int64_t i = (int64_t)blockIdx.x * kFlatBlock + threadIdx.x; i < nchunk; i += stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = x[4 * i + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc = amax_f32(acc, v[u].x); acc = amax_f32(acc, v[u].y);
      acc = amax_f32(acc, v[u].z); acc = amax_f32(acc, v[u].w);
    }
    if constexpr (HAS_Q) {
      uint4 o;
      o.x = enc4<FMT>(v[0].x, v[0].y, v[0].z, v[0].w, s);
      o.y = enc4<FMT>(v[1].x, v[1].y, v[1].z, v[1].w, s);
      o.z = enc4<FMT>(v[2].x, v[2].y, v[2].z, v[2].w, s);
      o.w = enc4<FMT>(v[3].x, v[3].y, v[3].z, v[3].w, s);
      q[i] = o;
    }
  }
  if (blockIdx.x == 0) acc = flat_tail<FMT, FP8MP_F32, HAS_Q>(x, reinterpret_cast<uint8_t*>(q), numel, s, acc);
  if (amax) block_amax_commit<kFlatBlock>(acc, amax);
}

// ---------------------------------------------------------------------------
// BF16 source in 128 x 128 tiles, 256 threads. Thread (rg, cg) = (t / 8, t % 8)
// owns rows 4rg .. 4rg+3 and columns 16cg .. 16cg+15 of the tile: two 16-byte
// loads per row (eight lanes read a 256-byte row), one 16-byte store of q per
// row. For q_t the thread's 4 x 16 codes are transposed in registers into
// sixteen dwords (one column, four rows each) and written to an LDS tile held
// in q_t orientation; after a barrier every thread copies four 16-byte pieces
// of it to q_t (eight lanes per 128-byte q_t row).
//
// LDS tile T: 128 q_t rows (tile columns) x 128 bytes (tile rows). The 16-byte
// chunk k of T row c sits at chunk slot k ^ ((c >> 4) & 7): the eight column
// groups of a wave then write eight different chunks (2-way bank sharing at
// most) and the 16-byte reads are conflict-free.

// 4 x 4 byte transpose: input dword i holds row i (byte j = column j); output
// dword j holds column j (byte i = row i). v_perm_b32 picks any four of the
// eight bytes {hi:lo}.
__device__ __forceinline__ void tr4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                    uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3) {
  const uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);  // r2.b0 r3.b0 r2.b1 r3.b1
  const uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);  // r2.b2 r3.b2 r2.b3 r3.b3
  c0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);                  // r0.b0 r1.b0 r2.b0 r3.b0
  c1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);                  // column 1
  c2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);                  // column 2
  c3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);                  // column 3
}

__device__ __forceinline__ int tslot(int c, int k) { return c * kTileRows + ((k ^ ((c >> 4) & 7)) << 4); }

template <int FMT, bool HAS_Q, bool HAS_QT>
__global__ __launch_bounds__(kTileBlock) void cast_tile_bf16(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    const float* __restrict__ scale, uint8_t* __restrict__ q, int64_t ld_q,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ amax, int64_t tiles_c,
    int64_t ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t T[kTileCols * kTileRows];
  const float s = (HAS_Q || HAS_QT) ? *scale : 1.0f;
  const int tid = threadIdx.x, cg = tid & 7, rg = tid >> 3;
  uint32_t acc = 0;        // packed BF16 magnitudes (vector path)
  uint32_t acc32 = 0;      // fp32 magnitudes (edge path)
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t tr = t / tiles_c, tc = t - tr * tiles_c;
    const int64_t R0 = tr * kTileRows, C0 = tc * kTileCols;
    const bool full = (R0 + kTileRows <= rows) && (C0 + kTileCols <= cols);
    if (full) {
      const int64_t r0 = R0 + rg * 4, c0 = C0 + cg * 16;
      u32x4 v[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (r0 + i) * ld_x + c0);
        v[i][0] = __builtin_nontemporal_load(src);
        v[i][1] = __builtin_nontemporal_load(src + 1);
      }
      uint32_t code[4][4];   // [row][dword]: dword d holds columns 4d .. 4d+3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc = amax_bf16x2(acc, v[i][h].x); acc = amax_bf16x2(acc, v[i][h].y);
          acc = amax_bf16x2(acc, v[i][h].z); acc = amax_bf16x2(acc, v[i][h].w);
          code[i][2 * h] = enc4_bf16<FMT>(v[i][h].x, v[i][h].y, s);
          code[i][2 * h + 1] = enc4_bf16<FMT>(v[i][h].z, v[i][h].w, s);
        }
      }
      if constexpr (HAS_Q) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(q + (r0 + i) * ld_q + c0) = u32x4{code[i][0], code[i][1], code[i][2], code[i][3]};
      }
      if constexpr (HAS_QT) {
        __syncthreads();   // the previous tile's T has been copied out
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t col[4];
          tr4(code[0][d], code[1][d], code[2][d], code[3][d], col[0], col[1], col[2], col[3]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = cg * 16 + d * 4 + e;      // tile column = T row
            *reinterpret_cast<uint32_t*>(T + tslot(c, rg >> 2) + (rg & 3) * 4) = col[e];
          }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int idx = it * kTileBlock + tid;
          const int c = idx >> 3, k = idx & 7;
          const u32x4 piece = *reinterpret_cast<const u32x4*>(T + tslot(c, k));
          *reinterpret_cast<u32x4*>(q_t + (C0 + c) * ld_qt + R0 + k * 16) = piece;
        }
      }
    } else {
      // edge tile: element by element, same thread-to-element map
      for (int i = 0; i < 4; ++i) {
        const int64_t r = R0 + rg * 4 + i;
        if (r >= rows) break;
        for (int j = 0; j < 16; ++j) {
          const int64_t c = C0 + cg * 16 + j;
          if (c >= cols) break;
          const float vv = __uint_as_float((uint32_t)x[r * ld_x + c] << 16);
          acc32 = amax_f32(acc32, vv);
          if constexpr (HAS_Q || HAS_QT) {
            const uint8_t code = enc1<FMT>(vv, s);
            if constexpr (HAS_Q) q[r * ld_q + c] = code;
            if constexpr (HAS_QT) q_t[c * ld_qt + r] = code;
          }
        }
      }
    }
  }
  if (amax) {
    uint32_t m = bf16x2_acc_to_f32_bits(acc);
    m = m > acc32 ? m : acc32;
    block_amax_commit<kTileBlock>(m, amax);
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Argument rules (validated by the C-ABI before this is called): x, q and q_t
// 16-byte aligned. A call is flat when the source and the codes are one
// contiguous run (one row, or ld_x == cols and ld_q == cols) and there is no
// transposed copy: BF16 and fp32 sources then take the flat kernels. Every
// other call has a BF16 source with 16-byte aligned rows (ld_x * 2, ld_q and
// ld_qt multiples of 16) and takes the 2-D tile kernel.
template <int FMT>
hipError_t launch_fmt(const void* x, fp8mp_dtype dt, int64_t rows, int64_t cols, int64_t ld_x,
                      const float* scale, uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                      float* amax, int num_cus, hipStream_t stream) {
  const int64_t numel = rows * cols;
  const bool flat = (rows == 1 || (ld_x == cols && (q == nullptr || ld_q == cols))) && q_t == nullptr;
  if (flat) {
    const int64_t nchunk = numel / 16;
    const int per_block = dt == FP8MP_BF16 ? kFlatBlock * kFlatUnroll : kFlatBlock;
    // at least one block: block 0 also converts the numel % 16 tail
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(nchunk, per_block), (int64_t)num_cus * 2));
    if (dt == FP8MP_BF16) {
      if (q) hipLaunchKernelGGL((cast_flat_bf16<FMT, true>), dim3(grid), dim3(kFlatBlock), 0, stream,
                                (const uint4*)x, (uint4*)q, numel, scale, amax);
      else hipLaunchKernelGGL((cast_flat_bf16<FMT, false>), dim3(grid), dim3(kFlatBlock), 0, stream,
                              (const uint4*)x, (uint4*)nullptr, numel, scale, amax);
    } else {
      if (q) hipLaunchKernelGGL((cast_flat_f32<FMT, true>), dim3(grid), dim3(kFlatBlock), 0, stream,
                                (const float4*)x, (uint4*)q, numel, scale, amax);
      else hipLaunchKernelGGL((cast_flat_f32<FMT, false>), dim3(grid), dim3(kFlatBlock), 0, stream,
                              (const float4*)x, (uint4*)nullptr, numel, scale, amax);
    }
    return hipGetLastError();
  }
  if (dt != FP8MP_BF16) return hipErrorInvalidValue;   // refused by the C-ABI's validation
  const int64_t tiles_r = cdiv(rows, kTileRows), tiles_c = cdiv(cols, kTileCols);
  const int64_t ntiles = tiles_r * tiles_c;
  const int grid = (int)std::min<int64_t>(ntiles, (int64_t)num_cus * 4);   // 4 per CU: measured best of 2-16
  const uint16_t* xb = static_cast<const uint16_t*>(x);
#define FP8MP_TILE(HQ, HQT)                                                                       \
  hipLaunchKernelGGL((cast_tile_bf16<FMT, HQ, HQT>), dim3(grid), dim3(kTileBlock), 0, stream, xb, \
                     rows, cols, ld_x, scale, q, ld_q, q_t, ld_qt, amax, tiles_c, ntiles)
  if (q && q_t) FP8MP_TILE(true, true);
  else if (q) FP8MP_TILE(true, false);
  else if (q_t) FP8MP_TILE(false, true);
  else FP8MP_TILE(false, false);
#undef FP8MP_TILE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_amax_cast_batched(CastBatch& batch, int num_cus, hipStream_t stream) {
  // Share num_cus * 8 workgroups among the tensors by size, at least one each
  // (measured: fewer, larger shares leave the tail of the launch under-filled).
  int64_t total = 0;
  for (int t = 0; t < batch.n; ++t) total += batch.numel[t] / 16 + 1;
  const int64_t budget = (int64_t)num_cus * 8;
  int start = 0;
  for (int t = 0; t < batch.n; ++t) {
    batch.block_start[t] = start;
    const int64_t need = cdiv(batch.numel[t] / 16 + 1, (int64_t)kFlatBlock * kFlatUnroll);
    int64_t share = (budget * (batch.numel[t] / 16 + 1) + total - 1) / total;
    share = std::max<int64_t>(1, std::min<int64_t>(share, need));
    start += (int)share;
  }
  batch.block_start[batch.n] = start;
  hipLaunchKernelGGL((cast_flat_bf16_batched<true>), dim3(start), dim3(kFlatBlock), 0, stream, batch);
  return hipGetLastError();
}

hipError_t launch_amax_cast(const void* x, fp8mp_dtype dt, int64_t rows, int64_t cols, int64_t ld_x,
                            fp8mp_format fmt, const float* scale, uint8_t* q, int64_t ld_q,
                            uint8_t* q_t, int64_t ld_qt, float* amax, int num_cus,
                            hipStream_t stream) {
  if (fmt == FP8MP_E4M3)
    return launch_fmt<FP8MP_E4M3>(x, dt, rows, cols, ld_x, scale, q, ld_q, q_t, ld_qt, amax, num_cus,
                                  stream);
  return launch_fmt<FP8MP_E5M2>(x, dt, rows, cols, ld_x, scale, q, ld_q, q_t, ld_qt, amax, num_cus,
                                stream);
}

}  // namespace fp8mp
