// Scaled FP8 GEMM on gfx950 MFMA: C = (A . B^T) * sa_inv * sb_inv, FP32
// accumulation, BF16 output.
//
// [MPT] §横断的知見 "FP8 への拡張": only the GEMMs run in FP8; §"HPC ソルバーとの目的の分岐":
// the matrix units accumulate in FP32.
//
// Both operands are K-contiguous (A[m][k], B[n][k]) and stay FP8 in HBM and
// LDS (one byte per element). Each lane widens its FP8 fragments to BF16 in
// registers (v_cvt_scalef32_pk_bf16_{fp8,bf8} with scale 1, exact for every
// code) and runs v_mfma_f32_32x32x16_bf16, whose products are exact and whose
// sums carry about 22 bits relative to sum|a*b| per instruction. gfx950's FP8
// MFMAs reduce each dot product with only about 17 bits relative to its
// largest product (measured: up to 7e-5 of sum|a*b| per instruction for the
// f8f6f4 forms, which run at twice the MAC rate, and up to 3e-4 for the older
// K = 16 fp8 forms, which run at this BF16 instruction's rate). That exceeds
// the tolerance on outputs that cancel, so the FP32-accumulation GEMM does not
// use them. (The 16x16x32 BF16 form draws less power per product: in a
// register-only loop it ran 14-23% faster than 32x32x16. In this kernel its
// lane layout costs more than that: read from LDS in 8-byte pieces, 16 rows
// of one column share eight bank pairs; read in 16-byte pieces, or regrouped
// from the 32 x 32 reads across lanes, the operands of a 128 x 64 wave tile
// no longer fit beside the accumulators at two waves per SIMD.)
//
// Fast accumulation (ACC = kAccFast) is the opt-in alternative: the same
// tiles, copies and epilogues, but the FP8 fragments go unwidened into
// v_mfma_f32_32x32x64_f8f6f4 at twice the MAC rate. Each such instruction
// aligns its 64 products to the largest one and keeps about 16 bits below it
// (measured on gfx950: errors up to 2^-10.9 of the largest product), so the
// result is only guaranteed within 2^-9 of sum|a*b| instead of FP32 accuracy.
//
// Tiling: 256 x 256 output tiles, K in steps of 128 bytes, 512 threads as 2 x 4
// waves of 128 x 64 (two waves per SIMD). When the tile count leaves a last,
// partly filled round on the CUs, the FP32-accumulation GEMM instead runs
// whole rounds of 256 x 256 tiles and re-tiles the remaining columns (or rows)
// into exactly one round of narrower tiles (256 x 192 or 256 x 128 as 4 x 2
// waves, or 192 x 256 or 128 x 256 as 2 x 4 waves): at 4096 x 11008 every CU
// then does 2.75 tiles' work instead of 3 rounds of whole tiles. One
// workgroup per CU walks its tiles (persistent launch) and stores each tile's
// output while the next one computes; the fast GEMM with the fused output
// cast instead launches one workgroup per tile. Tiles of A
// and B are copied global -> LDS directly (buffer_load_dwordx4 ... lds, no
// VGPR staging) into a double buffer, so the next K step streams in while
// this one is multiplied; in the FP32-accumulation loop each step's barrier
// sits at the top of its last chunk, so the first fragments of the next step
// are read while that chunk's MFMAs run. The 16-byte chunk c of tile row r
// sits in LDS at chunk slot c ^ (r & 7) ^ ((r >> 3) & 1): a wave's copy stays
// coalesced and the fragment reads of sixteen consecutive rows hit sixteen
// distinct bank groups. Tiles are numbered so that each XCD (workgroups are
// dealt to the eight XCDs round-robin) owns a contiguous run of tile ids, and
// runs are walked in groups of kGroupM tile rows so concurrently resident
// tiles share A and B panels in that XCD's L2.
//
// The MFMA is fed B as its first operand and A as its second, so it computes
// the tile transposed and each lane ends up holding four consecutive output
// columns of one output row. The epilogue scales by sa_inv * sb_inv, rounds to
// BF16 (v_cvt_pk_bf16_f32, round to nearest even), turns the lanes' pieces
// into row-contiguous 16-byte chunks through LDS (the persistent kernel
// through a private 4 KB slice per wave, the one-tile kernel through the
// whole 256 x 256 BF16 tile staged in the two stages' 128 KB) and writes
// them out with 16-byte stores.
//
// This header holds the kernels and their launch templates; gemm_exact_a4.hip,
// gemm_exact_a5.hip and gemm_fast.hip instantiate them (split so that the
// instantiations compile in parallel) and gemm.hip holds the entry points.
#pragma once
#include "common.h"
#include "gemm_parts.h"

namespace fp8mp {
namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kTileBytes = kBM * kBK;     // one operand's K step in LDS: 32 KB
constexpr int kGroupM = 4;
constexpr int kXcds = 8;
// Accumulation modes: FP32-accurate (BF16 MFMA on exactly widened codes) or
// the FP8 MFMA's own reduced-precision reduction.
constexpr int kAccExact = 0, kAccFast = 1;

constexpr int kThreads = 512;             // 8 waves, two per SIMD
constexpr int kSlabs = kTileBytes / (kThreads * 16);   // 1 KB LDS slabs each wave fills per operand
static_assert(kSlabs % 2 == 0, "slab parity must equal j parity");
constexpr int kCRow = kBN * 2;            // bytes of one staged BF16 output row in LDS (32 chunk slots)
static_assert(kBM * kCRow <= 4 * kTileBytes, "the BF16 output tile must fit in the two stages");

// Tile geometry: a BM x BN output tile computed by 8 waves laid out
// WAVES_M x (8 / WAVES_M), each owning a WM x WN block of 32 x 32 MFMA blocks.
// The LDS stages always hold 256-row operand tiles; a narrower tile uses
// their first BM (A) or BN (B) rows. Both accumulation modes use these
// layouts. (For the fast mode, 4 waves of 128 x 128 with the accumulators in
// AGPRs read a third less LDS per MFMA but measured 12-17% slower at
// 4096 x 11008 x 4096.)
template <int BM_, int BN_, int WAVES_M_>
struct Geom {
  static constexpr int BM = BM_, BN = BN_, WavesM = WAVES_M_, WavesN = (kThreads / 64) / WAVES_M_;
  static constexpr int WM = BM / WavesM, WN = BN / WavesN;
  static constexpr int PM = WM / 32, PN = WN / 32;   // 32 x 32 MFMA blocks per wave
  static constexpr int CPR = BN / 8;                  // 16-byte BF16 chunks per output row
  static constexpr int Passes = BM * CPR / kThreads;  // epilogue write-out passes
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM <= kBM && BN <= kBN, "32 x 32 blocks in 256-row stages");
  static_assert((BM * CPR) % kThreads == 0, "whole write-out passes");
};
using GFull = Geom<256, 256, 2>;     // 2 x 4 waves of 128 x 64
// Narrow tiles of the last round (see the tile plan below).
constexpr int kNarrowNone = 0, kNarrowN192 = 1, kNarrowN128 = 2, kNarrowM192 = 3, kNarrowM128 = 4;
template <int NARROW> struct NarrowGeom { using G = GFull; };
template <> struct NarrowGeom<kNarrowN192> { using G = Geom<256, 192, 4>; };   // 4 x 2 waves of 64 x 96
template <> struct NarrowGeom<kNarrowN128> { using G = Geom<256, 128, 4>; };   // 4 x 2 waves of 64 x 64
template <> struct NarrowGeom<kNarrowM192> { using G = Geom<192, 256, 2>; };   // 2 x 4 waves of 96 x 64
template <> struct NarrowGeom<kNarrowM128> { using G = Geom<128, 256, 2>; };   // 2 x 4 waves of 64 x 64

// Eight FP8 codes (two dwords) -> eight BF16 values, exactly.
template <int FMT>
__device__ __forceinline__ v8bf widen8(uint32_t lo, uint32_t hi) {
  v2bf p0, p1, p2, p3;
  if constexpr (FMT == FP8MP_E4M3) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, 1.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, 1.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, 1.0f, true);
  }
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two floats -> two BF16 (low half = first), round to nearest even, NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{x, y}, v2bf));
}

// Byte offset of logical chunk c of tile row r inside one operand's LDS tile.
// A 16-lane phase of a 16-byte fragment read touches rows r0 .. r0+15 at one
// logical chunk; with 64 four-byte banks, a 256-byte bank window holds two
// rows, so the slot of row r is c ^ (r & 7) ^ ((r >> 3) & 1): the sixteen
// rows then fall into sixteen distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4); }

// Tile id -> (tile row, tile column); a bijection on [0, tm * tn).
__host__ __device__ __forceinline__ void tile_coords(int bid, int tm, int tn, int& bm, int& bn) {
  const int ntiles = tm * tn;
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int t = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int group = kGroupM * tn;
  const int first_m = (t / group) * kGroupM;
  const int gm = min(tm - first_m, kGroupM);
  const int in = t % group;
  bm = first_m + in % gm;
  bn = in / gm;
}

// Per-thread part of one operand's copy: this thread fills, in each of its
// kSlabs 1 KB LDS slabs (slab = kSlabs * wave + j, 64 lanes x 16 B, lane-ordered),
// chunk slot p = 8 * row + (lane & 7) of tile row row = 8 * slab + lane / 8,
// i.e. logical chunk c = (lane & 7) ^ (row & 7) ^ (slab & 1) (the inverse of
// swz). Since 8 * slab is a multiple of 8, row & 7 = (lane >> 3) & 7, and
// slab & 1 = j & 1 (kSlabs is even): c takes one value on even slabs, c ^ 1
// on odd ones.
struct TileCopy {
  __amdgpu_buffer_rsrc_t rsrc;   // this tile's rows of the operand; loads past their end return 0
  uint32_t off[kSlabs];          // this lane's byte offset in slab j at k = 0
  int here;                      // rows of the tile that exist (wave-uniform)
  // the same offsets in the per-lane form of load_tile_rows
  uint32_t base;                 // byte offset of row 8 * kSlabs * wave + lane / 8 at k = 0
  uint32_t stride8;              // 8 rows
  uint32_t kc0, kc1;             // c * 16 on even and odd slabs
  uint32_t row_ok;               // bit j: slab j's row exists
};
static_assert(kBM == kBN, "one copy geometry serves both operands");

// Leading dimensions are at most kGemmMaxLd bytes, so a tile's rows span less
// than 2^30 bytes: every offset fits the 32-bit buffer offset, and
// kOutOfRange lies above all of them.
static_assert(kBM * kGemmMaxLd <= (int64_t(1) << 30), "tile span must fit 32-bit offsets");
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
// s_waitcnt operand (gfx9 encoding): vmcnt = 0, expcnt and lgkmcnt left at
// their maxima (not waited on).
constexpr int kWaitVmcnt0 = 0x0F70;

// Byte offset within the K step of the 16-byte chunk that a lane copies in
// slab j: row group lane / 8 takes chunk c = (lane % 8) ^ (lane / 8 % 8) on
// even slabs and c ^ 1 on odd ones (the LDS swizzle of the fragment reads).
__device__ __forceinline__ uint32_t slab_kc(int j, int lane) {
  const int c = (lane & 7) ^ ((lane >> 3) & 7);
  return (uint32_t)((j & 1) ? c ^ 1 : c) * 16u;
}

// The buffer resource starts at the tile's first row, so operands of any size
// are addressed with 32-bit offsets.
// cap: the tile's height in rows (256, or a narrow tile's 192 or 128).
__device__ __forceinline__ TileCopy make_copy(const uint8_t* G, int64_t ld, int64_t row0, int64_t rows, int64_t K,
                                              int cap, int wave, int lane) {
  TileCopy t;
  const int64_t here = rows - row0 < cap ? rows - row0 : cap;   // rows of this tile that exist (>= 1)
  const uint32_t bytes = (uint32_t)((here - 1) * ld + K);
  t.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(G + row0 * ld), (short)0, (int)bytes, 0x00020000);
  const int r = wave * 8 * kSlabs + (lane >> 3);
#pragma unroll
  for (int j = 0; j < kSlabs; ++j) t.off[j] = (uint32_t)((r + 8 * j) * ld) + slab_kc(j, lane);
  t.here = (int)here;
  const int c = (lane & 7) ^ ((lane >> 3) & 7);
  t.kc0 = (uint32_t)c * 16u;
  t.kc1 = (uint32_t)(c ^ 1) * 16u;
  t.base = (uint32_t)(r * ld);
  t.stride8 = (uint32_t)(8 * ld);
  t.row_ok = 0;
#pragma unroll
  for (int j = 0; j < kSlabs; ++j) t.row_ok |= (r + 8 * j < here ? 1u : 0u) << j;
  return t;
}

// Copies K step [k0, k0 + 128) of one operand into an LDS tile. A row
// beyond the tile's height lies past the end of the buffer resource (its
// offset is at least here * ld >= (here - 1) * ld + K), so its chunks read
// zeros. With SKIP_EMPTY, a wave whose rows all lie beyond the tile's height
// (a narrow tile's unused waves) issues nothing: those LDS rows are never
// read.
//
// load_tile_inner: a step wholly inside K (k0 + kBK <= K), every wave
// copying. k0 goes in the scalar offset and the LDS slab addresses are
// wave-uniform, so a load takes no vector arithmetic. Whether or not the
// hardware's range check counts the scalar offset, it finds the same rows in
// and out of range here.
__device__ __forceinline__ void load_tile_inner(const TileCopy& t, uint32_t k0, uint8_t* lds, int wave) {
  const int uw = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t uk = __builtin_amdgcn_readfirstlane(k0);
#pragma unroll
  for (int j = 0; j < kSlabs; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        t.rsrc, (__attribute__((address_space(3))) void*)(lds + (uw * kSlabs + j) * 1024), 16, t.off[j], (int)uk, 0,
        0);
}

// load_tile: any step. A chunk past K (which would read the next row's
// bytes) is read at an offset out of range, which stores zeros.
template <bool SKIP_EMPTY = true>
__device__ __forceinline__ void load_tile(const TileCopy& t, uint32_t k0, uint32_t K, uint8_t* lds, int wave) {
  const int uw = __builtin_amdgcn_readfirstlane(wave);
  if (SKIP_EMPTY && uw * 8 * kSlabs >= t.here) return;
  const int lane = (int)(threadIdx.x & 63u);
#pragma unroll
  for (int j = 0; j < kSlabs; ++j) {
    const uint32_t off = k0 + slab_kc(j, lane) < K ? t.off[j] + k0 : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        t.rsrc, (__attribute__((address_space(3))) void*)(lds + (uw * kSlabs + j) * 1024), 16, off, 0, 0, 0);
  }
}

// load_tile_rows: the copy of the FP8-MFMA K loop, as load_tile with the
// offsets, row and K masks formed per lane, and a lane none of whose rows
// exists issuing nothing. That loop measured 3-4% slower with the
// cheaper copies above (load_tile, or load_tile_inner for inner steps).
template <bool SKIP_EMPTY = true>
__device__ __forceinline__ void load_tile_rows(const TileCopy& t, uint32_t k0, uint32_t K, uint8_t* lds, int wave) {
  if (SKIP_EMPTY && t.row_ok == 0) return;
  // all-ones where the chunk exists: a branch-free choice between its offset and out of range
  const uint32_t km0 = 0u - (uint32_t)(k0 + t.kc0 < K), km1 = 0u - (uint32_t)(k0 + t.kc1 < K);
#pragma unroll
  for (int j = 0; j < kSlabs; ++j) {
    const uint32_t m = ((j & 1) ? km1 : km0) & (0u - ((t.row_ok >> j) & 1u));
    const uint32_t off = ((t.base + j * t.stride8 + ((j & 1) ? t.kc1 : t.kc0) + k0) & m) | (kOutOfRange & ~m);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        t.rsrc, (__attribute__((address_space(3))) void*)(lds + (wave * kSlabs + j) * 1024), 16, off, 0, 0, 0);
  }
}

// Accumulators of one wave's 128 x 64 tile: 4 x 2 blocks of 32 x 32, each
// held transposed (see exact_chunk), 128 floats per lane.
template <class G> struct Acc { v16f v[G::PM][G::PN]; };

// Operand format code of the f8f6f4 MFMAs: 0 = E4M3 (fp8), 1 = E5M2 (bf8).
template <int FMT>
constexpr int mfma_fmt() { return FMT == FP8MP_E4M3 ? 0 : 1; }

// One K step on the FP8 MFMA (fast accumulation). Lane group G = lane / 32
// owns chunks 4G .. 4G+3 of its row as in read_frags; sub-step h (0, 1) hands
// chunks 4G+2h and 4G+2h+1 (32 codes) to one 32 x 32 x 64 MFMA. A and B
// fragments are laid out alike, so products pair up; blocks are accumulated
// transposed (B first), giving the same accumulator layout as exact_chunk.
// Both sub-steps' fragments are read up front; the next K step's copies are
// issued after the first sub-step's MFMAs.
template <class GM, int FA, int FB, typename Issue>
__device__ __forceinline__ void mma_step_fast(const uint8_t* As, const uint8_t* Bs, Acc<GM>& acc, int wm, int wn,
                                              int lane, Issue&& issue_copies) {
  constexpr int kPM = GM::PM, kPN = GM::PN;
  const int G = lane >> 5;
  const int ra = wm * GM::WM + (lane & 31), rb = wn * GM::WN + (lane & 31);
  v8i af[2][kPM], bf[2][kPN];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < kPN; ++j) {
      const uint4 lo = *reinterpret_cast<const uint4*>(Bs + swz(rb + j * 32, 4 * G + 2 * h));
      const uint4 hi = *reinterpret_cast<const uint4*>(Bs + swz(rb + j * 32, 4 * G + 2 * h + 1));
      bf[h][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < kPM; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(As + swz(ra + i * 32, 4 * G + 2 * h));
      const uint4 hi = *reinterpret_cast<const uint4*>(As + swz(ra + i * 32, 4 * G + 2 * h + 1));
      af[h][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < kPM; ++i)
#pragma unroll
      for (int j = 0; j < kPN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[h][j], af[h][i], acc.v[i][j],
                                                                      mfma_fmt<FB>(), mfma_fmt<FA>(), 0, 0, 0, 0);
    if (h == 0) issue_copies();
  }
}

// Multiplies the step in `cur` on the FP8 MFMA and, from inside it, issues
// the copy of the next K step into `nxt`. The two stages never overlap;
// saying so (restrict) lets the compiler keep the copy in flight while the
// fragments of `cur` are read.
template <class GM, int FA, int FB>
__device__ __forceinline__ void pipelined_step_fast(const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt,
                                                    bool more, const TileCopy& ca, const TileCopy& cb,
                                                    uint32_t k_next, uint32_t K, Acc<GM>& acc, int wm, int wn,
                                                    int wave, int lane) {
  auto issue = [&]() {
    if (more) {
      load_tile_rows(ca, k_next, K, nxt, wave);
      load_tile_rows(cb, k_next, K, nxt + kTileBytes, wave);
    }
  };
  mma_step_fast<GM, FA, FB>(cur, cur + kTileBytes, acc, wm, wn, lane, issue);
}

// Register state of the FP32-accumulation K loop: the raw fragments of two
// chunks (slot = chunk & 1) and the widened operands of the next sub-step.
template <class GM> struct ExactRegs {
  uint4 aq[2][GM::PM], bq[2][GM::PN];
  v8bf aw[GM::PM], bw[GM::PN];
};

// Reads chunk c (0..3) of this lane's fragments from the stage at st. The K
// step (128 codes of each row) is cut into 8 chunks of 16 codes; lane group
// G = lane / 32 owns chunks 4G .. 4G+3 of its row (rows ra + 32 i of A and
// rb + 32 j of B), so one 16-byte read per fragment per chunk. A and B walk
// k in the same order, so products pair up and the step is covered once.
template <class GM>
__device__ __forceinline__ void read_frags(const uint8_t* st, int ra, int rb, int G, int c, uint4 (&a)[GM::PM],
                                           uint4 (&b)[GM::PN]) {
#pragma unroll
  for (int j = 0; j < GM::PN; ++j) b[j] = *reinterpret_cast<const uint4*>(st + kTileBytes + swz(rb + j * 32, 4 * G + c));
#pragma unroll
  for (int i = 0; i < GM::PM; ++i) a[i] = *reinterpret_cast<const uint4*>(st + swz(ra + i * 32, 4 * G + c));
}

// One chunk's two sub-steps of 32 x 32 x 16 BF16 MFMAs: sub-step h feeds
// bytes 8h .. 8h+7 of each fragment, widened exactly to BF16, as the lane's
// 8 k values. Half 0 widens the second half of chunk c (slot c & 1) and
// half 1 the first half of chunk c + 1 (the other slot), each while the
// MFMAs of the operands widened before run. mid() runs between the two
// halves; with kLast the chunk after c does not exist and is not widened.
//
// Block (i, j) is accumulated as B_j . A_i^T: lane l, register r then holds
// C[32 i + l % 32][32 j + 8 (r / 4) + 4 (l / 32) + r % 4] of the wave's tile.
template <class GM, int FA, int FB, bool kLast, typename Mid>
__device__ __forceinline__ void exact_chunk(ExactRegs<GM>& r, Acc<GM>& acc, int c, Mid&& mid) {
  constexpr int kPM = GM::PM, kPN = GM::PN;
  const int sc = c & 1, sn = sc ^ 1;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const bool widen = half == 0 || !kLast;
    v8bf an[kPM], bn[kPN];
    if (widen) {
#pragma unroll
      for (int i = 0; i < kPM; ++i)
        an[i] = half == 0 ? widen8<FA>(r.aq[sc][i].z, r.aq[sc][i].w) : widen8<FA>(r.aq[sn][i].x, r.aq[sn][i].y);
#pragma unroll
      for (int j = 0; j < kPN; ++j)
        bn[j] = half == 0 ? widen8<FB>(r.bq[sc][j].z, r.bq[sc][j].w) : widen8<FB>(r.bq[sn][j].x, r.bq[sn][j].y);
    }
#pragma unroll
    for (int i = 0; i < kPM; ++i)
#pragma unroll
      for (int j = 0; j < kPN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.bw[j], r.aw[i], acc.v[i][j], 0, 0, 0);
    if (half == 0) {
      // the halves stay apart: otherwise the scheduler hoists the widening of the
      // next chunk, whose fragments are still being read, above these MFMAs
      __builtin_amdgcn_sched_barrier(0);
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (widen) {
#pragma unroll
      for (int i = 0; i < kPM; ++i) r.aw[i] = an[i];
#pragma unroll
      for (int j = 0; j < kPN; ++j) r.bw[j] = bn[j];
    }
  }
}

// Chunks 0..2 of a K step from stage rd, each reading the fragments of the
// chunk after it first.
template <class GM, int FA, int FB>
__device__ __forceinline__ void exact_chunks012(const uint8_t* rd, ExactRegs<GM>& r, Acc<GM>& acc, int ra, int rb,
                                                int G) {
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    read_frags<GM>(rd, ra, rb, G, c + 1, r.aq[(c + 1) & 1], r.bq[(c + 1) & 1]);
    // keep the reads at the top of the chunk (the scheduler would otherwise sink them to their use)
    __builtin_amdgcn_sched_barrier(0);
    exact_chunk<GM, FA, FB, false>(r, acc, c, [] {});
  }
}

// The steady-state body for step k >= 1: the last chunk of step k - 1, whose
// stage `wr` then receives the copy of step k + 1, and the first three
// chunks of step k from stage `rd`. Its barrier (at the top) publishes step
// k, which each thread has waited for, and retires every read of `wr`: the
// last chunk's fragments were read during the chunk before. The first chunk
// of step k is read before the MFMAs of that last chunk are issued, so no
// wave waits on LDS after the barrier with no MFMA work queued.
//
// rd and wr never overlap; saying so (restrict) lets the compiler keep the
// copy into wr in flight while rd is read, here and in the next body (whose
// reads are of this body's wr, after its own wait and barrier). INNER: step
// k + 1 lies wholly inside K, and its copy takes the scalar-offset form.
template <class GM, int FA, int FB, bool INNER>
__device__ __forceinline__ void exact_body(const uint8_t* __restrict__ rd, uint8_t* __restrict__ wr, int k,
                                           const TileCopy& ca, const TileCopy& cb, uint32_t K, ExactRegs<GM>& r,
                                           Acc<GM>& acc, int ra, int rb, int G, int wave) {
  // Step 1 was copied with step 0 and waited for before the loop started;
  // later steps' copies were issued by the body before.
  if (k > 1) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  read_frags<GM>(rd, ra, rb, G, 0, r.aq[0], r.bq[0]);
  __builtin_amdgcn_sched_barrier(0);
  exact_chunk<GM, FA, FB, false>(r, acc, 3, [&] {
    // copy of step k + 1 (none for k + 1 = nk: every chunk would lie past K)
    const uint32_t k0 = (uint32_t)(k + 1) * kBK;
    if constexpr (INNER) {
      load_tile_inner(ca, k0, wr, wave);
      load_tile_inner(cb, k0, wr + kTileBytes, wave);
    } else if (k0 < K) {
      load_tile<false>(ca, k0, K, wr, wave);
      load_tile<false>(cb, k0, K, wr + kTileBytes, wave);
    }
  });
  exact_chunks012<GM, FA, FB>(rd, r, acc, ra, rb, G);
}

// Copies K steps 0 and 1 of a tile into stages s0 and s1 (only step 0 when
// nk = 1). The caller waits for them (vmcnt) and passes a barrier before the
// K loop reads them.
__device__ __forceinline__ void exact_first_copies(uint8_t* s0, uint8_t* s1, int nk, const TileCopy& ca,
                                                   const TileCopy& cb, uint32_t K, int wave) {
  load_tile<false>(ca, 0, K, s0, wave);
  load_tile<false>(cb, 0, K, s0 + kTileBytes, wave);
  if (nk > 1) {
    load_tile<false>(ca, kBK, K, s1, wave);
    load_tile<false>(cb, kBK, K, s1 + kTileBytes, wave);
  }
}

// Whole K loop of the FP32-accumulation GEMM (BF16 MFMA on widened codes),
// software-pipelined across K steps: even steps in stage s0, odd ones in s1.
// Steps 0 and 1 are already in the stages (exact_first_copies, waited for,
// then a barrier). Within a step, the fragments of chunk c + 1 are read
// while chunk c is multiplied, and each sub-step's operands are widened
// while the MFMAs of the sub-step before run; each step's barrier sits at
// the top of its last chunk (exact_body), and the copy of step k + 1 is
// issued during the last chunk of step k - 1, so it has a whole step to
// land. The waits for the copies are written out (buffer-to-LDS loads count
// in vmcnt). On return every copy has landed.
template <class GM, int FA, int FB>
__device__ __forceinline__ void exact_k_steps(uint8_t* s0, uint8_t* s1, int nk, const TileCopy& ca,
                                              const TileCopy& cb, uint32_t K, Acc<GM>& acc, int wm, int wn, int wave,
                                              int lane) {
  constexpr int kPM = GM::PM, kPN = GM::PN;
  const int G = lane >> 5;
  const int ra = wm * GM::WM + (lane & 31), rb = wn * GM::WN + (lane & 31);
  if (nk <= 0) return;
  ExactRegs<GM> r;
  read_frags<GM>(s0, ra, rb, G, 0, r.aq[0], r.bq[0]);
#pragma unroll
  for (int i = 0; i < kPM; ++i) r.aw[i] = widen8<FA>(r.aq[0][i].x, r.aq[0][i].y);
#pragma unroll
  for (int j = 0; j < kPN; ++j) r.bw[j] = widen8<FB>(r.bq[0][j].x, r.bq[0][j].y);
  exact_chunks012<GM, FA, FB>(s0, r, acc, ra, rb, G);
  uint8_t* rd = s1;
  uint8_t* wr = s0;
  // bodies whose copy (of step k + 1) lies wholly inside K, then the rest
  const int n_inner = (int)(K / kBK) - 1 < nk ? (int)(K / kBK) - 1 : nk;
  int k = 1;
  for (; k < n_inner; ++k) {
    exact_body<GM, FA, FB, true>(rd, wr, k, ca, cb, K, r, acc, ra, rb, G, wave);
    uint8_t* t = rd;
    rd = wr;
    wr = t;
  }
  for (; k < nk; ++k) {
    exact_body<GM, FA, FB, false>(rd, wr, k, ca, cb, K, r, acc, ra, rb, G, wave);
    uint8_t* t = rd;
    rd = wr;
    wr = t;
  }
  exact_chunk<GM, FA, FB, true>(r, acc, 3, [] {});
  // no copy of this tile is still in flight (each was waited for at the top of
  // the body that reads it); the wait keeps the tile's end free of them
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}

// The output is (acc * s1) * s2. Normally s1 = sa_inv * sb_inv and s2 = 1
// (one rounding of the scale, and multiplying by 1 is exact). When that
// product overflows or underflows binary32 while acc * sa_inv * sb_inv may
// still be representable, the two factors are applied one at a time: the
// smaller first when the product is too large (both exceed 1), the larger
// first when it is too small.
__device__ __forceinline__ void epilogue_scales(float sa_v, float sb_v, float& s1, float& s2) {
  const float s_ab = sa_v * sb_v;
  s1 = s_ab;
  s2 = 1.0f;
  if (!(__builtin_fabsf(s_ab) >= 1.17549435e-38f && __builtin_fabsf(s_ab) <= 3.40282347e38f) && s_ab == s_ab &&
      sa_v != 0.0f && sb_v != 0.0f) {
    const bool a_big = __builtin_fabsf(sa_v) >= __builtin_fabsf(sb_v);
    const float big = a_big ? sa_v : sb_v, small = a_big ? sb_v : sa_v;
    const bool too_large = __builtin_fabsf(s_ab) > 1.0f;
    s1 = too_large ? small : big;
    s2 = too_large ? big : small;
  }
}

// No FP8 copy of the output (YF of the plain GEMM).
constexpr int kNoY = -1;

// One output tile of geometry GM at (m0, n0), on the FP8 MFMA (fast
// accumulation; the FP32-accumulation GEMM runs in the persistent kernel).
template <class GM, int FA, int FB, int YF, int ACC>
__device__ __forceinline__ void tile_body(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sa, const float* __restrict__ sb,
    uint16_t* __restrict__ C, int64_t ldc, const float* __restrict__ y_scale,
    uint8_t* __restrict__ y_q, int64_t ld_yq, float* __restrict__ y_amax, uint8_t* smem, int64_t m0, int64_t n0) {
  static_assert(ACC == kAccFast, "the one-tile-per-workgroup launch runs the fast-accumulation GEMM only");
  constexpr int kPM = GM::PM, kPN = GM::PN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / GM::WavesN, wn = wave % GM::WavesN;
  const int nk = (int)((K + kBK - 1) / kBK);
  const uint32_t Ku = (uint32_t)K;
  float s1, s2;
  epilogue_scales(*sa, *sb, s1, s2);
  const bool do_c = YF == kNoY || C != nullptr;   // the fused call may skip the BF16 output

  Acc<GM> acc;
  float* accf = reinterpret_cast<float*>(&acc);
#pragma unroll
  for (int e = 0; e < (int)(sizeof(acc) / sizeof(float)); ++e) accf[e] = 0.f;

  const TileCopy ca = make_copy(A, lda, m0, M, K, GM::BM, wave, lane);
  const TileCopy cb = make_copy(B, ldb, n0, N, K, GM::BN, wave, lane);
  if (nk > 0) {
    load_tile(ca, 0, Ku, smem, wave);
    load_tile(cb, 0, Ku, smem + kTileBytes, wave);
  }
  // Step kt reads stage kt & 1 and, meanwhile, fills the other stage with
  // step kt + 1. At the top of a step each thread waits for its own copies
  // into the stage to be read (buffer-to-LDS loads count in vmcnt; the wait
  // is written out because the compiler does not insert it in every
  // instantiation of such a loop), and the barrier then both publishes the
  // stage and retires every read of the stage about to be overwritten.
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = smem + (kt & 1) * 2 * kTileBytes;
    uint8_t* nxt = smem + ((kt + 1) & 1) * 2 * kTileBytes;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    pipelined_step_fast<GM, FA, FB>(cur, nxt, kt + 1 < nk, ca, cb, (uint32_t)(kt + 1) * kBK, Ku, acc, wm, wn, wave,
                                    lane);
  }

  // Epilogue. Every wave must be done reading the last stage before the
  // output tile overwrites it.
  __syncthreads();
  // BF16 tile in LDS: row r (0..BM-1) at r * 512 bytes, its 16-byte chunk c
  // (columns 8c .. 8c+7) at slot c ^ (r & 31). A lane's 8-byte piece (four
  // columns) goes to the half chunk 4 (lane / 32) / 4 = lane / 32.
  {
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < kPM; ++i) {
      const int row = wm * GM::WM + i * 32 + (lane & 31);
      uint8_t* rp = smem + row * kCRow + half * 8;
#pragma unroll
      for (int j = 0; j < kPN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int chunk = (wn * GM::WN + j * 32 + 8 * q) >> 3;
          const v16f& a = acc.v[i][j];
          const uint2 v = {pack_bf16((a[4 * q] * s1) * s2, (a[4 * q + 1] * s1) * s2),
                           pack_bf16((a[4 * q + 2] * s1) * s2, (a[4 * q + 3] * s1) * s2)};
          *reinterpret_cast<uint2*>(rp + ((chunk ^ (row & 31)) << 4)) = v;
        }
    }
  }
  __syncthreads();
  // Write-out: pass p covers chunks p * 512 .. p * 512 + 511 of the tile in
  // row-major order (CPR chunks per row), one 16-byte chunk per thread. With a
  // fused cast, the same eight BF16 values feed the amax and become eight
  // codes of y_q.
  const bool do_q = YF != kNoY && y_q != nullptr, do_amax = YF != kNoY && y_amax != nullptr;
  const float ys = do_q ? *y_scale : 0.f;
  uint32_t am = 0;   // packed BF16 magnitudes of the in-range outputs
  // C and y_q are 16-byte aligned with 16-byte row pitches (checked by the C-ABI).
  const bool full = m0 + GM::BM <= M && n0 + GM::BN <= N;
  if (full) {
    // Interior tile: the chunks of up to 16 passes are read first (the
    // accumulators are dead, so the registers are free), then stored with
    // 16-byte stores and converted without branches.
    constexpr int kPasses = GM::Passes, kBatch = kPasses < 16 ? kPasses : 16;
    static_assert(kPasses % kBatch == 0, "passes split into equal batches");
#pragma unroll
    for (int p0 = 0; p0 < kPasses; p0 += kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int p = 0; p < kBatch; ++p) {
        const int idx = (p0 + p) * kThreads + tid, row = idx / GM::CPR, c = idx % GM::CPR;
        v[p] = *reinterpret_cast<const uint4*>(smem + row * kCRow + ((c ^ (row & 31)) << 4));
      }
      if (do_c) {
#pragma unroll
        for (int p = 0; p < kBatch; ++p) {
          const int idx = (p0 + p) * kThreads + tid, row = idx / GM::CPR, c = idx % GM::CPR;
          *reinterpret_cast<uint4*>(C + (m0 + row) * ldc + n0 + 8 * c) = v[p];
        }
      }
      if constexpr (YF != kNoY) {
        // Magnitude max of this batch's values: the amax contribution, and
        // the test for NaN sources (the two encoders agree on every other value).
        uint32_t mx = 0;
#pragma unroll
        for (int p = 0; p < kBatch; ++p)
          mx = amax_bf16x2(amax_bf16x2(amax_bf16x2(amax_bf16x2(mx, v[p].x), v[p].y), v[p].z), v[p].w);
        if (do_amax) am = amax_bf16x2(am, mx);
        if (do_q) {
          const uint32_t sb = __float_as_uint(ys) & 0x7FFFFFFFu;
          const bool no_nan = (mx & 0xFFFFu) <= 0x7F80u && (mx >> 16) <= 0x7F80u && sb != 0u && sb < 0x7F800000u;
          if (no_nan) {
#pragma unroll
            for (int p = 0; p < kBatch; ++p) {
              const int idx = (p0 + p) * kThreads + tid, row = idx / GM::CPR, c = idx % GM::CPR;
              const uint2 qq = {enc4_bf16_nonan<YF>(v[p].x, v[p].y, ys), enc4_bf16_nonan<YF>(v[p].z, v[p].w, ys)};
              *reinterpret_cast<uint2*>(y_q + (m0 + row) * ld_yq + n0 + 8 * c) = qq;
            }
          } else {
#pragma unroll
            for (int p = 0; p < kBatch; ++p) {
              const int idx = (p0 + p) * kThreads + tid, row = idx / GM::CPR, c = idx % GM::CPR;
              const uint2 qq = {enc4_bf16_sel<YF>(v[p].x, v[p].y, ys), enc4_bf16_sel<YF>(v[p].z, v[p].w, ys)};
              *reinterpret_cast<uint2*>(y_q + (m0 + row) * ld_yq + n0 + 8 * c) = qq;
            }
          }
        }
      }
    }
  } else {
    // Edge tiles: row and column checks, element stores where a chunk
    // straddles N.
    for (int p = 0; p < GM::Passes; ++p) {
      const int idx = p * kThreads + tid, row = idx / GM::CPR, c = idx % GM::CPR;
      const int64_t gm = m0 + row, gn = n0 + 8 * c;
      if (gm >= M) break;
      const uint4 v = *reinterpret_cast<const uint4*>(smem + row * kCRow + ((c ^ (row & 31)) << 4));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint16_t* dst = C + gm * ldc + gn;
      if (gn + 8 <= N) {
        if (do_c) *reinterpret_cast<uint4*>(dst) = v;
        if constexpr (YF != kNoY) {
          if (do_amax) am = amax_bf16x2(amax_bf16x2(amax_bf16x2(amax_bf16x2(am, w[0]), w[1]), w[2]), w[3]);
          if (do_q) {
            const uint32_t q0 = enc4_bf16_sel<YF>(w[0], w[1], ys), q1 = enc4_bf16_sel<YF>(w[2], w[3], ys);
            *reinterpret_cast<uint2*>(y_q + gm * ld_yq + gn) = uint2{q0, q1};
          }
        }
      } else {
        for (int e = 0; e < 8; ++e) {
          if (gn + e >= N) break;
          const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          if (do_c) dst[e] = (uint16_t)h;
          if constexpr (YF != kNoY) {
            if (do_amax) am = amax_bf16x2(am, h);
            if (do_q) y_q[gm * ld_yq + gn + e] = enc1<YF>(__uint_as_float(h << 16), ys);
          }
        }
      }
    }
  }
  if constexpr (YF != kNoY) {
    if (do_amax) block_amax_commit<kThreads>(bf16x2_acc_to_f32_bits(am), y_amax);
  }
}

// The launch's tiles: whole rounds of 256 x 256 tiles over the region
// [0, M) x [0, n_full_end) or [0, m_full_end) x [0, N) (tm x tn of them), then
// tm2 x tn2 narrow tiles of geometry NarrowGeom<NARROW> over the rest, whose
// origin is (m2_off, n2_off). Workgroups below tm * tn take the whole tiles.
struct TilePlan {
  int tm, tn, tm2, tn2;
  int64_t m2_off, n2_off;
};

// One workgroup per tile (the fast GEMM with the fused output cast). YF = a
// format: the epilogue also runs the cast of the BF16 output C on the fly,
// exactly as fp8_amax_cast would on C: *y_amax = max(*y_amax, max|C|) (if
// y_amax) and y_q = enc_YF(C * *y_scale) (if y_q).
template <int FA, int FB, int YF, int ACC, int NARROW>
__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sa, const float* __restrict__ sb,
    uint16_t* __restrict__ C, int64_t ldc, TilePlan plan, const float* __restrict__ y_scale,
    uint8_t* __restrict__ y_q, int64_t ld_yq, float* __restrict__ y_amax) {
  // Two stages, each an A tile followed by a B tile.
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kTileBytes];
  const int n_full = plan.tm * plan.tn;
  int bm, bn;
  if (NARROW == kNarrowNone || (int)blockIdx.x < n_full) {
    tile_coords(blockIdx.x, plan.tm, plan.tn, bm, bn);
    tile_body<GFull, FA, FB, YF, ACC>(A, lda, B, ldb, M, N, K, sa, sb, C, ldc, y_scale, y_q, ld_yq, y_amax, smem,
                                      (int64_t)bm * kBM, (int64_t)bn * kBN);
  } else {
    using G2 = typename NarrowGeom<NARROW>::G;
    tile_coords((int)blockIdx.x - n_full, plan.tm2, plan.tn2, bm, bn);
    tile_body<G2, FA, FB, YF, ACC>(A, lda, B, ldb, M, N, K, sa, sb, C, ldc, y_scale, y_q, ld_yq, y_amax, smem,
                                   plan.m2_off + (int64_t)bm * G2::BM, plan.n2_off + (int64_t)bn * G2::BN);
  }
}

// Persistent form of the GEMM (both accumulation modes, and the exact one
// with the fused output cast). A launch of one workgroup per tile lets every
// tile of a round finish at once, and then every CU waits while the whole
// round's output (32 MB at 4096 x 4096) drains to HBM and while its next
// tile's first K steps arrive. Here each workgroup walks its tiles (ids
// blockIdx.x, blockIdx.x + gridDim.x, ...; gridDim.x is a multiple of 8, so a
// workgroup stays on its XCD's run of tile ids): at the end of a tile it
// turns its BF16 output into row-contiguous chunks in registers through a
// separate 32 KB of LDS, copies the next tile's steps 0 and 1 into the free
// stages and waits for them, and only then issues the output stores, which
// drain while the next tile runs (its first wait for a copy comes at its
// step 2).
constexpr int kBandBytes = 8 * 4096;   // eight waves' 4 KB output slices

// Tile id -> origin and kind (narrow or whole) under the tile plan.
template <int NARROW>
__host__ __device__ __forceinline__ bool plan_tile(int bid, const TilePlan& plan, int64_t& m0, int64_t& n0) {
  using G2 = typename NarrowGeom<NARROW>::G;
  const int n_full = plan.tm * plan.tn;
  int bm, bn;
  if (NARROW == kNarrowNone || bid < n_full) {
    tile_coords(bid, plan.tm, plan.tn, bm, bn);
    m0 = (int64_t)bm * kBM;
    n0 = (int64_t)bn * kBN;
    return false;
  }
  tile_coords(bid - n_full, plan.tm2, plan.tn2, bm, bn);
  m0 = plan.m2_off + (int64_t)bm * G2::BM;
  n0 = plan.n2_off + (int64_t)bn * G2::BN;
  return true;
}

// Column groups of a wave's tile in the persistent epilogue: up to two
// 32-column MFMA blocks (64 columns, 128 bytes of BF16) each.
template <class GM> struct OutGroups {
  static constexpr int G = (GM::PN + 1) / 2;
  static __device__ __forceinline__ constexpr int blocks(int g) { return GM::PN - 2 * g < 2 ? GM::PN - 2 * g : 2; }
};

// End of a persistent tile: each wave turns its own accumulators into
// row-contiguous BF16 chunks in registers, 32 rows x one column group at a
// time, through a private 4 KB slice of the band: lane l writes the four
// consecutive columns it holds of row l % 32, then reads back 16-byte
// chunks, chunk t of the pass being row t / cpr, chunk t % cpr (cpr = 8 or
// 4 chunks a row). Within a wave LDS accesses are ordered, so no workgroup
// barrier is needed, and nothing waits for the copies in flight. Chunk slot
// of (row, c) is c ^ ((row >> 1) & 7) for 8-chunk rows and c ^ ((row >> 2) &
// 3) for 4-chunk rows, which spreads the 8-byte writes of 32 rows over the
// banks. Then, with has_next, the next tile's steps 0 and 1 are copied into
// the stages.
template <class GM>
__device__ __forceinline__ void next_copies_and_wave_out(
    uint8_t* __restrict__ stages, uint8_t* __restrict__ band, bool has_next, const uint8_t* A, int64_t lda,
    const uint8_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K, int64_t nm0, int64_t nn0, int cap_m, int cap_n,
    const Acc<GM>& acc, float s1, float s2, int elane, int ewave, uint4 (&out)[GM::PM][OutGroups<GM>::G][4]) {
  constexpr int kPM = GM::PM, kG = OutGroups<GM>::G;
  static_assert(8 * 32 * 64 * 2 <= kBandBytes, "eight 4 KB wave slices");
  const int nk = (int)((K + kBK - 1) / kBK);
  uint8_t* wbuf = band + ewave * 4096;
  const int half = elane >> 5, wrow = elane & 31;
#pragma unroll
  for (int i = 0; i < kPM; ++i)
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const int nb = OutGroups<GM>::blocks(g), cpr = 4 * nb;
      const int wsw = cpr == 8 ? (wrow >> 1) & 7 : (wrow >> 2) & 3;
#pragma unroll
      for (int jj = 0; jj < nb; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& a = acc.v[i][2 * g + jj];
          const uint2 v = {pack_bf16((a[4 * q] * s1) * s2, (a[4 * q + 1] * s1) * s2),
                           pack_bf16((a[4 * q + 2] * s1) * s2, (a[4 * q + 3] * s1) * s2)};
          *reinterpret_cast<uint2*>(wbuf + wrow * cpr * 16 + (((4 * jj + q) ^ wsw) << 4) + half * 8) = v;
        }
#pragma unroll
      for (int p = 0; p < cpr / 2; ++p) {
        const int t = p * 64 + elane, row = t / cpr, c = t % cpr;
        const int rsw = cpr == 8 ? (row >> 1) & 7 : (row >> 2) & 3;
        out[i][g][p] = *reinterpret_cast<const uint4*>(wbuf + row * cpr * 16 + ((c ^ rsw) << 4));
      }
    }
  // The copies go out after the band reads: the compiler cannot always tell
  // those reads from the copies' LDS writes and would otherwise wait for the
  // copies before them.
  if (has_next) {
    const TileCopy na = make_copy(A, lda, nm0, M, K, cap_m, ewave, elane);
    const TileCopy nb = make_copy(B, ldb, nn0, N, K, cap_n, ewave, elane);
    exact_first_copies(stages, stages + 2 * kTileBytes, nk, na, nb, (uint32_t)K, ewave);
  }
}

// Wave-level amax commit: the same skip-or-atomic rule as block_amax_commit,
// once per wave (the persistent kernel has no LDS left for a block reduction).
__device__ __forceinline__ void wave_amax_commit(uint32_t m, float* amax) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  if ((threadIdx.x & 63) == 0) {
    const uint32_t r = canonical_nan(m);
    unsigned int* a = reinterpret_cast<unsigned int*>(amax);
    if (r != 0u && r > __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(a, r);
  }
}

// K loop of the fast-accumulation GEMM (FP8 MFMA) from published stages:
// steps 0 and 1 are in the two stages (exact_first_copies, waited for, then
// a barrier). Step kt reads stage kt & 1 and, from inside it, copies step
// kt + 1 into the other stage (from step 1 on: step 1 is already there).
template <class GM, int FA, int FB>
__device__ __forceinline__ void fast_k_steps(uint8_t* smem, int nk, const TileCopy& ca, const TileCopy& cb,
                                             uint32_t K, Acc<GM>& acc, int wm, int wn, int wave, int lane) {
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = smem + (kt & 1) * 2 * kTileBytes;
    uint8_t* nxt = smem + ((kt + 1) & 1) * 2 * kTileBytes;
    // Steps 0 and 1 were waited for before the loop; a later step's copy was
    // issued by the step before it. The barrier publishes step kt and retires
    // every read of the stage the next copy overwrites (step 0 is published).
    if (kt > 1) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (kt > 0) __syncthreads();
    pipelined_step_fast<GM, FA, FB>(cur, nxt, kt >= 1 && kt + 1 < nk, ca, cb, (uint32_t)(kt + 1) * kBK, K, acc, wm,
                                    wn, wave, lane);
  }
}

// One tile of geometry GM at (m0, n0) whose steps 0 and 1 are in the stages
// and published. With has_next, the next tile's steps 0 and 1 (origin nm0,
// nn0, heights cap_m x cap_n) are copied in before this tile's output is
// stored; on return they are published. YF = a format: the output is also
// cast as fp8_amax_cast would cast C (codes to y_q under the scale ys when
// y_q is given; the tile's magnitude max committed to *y_amax, one atomic per
// wave at most, when y_amax is given). ACC picks the K loop: BF16 MFMA on
// widened codes, or the FP8 MFMA.
template <class GM, int FA, int FB, int YF, int ACC>
__device__ __forceinline__ void persistent_tile(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                                int64_t M, int64_t N, int64_t K, float s1, float s2, uint16_t* C,
                                                int64_t ldc, uint8_t* y_q, int64_t ld_yq, float ys, float* y_amax,
                                                uint8_t* smem, uint8_t* band, int64_t m0, int64_t n0, bool has_next,
                                                int64_t nm0, int64_t nn0, int cap_m, int cap_n) {
  constexpr int kPM = GM::PM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / GM::WavesN, wn = wave % GM::WavesN;
  const int nk = (int)((K + kBK - 1) / kBK);
  const uint32_t Ku = (uint32_t)K;
  Acc<GM> acc;
  float* accf = reinterpret_cast<float*>(&acc);
#pragma unroll
  for (int e = 0; e < (int)(sizeof(acc) / sizeof(float)); ++e) accf[e] = 0.f;
  {
    const TileCopy ca = make_copy(A, lda, m0, M, K, GM::BM, wave, lane);
    const TileCopy cb = make_copy(B, ldb, n0, N, K, GM::BN, wave, lane);
    if constexpr (ACC == kAccExact)
      exact_k_steps<GM, FA, FB>(smem, smem + 2 * kTileBytes, nk, ca, cb, Ku, acc, wm, wn, wave, lane);
    else
      fast_k_steps<GM, FA, FB>(smem, nk, ca, cb, Ku, acc, wm, wn, wave, lane);
  }
  // every wave is done reading the stages: the next tile's first steps may land there
  __syncthreads();
  // The epilogue's thread indices are taken afresh here (opaque to the
  // compiler), so that their address arithmetic is not hoisted out of the
  // tile loop and kept live through the K loop.
  int etid = (int)threadIdx.x;
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63, ewave = __builtin_amdgcn_readfirstlane(etid) >> 6;
  constexpr int kG = OutGroups<GM>::G;
  uint4 out[kPM][kG][4];
  next_copies_and_wave_out<GM>(smem, band, has_next, A, lda, B, ldb, M, N, K, nm0, nn0, cap_m, cap_n, acc, s1, s2,
                               elane, ewave, out);
  // The next tile's first copies (and any stores still in flight) have
  // landed and are published; nothing else is outstanding while the stores
  // below drain.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  // Chunk p of pass (i, g) of this lane: wave-tile row 32 i + (64 p + lane) / cpr,
  // columns 64 g + 8 ((64 p + lane) % cpr) .. +7. C and y_q are 16-byte
  // aligned with 16-byte row pitches (checked by the C-ABI).
  const int ewm = ewave / GM::WavesN, ewn = ewave % GM::WavesN;
  const int64_t r0 = m0 + ewm * GM::WM, c0 = n0 + ewn * GM::WN;
  const bool do_c = C != nullptr, do_q = YF != kNoY && y_q != nullptr;
  uint32_t am = 0;   // packed BF16 magnitudes of this thread's outputs in the tile
  if (m0 + GM::BM <= M && n0 + GM::BN <= N) {
    // interior tile: 16-byte C stores; with the cast, the magnitude max of
    // this thread's values also tells whether any is NaN (the two encoders
    // agree on every other value)
    uint32_t mx = 0;
    if constexpr (YF != kNoY) {
#pragma unroll
      for (int i = 0; i < kPM; ++i)
#pragma unroll
        for (int g = 0; g < kG; ++g)
#pragma unroll
          for (int p = 0; p < 2 * OutGroups<GM>::blocks(g); ++p) {
            const uint4 v = out[i][g][p];
            mx = amax_bf16x2(amax_bf16x2(amax_bf16x2(amax_bf16x2(mx, v.x), v.y), v.z), v.w);
          }
      am = amax_bf16x2(am, mx);
    }
    const uint32_t sb = __float_as_uint(ys) & 0x7FFFFFFFu;
    const bool no_nan = (mx & 0xFFFFu) <= 0x7F80u && (mx >> 16) <= 0x7F80u && sb != 0u && sb < 0x7F800000u;
#pragma unroll
    for (int i = 0; i < kPM; ++i)
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const int cpr = 4 * OutGroups<GM>::blocks(g);
#pragma unroll
        for (int p = 0; p < cpr / 2; ++p) {
          const int t = p * 64 + elane, row = 32 * i + t / cpr, col = 64 * g + 8 * (t % cpr);
          const uint4 v = out[i][g][p];
          if (do_c) *reinterpret_cast<uint4*>(C + (r0 + row) * ldc + c0 + col) = v;
          if constexpr (YF != kNoY) {
            if (do_q) {
              const uint2 qq = no_nan ? uint2{enc4_bf16_nonan<YF>(v.x, v.y, ys), enc4_bf16_nonan<YF>(v.z, v.w, ys)}
                                      : uint2{enc4_bf16_sel<YF>(v.x, v.y, ys), enc4_bf16_sel<YF>(v.z, v.w, ys)};
              *reinterpret_cast<uint2*>(y_q + (r0 + row) * ld_yq + c0 + col) = qq;
            }
          }
        }
      }
  } else {
    // edge tile: row and column checks, element stores where a chunk straddles N
#pragma unroll
    for (int i = 0; i < kPM; ++i)
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const int cpr = 4 * OutGroups<GM>::blocks(g);
#pragma unroll
        for (int p = 0; p < cpr / 2; ++p) {
          const int t = p * 64 + elane;
          const int64_t gm = r0 + 32 * i + t / cpr, gn = c0 + 64 * g + 8 * (t % cpr);
          if (gm >= M || gn >= N) continue;
          const uint4 v = out[i][g][p];
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
          if (gn + 8 <= N) {
            if (do_c) *reinterpret_cast<uint4*>(C + gm * ldc + gn) = v;
            if constexpr (YF != kNoY) {
              am = amax_bf16x2(amax_bf16x2(amax_bf16x2(amax_bf16x2(am, w[0]), w[1]), w[2]), w[3]);
              if (do_q)
                *reinterpret_cast<uint2*>(y_q + gm * ld_yq + gn) =
                    uint2{enc4_bf16_sel<YF>(w[0], w[1], ys), enc4_bf16_sel<YF>(w[2], w[3], ys)};
            }
          } else {
            for (int e = 0; e < 8 && gn + e < N; ++e) {
              const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
              if (do_c) C[gm * ldc + gn + e] = (uint16_t)h;
              if constexpr (YF != kNoY) {
                am = amax_bf16x2(am, h);
                if (do_q) y_q[gm * ld_yq + gn + e] = enc1<YF>(__uint_as_float(h << 16), ys);
              }
            }
          }
        }
      }
  }
  if constexpr (YF != kNoY) {
    if (y_amax != nullptr) wave_amax_commit(bf16x2_acc_to_f32_bits(am), y_amax);
  }
}

// YF = kNoY: the plain GEMM. YF = a format: the epilogue also runs the cast
// of the BF16 output C on the fly, exactly as fp8_amax_cast would on C:
// *y_amax = max(*y_amax, max|C|) (if y_amax) and y_q = enc_YF(C * *y_scale)
// (if y_q); C may then be null.
template <int FA, int FB, int YF, int ACC, int NARROW>
__global__ __launch_bounds__(kThreads) void gemm_persistent_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M, int64_t N,
    int64_t K, const float* __restrict__ sa, const float* __restrict__ sb, uint16_t* __restrict__ C, int64_t ldc,
    TilePlan plan, const float* __restrict__ y_scale, uint8_t* __restrict__ y_q, int64_t ld_yq,
    float* __restrict__ y_amax) {
  // Two stages, each an A tile followed by a B tile, and the output band.
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t band[kBandBytes];
  using G2 = typename NarrowGeom<NARROW>::G;
  const int total = plan.tm * plan.tn + plan.tm2 * plan.tn2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nk = (int)((K + kBK - 1) / kBK);
  float s1, s2;
  epilogue_scales(*sa, *sb, s1, s2);
  const float ys = YF != kNoY && y_q != nullptr ? *y_scale : 0.f;
  int bid = blockIdx.x;
  int64_t m0, n0;
  bool narrow = plan_tile<NARROW>(bid, plan, m0, n0);
  if (nk > 0) {
    const TileCopy ca = make_copy(A, lda, m0, M, K, narrow ? G2::BM : kBM, wave, lane);
    const TileCopy cb = make_copy(B, ldb, n0, N, K, narrow ? G2::BN : kBN, wave, lane);
    exact_first_copies(smem, smem + 2 * kTileBytes, nk, ca, cb, (uint32_t)K, wave);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }
  for (;;) {
    const int next = bid + (int)gridDim.x;
    const bool has_next = next < total;
    int64_t nm0 = 0, nn0 = 0;
    const bool next_narrow = has_next && plan_tile<NARROW>(next, plan, nm0, nn0);
    const int cap_m = next_narrow ? G2::BM : kBM, cap_n = next_narrow ? G2::BN : kBN;
    if (NARROW != kNarrowNone && narrow)
      persistent_tile<G2, FA, FB, YF, ACC>(A, lda, B, ldb, M, N, K, s1, s2, C, ldc, y_q, ld_yq, ys, y_amax, smem, band,
                                           m0, n0, has_next, nm0, nn0, cap_m, cap_n);
    else
      persistent_tile<GFull, FA, FB, YF, ACC>(A, lda, B, ldb, M, N, K, s1, s2, C, ldc, y_q, ld_yq, ys, y_amax, smem,
                                              band, m0, n0, has_next, nm0, nn0, cap_m, cap_n);
    if (!has_next) break;
    bid = next;
    m0 = nm0;
    n0 = nn0;
    narrow = next_narrow;
  }
}


// The tile plan of an m x n output on num_cus CUs. With T = tm * tn whole
// tiles and R = T / num_cus whole rounds, a launch of whole tiles only takes
// R + 1 rounds when T is not a multiple of num_cus. If num_cus is a multiple
// of tm, the first R * num_cus / tm tile columns are kept as whole tiles and
// the remaining columns are cut into narrow tiles num_cus / tm to a tile row,
// each at most 192 wide (geometry 256 x 192, or 256 x 128 when 128 suffices):
// R + 0.75 (or R + 0.5) rounds of work. The same holds for rows when num_cus
// is a multiple of tn. The split with the narrower tiles wins; otherwise
// (or with no partial round) the plan is whole tiles only.
int plan_tiles(int64_t m, int64_t n, int num_cus, TilePlan& p) {
  const int tm = (int)((m + kBM - 1) / kBM), tn = (int)((n + kBN - 1) / kBN);
  p = TilePlan{tm, tn, 0, 0, 0, 0};
  const int64_t tiles = (int64_t)tm * tn;
  if (num_cus <= 0 || tiles <= num_cus || tiles % num_cus == 0) return kNarrowNone;
  const int64_t rounds = tiles / num_cus;
  int best = kNarrowNone, best_w = kBN;
  // along N: rest columns, num_cus / tm narrow tiles per tile row
  if (num_cus % tm == 0) {
    const int64_t per = num_cus / tm, keep = rounds * per, rest = n - keep * kBN;
    const int64_t w = (rest + per - 1) / per;
    if (rest > 0 && w <= 192) {
      const int bw = w <= 128 ? 128 : 192;
      best = bw == 128 ? kNarrowN128 : kNarrowN192;
      best_w = bw;
      p = TilePlan{tm, (int)keep, tm, (int)((rest + bw - 1) / bw), 0, keep * kBN};
    }
  }
  // along M: rest rows, num_cus / tn narrow tiles per tile column
  if (num_cus % tn == 0) {
    const int64_t per = num_cus / tn, keep = rounds * per, rest = m - keep * kBM;
    const int64_t h = (rest + per - 1) / per;
    if (rest > 0 && h <= 192) {
      const int bh = h <= 128 ? 128 : 192;
      if (bh < best_w) {
        best = bh == 128 ? kNarrowM128 : kNarrowM192;
        p = TilePlan{(int)keep, tn, (int)((rest + bh - 1) / bh), tn, keep * kBM, 0};
      }
    }
  }
  return best;
}

template <int FA, int FB, int YF, int ACC, int NARROW>
hipError_t launch_plan(const GemmArgs& g, const TilePlan& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(p.tm * p.tn + p.tm2 * p.tn2);
  hipLaunchKernelGGL((gemm_fp8_kernel<FA, FB, YF, ACC, NARROW>), dim3(grid), dim3(kThreads), 0, stream, g.a, g.lda,
                     g.b, g.ldb, g.m, g.n, g.k, g.sa, g.sb, g.c, g.ldc, p, g.y_scale, g.y_q, g.ld_yq, g.y_amax);
  return hipGetLastError();
}

// Launch choice. The FP32-accumulation GEMM, plain or with the fused output
// cast, takes the tile plan and runs persistent. The plain fast-accumulation
// GEMM runs persistent on whole tiles; its fused-cast form keeps one
// workgroup per tile (in the persistent kernel its K loop spills registers).
// Measured on one MI355X:
// - the tile plan is 1-3% faster for the exact GEMM at 4096 x 11008 x 4096
//   (7B backward, 13B projections) and up to 6% slower for the fast one (the
//   chip runs at its power limit there, and a full last round lowers the
//   clock);
// - the persistent walk gains 1.5-7.5% for the exact GEMM where K is small
//   next to the output (16384 x 16384 x 512 .. 8192 x 8192 x 2048) and is
//   even at K = 4096 and 8192, where the chip sits at its power limit either
//   way; with the fused output cast, whose code stores also drain under the
//   next tile, the 7B GEMM took 265 instead of 272 us;
// - for the fast GEMM it gains 2-3% at 4096 x 11008 x 4096 and at the 70B
//   slice and 4-13% at the small-K shapes.
// Workgroups of a persistent launch over `total` tiles: one per CU, a
// multiple of 8 so that each keeps to its XCD's tile ids (all tiles when
// fewer, or when the device reports fewer than 8 CUs).
inline int persistent_grid(int total, int num_cus) {
  const int slots = num_cus >= 8 ? num_cus / 8 * 8 : total;
  return total < slots ? total : slots;
}

template <int FA, int FB, int YF, int ACC, int NARROW>
hipError_t launch_persistent(const GemmArgs& g, const TilePlan& p, int num_cus, hipStream_t stream) {
  const unsigned grid = (unsigned)persistent_grid(p.tm * p.tn + p.tm2 * p.tn2, num_cus);
  hipLaunchKernelGGL((gemm_persistent_kernel<FA, FB, YF, ACC, NARROW>), dim3(grid), dim3(kThreads), 0, stream,
                     g.a, g.lda, g.b, g.ldb, g.m, g.n, g.k, g.sa, g.sb, g.c, g.ldc, p, g.y_scale, g.y_q, g.ld_yq,
                     g.y_amax);
  return hipGetLastError();
}

template <int FA, int FB, int YF, int ACC>
hipError_t launch_one(const GemmArgs& g, int num_cus, hipStream_t stream) {
  TilePlan p;
  const int kind = plan_tiles(g.m, g.n, ACC == kAccExact ? num_cus : 0, p);
  if constexpr (ACC == kAccExact) {
    switch (kind) {
      case kNarrowN192: return launch_persistent<FA, FB, YF, ACC, kNarrowN192>(g, p, num_cus, stream);
      case kNarrowN128: return launch_persistent<FA, FB, YF, ACC, kNarrowN128>(g, p, num_cus, stream);
      case kNarrowM192: return launch_persistent<FA, FB, YF, ACC, kNarrowM192>(g, p, num_cus, stream);
      case kNarrowM128: return launch_persistent<FA, FB, YF, ACC, kNarrowM128>(g, p, num_cus, stream);
      default: return launch_persistent<FA, FB, YF, ACC, kNarrowNone>(g, p, num_cus, stream);
    }
  } else if constexpr (YF == kNoY) {
    return launch_persistent<FA, FB, YF, ACC, kNarrowNone>(g, p, num_cus, stream);
  } else {
    return launch_plan<FA, FB, YF, ACC, kNarrowNone>(g, p, stream);
  }
}

template <int FA, int FB, int ACC>
hipError_t launch_y(const GemmArgs& g, int y_fmt, int num_cus, hipStream_t stream) {
  if (y_fmt == FP8MP_E4M3) return launch_one<FA, FB, FP8MP_E4M3, ACC>(g, num_cus, stream);
  if (y_fmt == FP8MP_E5M2) return launch_one<FA, FB, FP8MP_E5M2, ACC>(g, num_cus, stream);
  return launch_one<FA, FB, kNoY, ACC>(g, num_cus, stream);
}

template <int ACC>
hipError_t dispatch_acc(const GemmArgs& g, fp8mp_format a_fmt, fp8mp_format b_fmt, int y_fmt, int num_cus,
                        hipStream_t stream) {
  if (a_fmt == FP8MP_E4M3 && b_fmt == FP8MP_E4M3)
    return launch_y<FP8MP_E4M3, FP8MP_E4M3, ACC>(g, y_fmt, num_cus, stream);
  if (a_fmt == FP8MP_E5M2 && b_fmt == FP8MP_E4M3)
    return launch_y<FP8MP_E5M2, FP8MP_E4M3, ACC>(g, y_fmt, num_cus, stream);
  if (a_fmt == FP8MP_E4M3 && b_fmt == FP8MP_E5M2)
    return launch_y<FP8MP_E4M3, FP8MP_E5M2, ACC>(g, y_fmt, num_cus, stream);
  return launch_y<FP8MP_E5M2, FP8MP_E5M2, ACC>(g, y_fmt, num_cus, stream);
}

}  // namespace
}  // namespace fp8mp
