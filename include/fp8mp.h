/*
 * fp8mp: the per-tensor-scaled FP8 linear layer of mixed-precision training,
 * as a C-ABI library for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages):
 *   [TE]  「AI：NVIDIA Transformer EngineとFP8混合精度の実装ガイド｜環境構築からベンチマークまで」
 *   [TRT] 「NVIDIA TensorRTによるFP8量子化：高性能推論エンジンの実現」
 *   [MPT] 「混合精度訓練」 (notes.yuuk.io wiki)
 *
 * The layer's hot path: record each tensor's amax while casting it to FP8 with
 * the scale from the previous step (delayed scaling), update the scale from the
 * amax history, and multiply the FP8 operands with FP32 accumulation into a
 * BF16 output dequantised by the inverse scales.
 *
 * Conventions for every call:
 *   - All data pointers are device pointers owned by the caller. The library
 *     allocates nothing and keeps no state other than a per-device arch check.
 *   - Work is enqueued on `stream` (NULL = the legacy default stream). No call
 *     synchronises the stream or copies data to the host; scales and amaxes
 *     stay on the device.
 *   - Arguments are validated on the host before anything is launched. A bad
 *     argument returns FP8MP_ERR_INVALID_ARG and touches nothing.
 *   - Layouts are row-major with a leading dimension (elements between rows).
 *   - FP8 codes are bytes: OCP E4M3 (bias 7, largest 448, NaN = S.1111.111,
 *     no Inf) or OCP E5M2 (bias 15, largest 57344, IEEE Inf/NaN).
 *   - Calls are thread-safe. Errors of kernels that fault surface at the
 *     caller's next synchronisation, as usual in HIP.
 */
#ifndef FP8MP_H
#define FP8MP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 formats. [TE] §NVIDIA Transformer EngineとFP8混合精度とは: E4M3 has 4 exponent
 * and 3 mantissa bits and suits the forward pass, E5M2 has 5 and 2 and suits
 * the backward pass. [MPT] §定義 precision table: largest values 448 and 57344.
 * FP8MP_FP16 (largest value 65504, same table) names tensor-scaled FP16
 * storage; only fp8_scale_update accepts it (the FP16 master weights of
 * fp8_adam_step), every other entry point rejects it. */
typedef enum { FP8MP_E4M3 = 0, FP8MP_E5M2 = 1, FP8MP_FP16 = 2 } fp8mp_format;

/* Source element types of the cast: fp32, or BF16 passed as 16-bit patterns. */
typedef enum { FP8MP_F32 = 0, FP8MP_BF16 = 1 } fp8mp_dtype;

typedef enum {
  FP8MP_OK = 0,
  FP8MP_ERR_INVALID_ARG = 1,  /* NULL where required, negative size, ld too small, bad enum */
  FP8MP_ERR_UNSUPPORTED = 2,  /* a well-formed request the kernels do not handle (e.g. K % 16 != 0) */
  FP8MP_ERR_NO_DEVICE = 3,    /* no HIP device visible */
  FP8MP_ERR_WRONG_ARCH = 4,   /* current device is not gfx950 */
  FP8MP_ERR_HIP = 5           /* a HIP call or kernel launch failed */
} fp8mp_status;

/*
 * fp8_amax_cast: amax reduction fused with the scaled saturating cast, and
 * optionally the transposed copy of the codes, in one pass over x.
 *
 * [TE] §NVIDIA Transformer EngineとFP8混合精度とは: each tensor's value range is
 * watched and its scaling factor adjusted so values fit FP8's narrow range;
 * [TE] §動的スケーリングとFP8レシピの設定: the recipe keeps an amax history.
 *
 *   x       rows x cols source, element stride ld_x (>= cols), type x_dtype.
 *   scale   one fp32 on the device: the scale in force (the previous step's).
 *   q       rows x cols codes, ld_q (>= cols): q[r][c] = enc(fp32(x[r][c]) * scale).
 *   q_t     cols x rows codes, ld_qt (>= rows): q_t[c][r] = q[r][c].
 *   amax    one fp32 on the device, updated as *amax = max(*amax, max |x|).
 *
 * enc rounds to nearest (ties to even), saturates every |v| >= the format's
 * largest value, +-Inf included, to the largest finite code of that sign, maps
 * NaN to sign|0x7F, keeps FP8 subnormals and the sign of zero. The product
 * fp32(x) * scale is one IEEE binary32 multiply (no flushing of subnormals).
 * amax is exact; any NaN in x makes *amax the canonical NaN 0x7FC00000. *amax
 * must hold +0..+Inf or that NaN on entry (fp8_scale_update leaves history[0]
 * at +0).
 *
 * q, q_t and amax may each be NULL; scale may be NULL only when q and q_t are
 * both NULL (an amax-only pass). rows or cols == 0 is a no-op returning OK.
 *
 * Layout rules (the kernels move 16-byte vectors; there is no scalar path):
 *   - x, q and q_t start on 16-byte boundaries, else FP8MP_ERR_INVALID_ARG.
 *   - A flat call, one contiguous run (rows == 1, or ld_x == cols and
 *     ld_q == cols) with q_t NULL, takes any cols, BF16 or fp32.
 *   - Any other call needs a BF16 source and 16-byte row pitches: ld_x * 2,
 *     ld_q and ld_qt multiples of 16, else FP8MP_ERR_INVALID_ARG. Ragged
 *     rows and cols are fine. An fp32 source that is strided or needs q_t is
 *     FP8MP_ERR_UNSUPPORTED.
 */
fp8mp_status fp8_amax_cast(const void* x, fp8mp_dtype x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, fp8mp_format fmt, const float* scale,
                           uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                           float* amax, hipStream_t stream);

/* One tensor of fp8_amax_cast_batched: a contiguous source of numel elements. */
typedef struct {
  const void* x;          /* numel source values (x_dtype), contiguous */
  fp8mp_dtype x_dtype;
  int64_t numel;
  fp8mp_format fmt;
  const float* scale;     /* required when q is given */
  uint8_t* q;             /* numel codes, or NULL (amax only) */
  float* amax;            /* max-accumulated, or NULL */
} fp8mp_cast_item;

/*
 * fp8_amax_cast_batched: fp8_amax_cast for n_items contiguous tensors, with
 * the same results as n_items separate calls. A layer casts all its operands
 * at the start of a step ([TE] §動的スケーリングとFP8レシピの設定); BF16 sources
 * share one launch per 8 tensors, the workgroups split among them by size;
 * fp32 sources take fp8_amax_cast's flat kernel one by one. items is a host
 * array; each item is validated as fp8_amax_cast validates a rows = 1,
 * cols = numel call (x and q on 16-byte boundaries), all before anything is
 * launched. Items must not overlap one another's outputs.
 */
fp8mp_status fp8_amax_cast_batched(int32_t n_items, const fp8mp_cast_item* items, hipStream_t stream);

/*
 * fp8_scale_update: the delayed-scaling update of one tensor's recipe state.
 *
 * [TE] §動的スケーリングとFP8レシピの設定: DelayedScaling with margin (default 0;
 * larger means fewer overflows, more underflows) and amax_history_len (default
 * 1024; the history the scale is computed from). [MPT] §横断的知見 on tensor
 * scaling: delayed per-tensor scaling uses past amaxes.
 *
 *   amax_history  history_len fp32 values; entry 0 holds this step's amax.
 *   scale, scale_inv  one fp32 each, read and written.
 *
 * a = max over all entries (NaN propagates). If a is finite and > 0:
 *   s' = fp32(fp32(fmax / a) * 2^-margin)   (IEEE division, exact power-of-two step)
 * with fmax = 448 (E4M3), 57344 (E5M2) or 65504 (FP8MP_FP16 storage)
 * and if s' and fp32(1 / s') are finite and > 0 they replace scale and
 * scale_inv; otherwise both are held. Then the history rolls by one entry
 * (entry i takes entry i-1, entry 0 becomes +0). history_len >= 1, margin >= 0.
 * One workgroup; stream-ordered after the casts that wrote entry 0.
 */
fp8mp_status fp8_scale_update(float* amax_history, int32_t history_len, fp8mp_format fmt,
                              int32_t margin, float* scale, float* scale_inv,
                              hipStream_t stream);

/*
 * fp8_scale_update_batched: fp8_scale_update for n_tensors tensors in one
 * launch per 16 tensors (one workgroup per tensor), with the same result as
 * n_tensors separate calls. A layer updates all of its tensors' recipe state
 * after its GEMMs ([TE] §動的スケーリングとFP8レシピの設定); batching saves the
 * launches.
 *
 *   amax_histories, scales, scale_invs   host arrays of n_tensors device pointers.
 *   history_lens, fmts, margins          host arrays of n_tensors values, each
 *                                        checked as fp8_scale_update checks it.
 * The tensors' buffers must not overlap. n_tensors == 0 is a no-op.
 */
fp8mp_status fp8_scale_update_batched(int32_t n_tensors, float* const* amax_histories,
                                      const int32_t* history_lens, const fp8mp_format* fmts,
                                      const int32_t* margins, float* const* scales,
                                      float* const* scale_invs, hipStream_t stream);

/*
 * fp8_scaled_gemm: C = (A . B^T) * a_scale_inv * b_scale_inv with FP32
 * accumulation and a BF16 result (round to nearest even).
 *
 * [MPT] §横断的知見 "FP8 への拡張": only the GEMMs run in FP8; §"HPC ソルバーとの目的の分岐":
 * tensor cores accumulate in FP32. [TE] §NVIDIA Transformer EngineとFP8混合精度とは:
 * FP8 doubles tensor-core throughput over 16-bit types.
 *
 *   a   m x k codes in a_fmt, leading dimension lda (>= k), K contiguous.
 *   b   n x k codes in b_fmt, leading dimension ldb (>= k), K contiguous.
 *   a_scale_inv, b_scale_inv  one fp32 each on the device.
 *   c   m x n BF16 (16-bit patterns), leading dimension ldc (>= n).
 *
 * Format pairs: (E4M3, E4M3) for the forward pass; (E5M2, E4M3) for dgrad and
 * wgrad of the HYBRID recipe ([TE] §動的スケーリングとFP8レシピの設定); (E4M3, E5M2)
 * and (E5M2, E5M2) are also accepted. k must be a multiple of 16 (the
 * kernel's K granule; else FP8MP_ERR_UNSUPPORTED). a, b and c start on
 * 16-byte boundaries, lda and ldb are multiples of 16 and ldc a multiple of
 * 8 (16-byte row pitches), else FP8MP_ERR_INVALID_ARG. lda, ldb at most
 * 4 MiB (else FP8MP_ERR_UNSUPPORTED).
 * m, n arbitrary; m == 0 or n == 0 is a no-op; k == 0 writes zeros (times the
 * inverse scales). NaN codes propagate to NaN outputs. The output is
 * (acc * (sa_inv * sb_inv)) rounded to BF16, or, when that product of the
 * inverse scales overflows or underflows binary32, the two factors applied
 * one after the other.
 */
fp8mp_status fp8_scaled_gemm(const uint8_t* a, fp8mp_format a_fmt, int64_t lda,
                             const uint8_t* b, fp8mp_format b_fmt, int64_t ldb,
                             int64_t m, int64_t n, int64_t k,
                             const float* a_scale_inv, const float* b_scale_inv,
                             uint16_t* c, int64_t ldc, hipStream_t stream);

/*
 * fp8_scaled_gemm_fast_accum: fp8_scaled_gemm with every argument, rule and
 * error the same, run on gfx950's FP8 matrix instruction
 * (v_mfma_f32_32x32x64_f8f6f4) instead of exactly widened BF16 operands.
 *
 * [TE] §NVIDIA Transformer EngineとFP8混合精度とは: FP8 runs the matrix units at
 * twice the 16-bit rate. That instruction does not accumulate in FP32: it
 * aligns its 64 products to the largest and keeps about 16 bits below it
 * (measured on gfx950: errors up to 2^-10.9 of the largest product per
 * instruction). The result is therefore guaranteed only within
 *   |y - y_ref| <= 2^-7 |y_ref| + 2^-9 sum_k |a_k b_k|
 * (a_k, b_k the dequantised operands), not within the FP32-accumulation bound
 * of fp8_scaled_gemm. Rows whose products in each 64-wide K block share one
 * magnitude are summed exactly. Opt-in for callers that accept that error.
 */
fp8mp_status fp8_scaled_gemm_fast_accum(const uint8_t* a, fp8mp_format a_fmt, int64_t lda,
                                        const uint8_t* b, fp8mp_format b_fmt, int64_t ldb,
                                        int64_t m, int64_t n, int64_t k,
                                        const float* a_scale_inv, const float* b_scale_inv,
                                        uint16_t* c, int64_t ldc, hipStream_t stream);

/*
 * fp8_scaled_gemm_amax_cast: fp8_scaled_gemm, and in the same kernel the cast
 * of its BF16 output C for the next layer, with exactly the result of
 * fp8_amax_cast(C, FP8MP_BF16, m, n, ldc, y_fmt, y_scale, y_q, ld_yq, NULL, 0,
 * y_amax) run afterwards on C:
 *   *y_amax = max(*y_amax, max |C|)      (if y_amax; NaN -> 0x7FC00000)
 *   y_q[i][j] = enc_{y_fmt}(C[i][j] * *y_scale)   (if y_q; saturating RNE)
 *
 * [TE] §基本的なFP8トレーニングコードの構成: consecutive te.Linear layers feed one
 * another, so the output of one is the FP8 operand of the next; under the
 * delayed recipe ([TE] §動的スケーリングとFP8レシピの設定) that operand is cast with
 * the next layer's current scale and its amax goes into that layer's
 * history. Fusing the cast saves a read of C.
 *
 *   c        as for fp8_scaled_gemm (all its rules apply), or NULL when y_q or
 *            y_amax is given: the BF16 output is then computed but not stored.
 *   y_fmt    the format of y_q (validated even when y_q is NULL).
 *   y_scale  one fp32 on the device; required when y_q is given.
 *   y_q      m x n codes, leading dimension ld_yq (>= n, a multiple of 16),
 *            starting on a 16-byte boundary, or NULL.
 *   y_amax   one fp32 on the device, max-accumulated, or NULL.
 * With y_q and y_amax both NULL the call equals fp8_scaled_gemm. y_q and
 * y_amax must not overlap c, a or b.
 */
fp8mp_status fp8_scaled_gemm_amax_cast(const uint8_t* a, fp8mp_format a_fmt, int64_t lda,
                                       const uint8_t* b, fp8mp_format b_fmt, int64_t ldb,
                                       int64_t m, int64_t n, int64_t k,
                                       const float* a_scale_inv, const float* b_scale_inv,
                                       uint16_t* c, int64_t ldc,
                                       fp8mp_format y_fmt, const float* y_scale,
                                       uint8_t* y_q, int64_t ld_yq, float* y_amax,
                                       hipStream_t stream);

/*
 * fp8_scaled_gemm_amax_cast_fast_accum: fp8_scaled_gemm_amax_cast on the FP8
 * matrix instruction, with the accumulation and error bound of
 * fp8_scaled_gemm_fast_accum. The epilogue is unchanged: y_q and y_amax are
 * exactly fp8_amax_cast of the BF16 output this call produces.
 */
fp8mp_status fp8_scaled_gemm_amax_cast_fast_accum(const uint8_t* a, fp8mp_format a_fmt, int64_t lda,
                                                  const uint8_t* b, fp8mp_format b_fmt, int64_t ldb,
                                                  int64_t m, int64_t n, int64_t k,
                                                  const float* a_scale_inv, const float* b_scale_inv,
                                                  uint16_t* c, int64_t ldc,
                                                  fp8mp_format y_fmt, const float* y_scale,
                                                  uint8_t* y_q, int64_t ld_yq, float* y_amax,
                                                  hipStream_t stream);

/*
 * fp8_layernorm_amax_cast: LayerNorm over each row of x, its BF16 output, and
 * in the same pass the cast of that output for the following FP8 linear layer.
 *
 * [TE] §基本的なFP8トレーニングコードの構成: nn.LayerNorm is swapped for the FP8-aware
 * LayerNorm together with nn.Linear. The pages give no formula; the textbook
 * form over the contiguous dimension is computed in FP32:
 *   mu_i = mean_j x_ij, var_i = mean_j (x_ij - mu_i)^2 (divides by cols),
 *   rstd_i = 1 / sqrt(var_i + eps),
 *   y_ij = bf16_rne(((x_ij - mu_i) * rstd_i) * gamma_j + beta_j).
 * The cast is exactly fp8_amax_cast(y, FP8MP_BF16, rows, cols, .., fmt, scale,
 * q, ld_q, NULL, 0, amax) applied to that y:
 *   *amax = max(*amax, max |y|)  (NaN -> 0x7FC00000), q = enc_fmt(y * *scale).
 *
 *   x      rows x cols source (x_dtype), leading dimension ld_x (>= cols).
 *   gamma  cols fp32 (required); beta cols fp32 or NULL (zero).
 *   eps    finite, >= 0.
 *   y      rows x cols BF16, leading dimension ld_y (>= cols), or NULL.
 *   q      rows x cols codes, leading dimension ld_q (>= cols), or NULL;
 *          scale (one fp32 on the device) is required with q.
 *   amax   one fp32 on the device, max-accumulated, or NULL.
 *   mean, rstd  rows fp32 each (the row statistics, for a backward pass), or NULL.
 * rows == 0 or no output is a no-op; cols must be >= 1. Any layout is
 * accepted; BF16 rows with 16-byte alignment, cols a multiple of 8 (<= 16384),
 * ld_x and ld_y multiples of 8, q 8-byte aligned with ld_q a multiple of 8 and
 * gamma/beta 16-byte aligned take the single-read register path.
 */
fp8mp_status fp8_layernorm_amax_cast(const void* x, fp8mp_dtype x_dtype, int64_t rows, int64_t cols,
                                     int64_t ld_x, const float* gamma, const float* beta, float eps,
                                     uint16_t* y, int64_t ld_y, fp8mp_format fmt, const float* scale,
                                     uint8_t* q, int64_t ld_q, float* amax, float* mean, float* rstd,
                                     hipStream_t stream);

/*
 * fp8_reduce_shared_scale: the receive-side arithmetic of an FP8 gradient
 * all-reduce whose ranks share one scale:
 *   out[i] = round_out( (sum_{r=0}^{n_ranks-1} dec(q_r[i])) * (*scale_inv) ),
 * the sum in FP32 in rank order starting from rank 0's value (so a lone -0
 * stays -0), one multiply, then round to nearest even into out_dtype
 * (FP8MP_BF16 or FP8MP_F32).
 *
 * [MPT] §横断的知見 "テンソルスケーリングが FP8 実用化の鍵": FP8-LM shares one scalar
 * over all GPUs for its FP8 all-reduce, s'_g = min(s'_1, ..., s'_N). Since a
 * rank's delayed-scaling scale does not increase with its amax, s'_g is the
 * ordinary update (fp8_scale_update) of the largest amax over the ranks: one
 * MAX all-reduce of the amax slots before the update gives every rank s'_g.
 * Each rank then casts its gradient with s'_g (fp8_amax_cast) and the
 * collective delivers the shards this call sums.
 *
 *   q            n_ranks blocks of numel codes in fmt; block r at q + r * rank_stride
 *                (rank_stride >= numel).
 *   scale_inv    one fp32 on the device: 1 / s'_g.
 *   out          numel values of out_dtype.
 * numel == 0 is a no-op. NaN codes give NaN; E5M2 infinities give infinities.
 * 16-byte aligned q, out and rank_stride take 16-byte loads.
 */
fp8mp_status fp8_reduce_shared_scale(const uint8_t* q, fp8mp_format fmt, int32_t n_ranks, int64_t numel,
                                     int64_t rank_stride, const float* scale_inv, void* out,
                                     fp8mp_dtype out_dtype, hipStream_t stream);

/*
 * fp8_adam_step: one Adam step over decoupled-precision optimizer state.
 *
 * [MPT] §定義 (precision sensitivity of training variables) and §横断的知見
 * "精度分離 (Precision Decoupling)": the first moment tolerates FP8; the second
 * moment and the master weights need more. FP8-LM keeps m in FP8, v in FP16
 * and the master weights in FP16 with tensor scaling (6 bytes per parameter
 * instead of 16). Per parameter, in binary32 in this order (no contraction):
 *   g = grad; m = dec_e4m3(m_q) * m_dq_in; v = fp16 v; w = fp16 w * w_dq_in
 *   m = beta1 * m + (1 - beta1) * g
 *   v = beta2 * v + (1 - beta2) * (g * g)
 *   u = (m * c1) / (sqrt(v * c2) + eps)
 *   w = w - lr * (u + weight_decay * w)
 *   m_q = enc_e4m3(m * m_scale); v = fp16(v); w = fp16(w * w_scale)
 * (FP16 stores: round to nearest even, saturating at +-65504; the FP8 store is
 * the saturating cast of fp8_amax_cast.) *m_amax = max(*m_amax, max |m|) and
 * *w_amax = max(*w_amax, max |w|) feed the delayed updates of m_scale (E4M3)
 * and w_scale (FP8MP_FP16) by fp8_scale_update. *m_dq_out = *m_scale_inv and
 * *w_dq_out = *w_scale_inv: the dequantisation factors of what this step
 * wrote, to be passed as m_dq_in / w_dq_in next step (the out pointers must
 * differ from the in pointers; a caller alternates two of each).
 *
 *   n                 parameters (0: no-op).
 *   grad              n values, FP8MP_BF16 or FP8MP_F32.
 *   m_q, v, w         n bytes / n FP16 / n FP16, read and written in place.
 *   m_dq_in, w_dq_in, m_scale, m_scale_inv, w_scale, w_scale_inv
 *                     one fp32 each on the device (read).
 *   m_dq_out, w_dq_out  one fp32 each (written).
 *   m_amax, w_amax    one fp32 each (max-accumulated) or NULL.
 *   step              t >= 1, the number of this step. The bias corrections are
 *                     formed on the host in binary64 and rounded once to binary32:
 *                     c1 = fp32(1 / (1 - beta1^t)), c2 = fp32(1 / (1 - beta2^t)),
 *                     with beta1, beta2 the binary32 arguments widened
 *                     (0 <= beta1, beta2 < 1, else FP8MP_ERR_INVALID_ARG).
 */
fp8mp_status fp8_adam_step(int64_t n, const void* grad, fp8mp_dtype grad_dtype,
                           uint8_t* m_q, const float* m_dq_in, float* m_dq_out,
                           const float* m_scale, const float* m_scale_inv, float* m_amax,
                           uint16_t* v,
                           uint16_t* w, const float* w_dq_in, float* w_dq_out,
                           const float* w_scale, const float* w_scale_inv, float* w_amax,
                           float lr, float beta1, float beta2, float eps, float weight_decay,
                           int64_t step, hipStream_t stream);

/*
 * fp8_adam_step_weight_cast: fp8_adam_step, and in the same pass the FP8
 * codes of the updated master weights for the next forward GEMM.
 *
 * [MPT] §横断的知見 "FP8 への拡張": the GEMMs run on FP8 operands, so every
 * optimizer step is followed by a cast of the new weights for the next
 * forward; [TE] §動的スケーリングとFP8レシピの設定: that operand keeps its own
 * amax history and delayed scale. Doing the cast here saves the pass that
 * would read the 2-byte master weights again. The weight is taken as stored:
 *   W = fp32(fp16 w) * *w_scale_inv   (binary32; what the next step reads back)
 *   wq[i] = enc_wq_fmt(W[i] * *wq_scale)   (the saturating cast of fp8_amax_cast)
 *   *wq_amax = max(*wq_amax, max |W|)
 * Every other output is exactly fp8_adam_step's.
 *
 *   wq_fmt    FP8MP_E4M3 or FP8MP_E5M2 (FP8MP_FP16 is rejected).
 *   wq_scale  one fp32 on the device: the forward weight's scale in force;
 *             required when wq is given.
 *   wq        n codes, or NULL (amax only).
 *   wq_amax   one fp32, max-accumulated, or NULL; wq and wq_amax are not
 *             both NULL.
 * Errors and ownership as fp8_adam_step.
 */
fp8mp_status fp8_adam_step_weight_cast(int64_t n, const void* grad, fp8mp_dtype grad_dtype,
                                       uint8_t* m_q, const float* m_dq_in, float* m_dq_out,
                                       const float* m_scale, const float* m_scale_inv, float* m_amax,
                                       uint16_t* v,
                                       uint16_t* w, const float* w_dq_in, float* w_dq_out,
                                       const float* w_scale, const float* w_scale_inv, float* w_amax,
                                       float lr, float beta1, float beta2, float eps, float weight_decay,
                                       int64_t step,
                                       fp8mp_format wq_fmt, const float* wq_scale, uint8_t* wq, float* wq_amax,
                                       hipStream_t stream);

/* A static, human-readable name of a status code. Never NULL. */
const char* fp8mp_status_string(fp8mp_status status);

/*
 * Writes "arch=<gcnArchName> cus=<n> formats=e4m3:448,e5m2:57344" for the
 * current device into buf (NUL-terminated, truncated to len). Logs which
 * precision mode runs, as [TE] §FP8非対応GPUでのフォールバック実装 advises.
 * Returns FP8MP_ERR_NO_DEVICE without a device, FP8MP_ERR_WRONG_ARCH (with the
 * text still written) on a device other than gfx950.
 */
fp8mp_status fp8mp_device_info(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* FP8MP_H */
