"""CPU oracle for the per-tensor-scaled FP8 linear layer (test infrastructure).

This package is test infrastructure. Only the tests, the smoke check in
``__graft_entry__`` and the benchmark's CPU-baseline leg may import it. The
product path (the HIP library and its Python binding) never calls it, and it
never calls the product path: the two share no code. Both consume the same
host arrays from ``workloads``.

It is plain, slow and written to be checked by eye: NumPy, float64 wherever a
value is formed, one function per step of the method, each citing the passage
it follows. The sources are three web pages:

  [TE]   「AI：NVIDIA Transformer EngineとFP8混合精度の実装ガイド｜環境構築からベンチマークまで」
         https://ai-tool-zukan.com/?p=579
  [TRT]  「NVIDIA TensorRTによるFP8量子化：高性能推論エンジンの実現」
         https://ai.warp-studio.com/blog/2026-06-09-19551-model-quantization-turn-fp8-checkpoints-into-high-performance-inference-engines-with-nvidia-tensorrt/
  [MPT]  「混合精度訓練」 https://notes.yuuk.io/wiki/concepts/混合精度訓練

What the pages fix: the two FP8 layouts (E4M3 = 4 exponent + 3 mantissa bits,
E5M2 = 5 + 2; [TE] §TEとFP8混合精度とは, [TRT] §FP8量子化の技術的優位性と背景),
their largest values 448 and 57344 and "E5M2 has FP16's range"
([MPT] §定義, precision table), the delayed-scaling recipe with an amax history,
margin and format choice ([TE] §動的スケーリングとFP8レシピの設定, [MPT]
§横断的知見 "テンソルスケーリングが FP8 実用化の鍵"), and that only the GEMMs run in
FP8 with FP32 accumulation ([MPT] §横断的知見 "FP8 への拡張" and "HPC ソルバーとの目的の分岐").

What the pages leave open is read as follows (each reading is pinned by a
test under tests/):
  * scale s multiplies to quantise, q = enc(fp32(x) * s); 1/s dequantises;
  * s = fp32(fp32(fmax / max(history)) * 2**-margin), held (not changed) when
    max(history) is not finite and positive, or when the new s or its inverse
    fp32(1 / s) is not finite and positive; s_inv = fp32(1 / s);
  * "delayed": the cast at step t uses the s computed after step t-1 and
    records step t's amax in the same pass; cold start is s = 1, history = 0;
  * the update runs every step; it takes the max over all history entries,
    then rolls the history by one (the newest slot becomes 0);
  * encode rounds to nearest, ties to even, and saturates: every |v| >= fmax,
    +-Inf included, maps to the largest finite code of that sign; NaN maps to
    sign | 0x7F; FP8 subnormals are produced; a zero result keeps its sign;
  * the sign of a NaN product x * s is sign(x) xor sign(s) (IEEE 754 leaves
    it open);
  * OCP variants: E4M3 has bias 7, no infinities and one NaN code per sign;
    E5M2 has bias 15 and IEEE-style Inf/NaN;
  * amax is max |x| in fp32; any NaN gives the canonical NaN 0x7FC00000.
"""
from .codec import (FMT, FP8Format, decode, decode_table, encode, encode_scalar,
                    bf16_to_f32)
from .recipe import (amax, cast, DelayedScaling, max_nan, primed_scale, update_scale, update_scale_fmax)
from .gemm import gemm_ref, gemm_abs_ref, gemm_bound, gemm_check, gemm_entry, gemm_ratio
from .layernorm import layer_norm_bound, layer_norm_check, layer_norm_ref
from .allreduce import reduce_bound, reduce_check, reduce_ref, shared_scale
from .adam import (adam_step_f64, adam_step_ref, adam_weight_codes_ref, bias_corrections, f16_decode, f16_encode,
                   update_fp16_scale)

__all__ = [
    "FMT", "FP8Format", "decode", "decode_table", "encode", "encode_scalar", "bf16_to_f32",
    "amax", "cast", "DelayedScaling", "max_nan", "primed_scale", "update_scale", "update_scale_fmax",
    "gemm_ref", "gemm_abs_ref", "gemm_bound", "gemm_check", "gemm_entry", "gemm_ratio",
    "layer_norm_ref", "layer_norm_bound", "layer_norm_check",
    "shared_scale", "reduce_ref", "reduce_bound", "reduce_check",
    "adam_step_ref", "adam_step_f64", "adam_weight_codes_ref", "bias_corrections", "f16_encode", "f16_decode", "update_fp16_scale",
]
