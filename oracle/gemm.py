"""FP64 reference for the scaled FP8 GEMM and its tolerance.

Test infrastructure only (see the package docstring).

[MPT] §横断的知見 "FP8 への拡張": Transformer Engine runs only the GEMMs in FP8.
[MPT] §横断的知見 "HPC ソルバーとの目的の分岐": tensor cores accumulate in FP32.
The layer's output is Y = (Xq . Wq^T) / (sx * sw): the FP8 operands are decoded,
multiplied and summed, and the inverse scales dequantise the sum. Here both
operands are K-contiguous: A[m x k], B[n x k], C = A . B^T.

Every product of two FP8 values is exact in float64 (at most 4 x 4 significant
bits) and the float64 sum's error, at most (K-1) * 2**-53 * sum|a*b|, is far
below the tolerance, so the float64 result stands for the exact one.

Tolerance for a BF16 output y (widened to float64):
    |y - y_ref| <= 2**-7 * |y_ref| + 1e-6 * sum_k |a_k * b_k|
with a_k, b_k the dequantised operands (decoded code times inverse scale).
2**-7 is BF16's epsilon ([MPT] §定義 precision table lists BF16's relative
error as about 1e-2); the second term absorbs FP32 accumulation.

Fast accumulation (the opt-in GEMM on the FP8 matrix instruction) does not
accumulate in FP32, so it is graded with a larger second coefficient,
FAST_ACCUM_SUM_COEF = 2**-9. The pages say nothing of it; the figure follows
from how that instruction sums: each block of 64 products is aligned to its
largest product and kept to 16 bits below that product's binade, so a block
loses less than 64 * 2**-16 = 2**-10 of its largest |product|, hence of its
sum|a*b|; 2**-9 leaves a factor of two for the FP32 adds between blocks and
the BF16 rounding. This bound is a property of that hardware reduction
(measured: at most 2**-10.9 of the largest product per block), not a pinned
statement of the pages.
"""
from __future__ import annotations

import numpy as np

from .codec import _fmt, decode_table


def _dec(codes, fmt) -> np.ndarray:
    return decode_table(_fmt(fmt))[np.asarray(codes, dtype=np.uint8)]


def gemm_ref(a_codes, a_fmt, b_codes, b_fmt, a_scale_inv, b_scale_inv) -> np.ndarray:
    """y_ref = (dec(A) . dec(B)^T) * a_scale_inv * b_scale_inv, float64."""
    A = _dec(a_codes, a_fmt)
    B = _dec(b_codes, b_fmt)
    return (A @ B.T) * float(a_scale_inv) * float(b_scale_inv)


def gemm_abs_ref(a_codes, a_fmt, b_codes, b_fmt, a_scale_inv, b_scale_inv) -> np.ndarray:
    """sum_k |a_k * b_k| for every output entry (the accumulation term of the bound)."""
    A = np.abs(_dec(a_codes, a_fmt))
    B = np.abs(_dec(b_codes, b_fmt))
    return (A @ B.T) * abs(float(a_scale_inv)) * abs(float(b_scale_inv))


def gemm_entry(a_codes, a_fmt, b_codes, b_fmt, a_scale_inv, b_scale_inv, i, j):
    """One output entry and its bound term, for sampled checks at full size."""
    a = _dec(np.asarray(a_codes)[i], a_fmt)
    b = _dec(np.asarray(b_codes)[j], b_fmt)
    sa, sb = float(a_scale_inv), float(b_scale_inv)
    return float(np.dot(a, b)) * sa * sb, float(np.dot(np.abs(a), np.abs(b))) * abs(sa) * abs(sb)


SUM_COEF = 1e-6
FAST_ACCUM_SUM_COEF = 2.0 ** -9


def gemm_bound(y_ref, abs_ref, sum_coef=SUM_COEF) -> np.ndarray:
    return 2.0 ** -7 * np.abs(y_ref) + sum_coef * np.asarray(abs_ref)


def bf16_bits_to_f64(y_bits) -> np.ndarray:
    y = np.asarray(y_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return y.view(np.float32).astype(np.float64)


def gemm_ratio(y_bits, y_ref, abs_ref, sum_coef=SUM_COEF) -> np.ndarray:
    """|y - y_ref| / bound for every entry (float64, the shape of y_ref).

    A finite reference with a zero bound gives 0 when y equals it and inf
    otherwise. A non-finite reference (NaN or Inf codes among the operands)
    gives 0 when y matches it in kind (NaN for NaN, the same infinity) and inf
    otherwise. An entry is within the tolerance exactly when its ratio is <= 1.
    """
    y = bf16_bits_to_f64(y_bits)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    abs_ref = np.asarray(abs_ref, dtype=np.float64)
    ratio = np.zeros(y_ref.shape, np.float64)
    fin = np.isfinite(y_ref)
    if (~fin).any():
        yr, yy = y_ref[~fin], y[~fin]
        same = (np.isnan(yr) & np.isnan(yy)) | (yr == yy)
        ratio[~fin] = np.where(same, 0.0, np.inf)
    bound = gemm_bound(y_ref[fin], abs_ref[fin], sum_coef)
    with np.errstate(invalid="ignore"):
        err = np.abs(y[fin] - y_ref[fin])
    err = np.where(np.isfinite(err), err, np.inf)
    safe = np.where(bound > 0, bound, 1.0)
    ratio[fin] = np.where(bound > 0, err / safe, np.where(err > 0, np.inf, 0.0))
    return ratio


def gemm_check(y_bits, y_ref, abs_ref, sum_coef=SUM_COEF):
    """Grade BF16 output bits against the reference.

    Returns (ok, worst): ok when every entry is within the tolerance (see
    gemm_ratio), worst the largest |y - y_ref| / bound over the entries with a
    finite reference (0.0 when there are none). sum_coef is the coefficient of
    sum_k |a_k b_k| in the bound: SUM_COEF for FP32 accumulation,
    FAST_ACCUM_SUM_COEF for fast accumulation.
    """
    ratio = gemm_ratio(y_bits, y_ref, abs_ref, sum_coef)
    fin = np.isfinite(np.asarray(y_ref, dtype=np.float64))
    ok = bool((ratio <= 1.0).all())
    worst = float(ratio[fin].max()) if fin.any() else 0.0
    return ok, worst
