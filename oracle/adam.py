"""Reference for one Adam step over FP8/FP16 optimizer state (precision decoupling).

Test infrastructure only (see the package docstring).

[MPT] §定義 (the precision-sensitivity list after the table) and §横断的知見
"精度分離 (Precision Decoupling)": master weights and the second moment need
high precision (tiny updates; squaring underflows), the first moment
tolerates low precision. FP8-LM keeps Adam's first moment in FP8, the second
moment in FP16 and the master weights in FP16 with tensor scaling, 6 bytes per
parameter instead of 16. FP16 tops out at 65504 ([MPT] §定義, precision table).

The pages name the storage precisions only. Readings taken:
  * Adam with decoupled weight decay (wd = 0 is plain Adam); the bias
    corrections of step t are c1 = 1 / (1 - beta1**t), c2 = 1 / (1 - beta2**t),
    formed in float64 from the binary32 betas and rounded once to binary32
    (`bias_corrections`);
  * the first moment is E4M3 codes with one scale per tensor; the master
    weights are FP16 values of w * s_w with one scale per tensor; both scales
    follow the delayed recipe (the step writes with the current scale and
    records the new tensor's amax); the second moment is plain FP16;
  * stored values are read back with the inverse of the scale they were
    written with (dq); FP16 stores round to nearest even and saturate at
    +-65504, like the FP8 casts.

`adam_step_ref` is the step as the kernel evaluates it, in binary32, one
operation at a time in this order (numpy float32 arithmetic is IEEE binary32
with round to nearest even):
    g  = grad;  m = dec(m_q) * m_dq;  v = fp16(v);  w = fp16(w) * w_dq
    m  = beta1 * m + (1 - beta1) * g
    v  = beta2 * v + (1 - beta2) * (g * g)
    u  = (m * c1) / (sqrt(v * c2) + eps)
    w  = w - lr * (u + wd * w)
    m_q = enc_e4m3(m * m_scale);  v = fp16(v);  w = fp16(w * w_scale)
    m_amax = max |m|;  w_amax = max |w|
The stored codes are decided in that precision, so the kernel's codes must
match these bit for bit. `adam_step_f64` is the textbook step in float64 on
the same decoded state; it pins the binary32 evaluation.
"""
from __future__ import annotations

import numpy as np

from .codec import bf16_to_f32, decode_table
from .recipe import cast, max_nan, update_scale_fmax

FP16_MAX = 65504.0


def bias_corrections(beta1, beta2, t: int):
    """Adam's bias corrections of step t >= 1: fp32(1 / (1 - beta**t)) for each beta, with beta the
    binary32 value widened to float64 and the power, difference and quotient taken in float64."""
    if t < 1:
        raise ValueError("step numbers start at 1")
    b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
    return np.float32(1.0 / (1.0 - b1 ** t)), np.float32(1.0 / (1.0 - b2 ** t))


def f16_encode(x) -> np.ndarray:
    """binary32 -> FP16 bits, round to nearest even, saturating at +-65504 (NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        h = x.astype(np.float16)                         # IEEE conversion, round to nearest even
    h = np.where(np.isinf(h) & ~np.isinf(x) | np.isinf(x), np.copysign(np.float16(FP16_MAX), x).astype(np.float16), h)
    return h.view(np.uint16)


def f16_decode(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def _grad(grad, g_dtype):
    return bf16_to_f32(grad) if g_dtype == "bf16" else np.asarray(grad, dtype=np.float32)


def adam_step_ref(grad, g_dtype, m_q, m_dq, m_scale, v_bits, w_bits, w_dq, w_scale,
                  lr, beta1, beta2, eps, wd, c1, c2):
    """The binary32 step. Returns (m_q, v_bits, w_bits, m_amax, w_amax)."""
    f = np.float32
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        g = _grad(grad, g_dtype)
        m = decode_table("e4m3")[np.asarray(m_q, np.uint8)].astype(f) * f(m_dq)
        v = f16_decode(v_bits)
        w = f16_decode(w_bits) * f(w_dq)
        m = f(beta1) * m + (f(1) - f(beta1)) * g
        v = f(beta2) * v + (f(1) - f(beta2)) * (g * g)
        u = (m * f(c1)) / (np.sqrt(v * f(c2)) + f(eps))
        w = w - f(lr) * (u + f(wd) * w)
        m_new = cast(m, f(m_scale), "e4m3", "f32")
        v_new = f16_encode(v)
        w_new = f16_encode(w * f(w_scale))
    return m_new, v_new, w_new, max_nan(np.abs(m)), max_nan(np.abs(w))


def adam_weight_codes_ref(w_bits, w_scale_inv, wq_scale, fmt):
    """The next forward's weight operand from the master weights as stored.

    [MPT] §横断的知見 "FP8 への拡張": the GEMM operands are FP8, so the updated weights
    are cast before the next forward, with their own delayed scale ([TE]
    §動的スケーリングとFP8レシピの設定). Reading taken: the weight cast is the stored
    master weight, read back the way the next step reads it,
        W = fp32(fp16 w) * w_scale_inv   (binary32),
    then the saturating cast of W with the forward weight's scale; amax = max |W|.
    Returns (codes, amax)."""
    with np.errstate(over="ignore", invalid="ignore"):
        W = f16_decode(w_bits) * np.float32(w_scale_inv)
    return cast(W, np.float32(wq_scale), fmt, "f32"), max_nan(np.abs(W))


def adam_step_f64(g, m, v, w, lr, beta1, beta2, eps, wd, c1, c2):
    """Textbook Adam with decoupled weight decay, float64. Returns (m, v, w)."""
    g, m, v, w = (np.asarray(a, dtype=np.float64) for a in (g, m, v, w))
    m = beta1 * m + (1 - beta1) * g
    v = beta2 * v + (1 - beta2) * g * g
    w = w - lr * ((m * c1) / (np.sqrt(v * c2) + eps) + wd * w)
    return m, v, w


def update_fp16_scale(history, scale, scale_inv, margin: int = 0):
    """The delayed-scaling update towards FP16 storage (largest value 65504)."""
    return update_scale_fmax(history, scale, scale_inv, FP16_MAX, margin)
