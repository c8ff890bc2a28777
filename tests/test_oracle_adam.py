"""Pins of the Adam-over-FP8/FP16-state oracle: FP16 encoding against hand cases and numpy's
float16, closed forms of the textbook step, the binary32 step against the float64 one, and
mistakes that the binary32 step must not make."""
import math

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits


def test_fp16_encoding_hand_cases():
    """65504 is FP16's largest value ([MPT] §定義 table); 2049 and 2051 are ties at spacing 2."""
    got = oracle.f16_encode([65504.0, 65519.0, 65520.0, 1e30, -np.inf, 2049.0, 2051.0, 2.0 ** -24, 2.0 ** -26, -0.0])
    want = [0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF, 0xFBFF, 0x6800, 0x6802, 0x0001, 0x0000, 0x8000]
    assert [int(x) for x in got] == want
    assert np.isnan(oracle.f16_decode(oracle.f16_encode([np.nan]))[0])


def test_fp16_encoding_matches_numpy_below_overflow():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-30, 15, 100000))).astype(np.float32)
    x = x[np.abs(x) < 65504]
    assert np.array_equal(oracle.f16_encode(x), x.astype(np.float16).view(np.uint16))


def test_fp16_scale_update_uses_65504():
    s, si, _ = oracle.update_fp16_scale(np.array([2.0, 0.5], np.float32), np.float32(1), np.float32(1))
    assert s == np.float32(32752.0) and si == np.float32(1) / np.float32(32752.0)


def test_first_step_from_zero_state_is_sign_like():
    """t = 1, m = v = 0, wd = 0: m_hat = g, v_hat = g^2, so w' = w - lr g / (|g| + eps)."""
    g = np.array([3.0, -0.25, 1e-3, 0.0])
    b1, b2, lr, eps = 0.9, 0.999, 1e-2, 1e-8
    m, v, w = oracle.adam_step_f64(g, 0, 0, 1.0, lr, b1, b2, eps, 0.0, 1 / (1 - b1), 1 / (1 - b2))
    assert np.allclose(w, 1.0 - lr * g / (np.abs(g) + eps), rtol=0, atol=1e-15)
    assert np.allclose(m, (1 - b1) * g) and np.allclose(v, (1 - b2) * g * g)


def test_zero_betas_and_pure_weight_decay():
    g = np.array([2.0, -4.0])
    m, v, w = oracle.adam_step_f64(g, 5.0, 7.0, 3.0, 0.1, 0.0, 0.0, 0.0, 0.0, 1.0, 1.0)
    assert np.array_equal(m, g) and np.array_equal(v, g * g) and np.allclose(w, 3.0 - 0.1 * np.sign(g))
    m, v, w = oracle.adam_step_f64(np.zeros(2), 0.0, 1.0, np.array([2.0, -8.0]), 0.5, 0.9, 0.99, 1e-8, 0.1, 1.0, 1.0)
    assert np.allclose(w, np.array([2.0, -8.0]) * (1 - 0.5 * 0.1))


def _state(rng, n):
    g = f32_to_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32))
    m_q = oracle.cast((rng.standard_normal(n) * 1e-3).astype(np.float32), np.float32(2.0 ** 14), "e4m3")
    v = oracle.f16_encode(np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32))
    w = oracle.f16_encode((rng.standard_normal(n) * 0.02 * 1024).astype(np.float32))
    return g, m_q, v, w


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01, c1=1 / (1 - 0.9 ** 7), c2=1 / (1 - 0.999 ** 7))


def test_binary32_step_agrees_with_float64_step():
    rng = np.random.default_rng(1)
    n = 20000
    g, m_q, v, w = _state(rng, n)
    m_dq, w_dq = np.float32(2.0 ** -14), np.float32(1 / 1024)
    mq2, v2, w2, m_amax, w_amax = oracle.adam_step_ref(g, "bf16", m_q, m_dq, 2.0 ** 14, v, w, w_dq, 1024.0, **HP)
    gd = oracle.bf16_to_f32(g).astype(np.float64)
    md = oracle.decode_table("e4m3")[m_q] * float(m_dq)
    vd = oracle.f16_decode(v).astype(np.float64)
    wd_ = oracle.f16_decode(w).astype(np.float64) * float(w_dq)
    m64, v64, w64 = oracle.adam_step_f64(gd, md, vd, wd_, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"],
                                         HP["c1"], HP["c2"])
    # stored values: within the storage rounding (FP16 half unit, FP8 half unit) plus a few binary32 units
    w_got = oracle.f16_decode(w2).astype(np.float64) / 1024.0
    assert np.all(np.abs(w_got - w64) <= 2.0 ** -11 * np.abs(w64) + 1e-9)
    v_got = oracle.f16_decode(v2).astype(np.float64)
    assert np.all(np.abs(v_got - v64) <= 2.0 ** -11 * np.abs(v64) + 2.0 ** -25)
    m_got = oracle.decode_table("e4m3")[mq2] / 2.0 ** 14
    assert np.all(np.abs(m_got - m64) <= 2.0 ** -4 * np.abs(m64) + 2.0 ** -9 / 2.0 ** 14)
    assert abs(float(m_amax) - np.abs(m64).max()) <= 1e-6 * np.abs(m64).max()
    assert abs(float(w_amax) - np.abs(w64).max()) <= 1e-6 * np.abs(w64).max()


def test_binary32_step_rejects_plausible_mistakes():
    """A dropped bias correction, eps inside the root, swapped betas or a weight-decay sign flip change the
    stored master weights."""
    rng = np.random.default_rng(2)
    g, m_q, v, w = _state(rng, 4000)
    args = (g, "bf16", m_q, 2.0 ** -14, 2.0 ** 14, v, w, 1 / 1024, 1024.0)
    ref = oracle.adam_step_ref(*args, **HP)[2]
    for name, hp in {"no bias correction": dict(HP, c1=1.0, c2=1.0),
                     "betas swapped": dict(HP, beta1=HP["beta2"], beta2=HP["beta1"]),
                     "weight decay sign": dict(HP, wd=-HP["wd"]),
                     "lr doubled": dict(HP, lr=2 * HP["lr"])}.items():
        assert not np.array_equal(oracle.adam_step_ref(*args, **hp)[2], ref), name


def test_weight_codes_hand_cases():
    """Stored FP16 weights read back with the inverse scale, then cast. OCP E4M3: 1.0 = 0x38, 2.0 = 0x40,
    0.375 = 0x2C (1.5 * 2^-2: exponent field 5, mantissa 100), 448 = 0x7E (largest), the NaN code 0x7F; E5M2: 1.0 = 0x3C, 57344 = 0x7B."""
    w = oracle.f16_encode([4.0, -4.0, 1.5, 0.0, 60000.0, np.nan])          # stored values of w * s_w
    q, am = oracle.adam_weight_codes_ref(w, 0.5, 0.5, "e4m3")             # W = 2, -2, 0.75, 0, 30000, NaN
    assert [int(x) for x in q[:5]] == [0x38, 0xB8, 0x2C, 0x00, 0x7E]     # W * 0.5 = 1, -1, 0.375, 0, 15000 -> 448
    assert int(q[5]) & 0x7F == 0x7F and np.isnan(am)
    q, am = oracle.adam_weight_codes_ref(w[:5], 0.5, 2.0, "e5m2")        # W * 2 = 4, -4, 1.5, 0, 60000 -> 57344
    assert [int(x) for x in q] == [0x44, 0xC4, 0x3E, 0x00, 0x7B]
    assert am == np.float32(30000.0)


def test_weight_codes_follow_the_stored_value_not_the_fp32_one():
    """W is read back from FP16: 1 + 2^-12 is stored as 1.0 (spacing 2^-10 there), so a scale that puts
    1.0 exactly on an E4M3 code gives that code, while the unrounded value would sit above it."""
    w = oracle.f16_encode([1.0 + 2.0 ** -12])
    assert int(w[0]) == 0x3C00
    q, am = oracle.adam_weight_codes_ref(w, 1.0, 1.0, "e4m3")
    assert int(q[0]) == 0x38 and am == np.float32(1.0)



def test_bias_corrections_exact_rationals():
    """fp32(1 / (1 - beta**t)) from the binary32 beta: against exact rational arithmetic rounded to binary32
    where the exact value is not within 2**-40 (relative) of a binary32 rounding boundary, for the usual
    betas over many steps; t = 1 gives 1 / (1 - beta); the corrections fall towards 1 as t grows."""
    from fractions import Fraction
    for beta in (0.9, 0.95, 0.99, 0.999, 0.9999, 0.5, 0.0):
        b = Fraction(float(np.float32(beta)))
        prev = None
        for t in (1, 2, 3, 7, 10, 100, 1000, 10000, 123457):
            c1, _ = oracle.bias_corrections(beta, 0.5, t)
            exact = 1 / (1 - b ** t)
            lo = np.float32(float(exact))            # nearest binary32 (ties aside)
            nb = np.nextafter(lo, np.float32(np.inf)) if Fraction(float(lo)) < exact else np.nextafter(lo, np.float32(0))
            mid = (Fraction(float(lo)) + Fraction(float(nb))) / 2
            if abs(exact - mid) > exact * Fraction(1, 2 ** 40):
                assert c1 == lo, (beta, t, c1, lo)
            if prev is not None:
                assert c1 <= prev
            prev = c1
        assert oracle.bias_corrections(beta, beta, 1)[0] == np.float32(1 / (1 - float(np.float32(beta))))
    assert oracle.bias_corrections(0.0, 0.0, 5) == (np.float32(1), np.float32(1))
    with pytest.raises(ValueError):
        oracle.bias_corrections(0.9, 0.999, 0)
