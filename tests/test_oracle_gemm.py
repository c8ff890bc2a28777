"""Pins for the oracle's FP64 GEMM and its tolerance.

The checks use exact integer arithmetic on the codes' bit fields, Python
integers, and a brute-force triple loop, so that a transposed operand, a wrong
index, a dropped term or a wrong scale in the oracle fails one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle.codec import FMT
from oracle.gemm import (SUM_COEF, bf16_bits_to_f64, gemm_abs_ref, gemm_check, gemm_entry, gemm_ratio, gemm_ref)


def _finite_codes(rng, shape, name):
    top = FMT[name].max_code
    c = rng.integers(0, top + 1, shape, dtype=np.int64)
    sign = rng.integers(0, 2, shape, dtype=np.int64) << 7
    return (c | sign).astype(np.uint8)


def _int_value(code: int, name: str) -> int:
    """Value of a finite code as an integer multiple of its format's smallest subnormal.

    Written from the fields with integer arithmetic only: subnormal m, normal
    (2**M + m) * 2**(e - 1).
    """
    f = FMT[name]
    s = -1 if code & 0x80 else 1
    e = (code >> f.man_bits) & ((1 << f.exp_bits) - 1)
    m = code & ((1 << f.man_bits) - 1)
    if e == 0:
        return s * m
    return s * (((1 << f.man_bits) + m) << (e - 1))


UNIT = {"e4m3": Fraction(1, 2 ** 9), "e5m2": Fraction(1, 2 ** 16)}


def test_e4m3_gemm_is_exact_integer_gemm():
    rng = np.random.default_rng(0)
    A = _finite_codes(rng, (37, 200), "e4m3")
    B = _finite_codes(rng, (45, 200), "e4m3")
    lut = np.array([_int_value(c, "e4m3") if (c & 0x7F) <= 0x7E else 0 for c in range(256)], np.int64)
    exact = lut[A] @ lut[B].T                       # int64: |sum| < 2**50
    ref = gemm_ref(A, "e4m3", B, "e4m3", 1.0, 1.0)
    assert np.array_equal(ref, exact.astype(np.float64) * 2.0 ** -18)
    assert np.array_equal(exact.astype(np.float64) * 2.0 ** -18, exact * 2.0 ** -18)


def test_e5m2_by_e4m3_matches_python_integers():
    rng = np.random.default_rng(1)
    A = _finite_codes(rng, (5, 33), "e5m2")
    B = _finite_codes(rng, (7, 33), "e4m3")
    sa, sb = np.float32(0.375), np.float32(3.0)
    ref = gemm_ref(A, "e5m2", B, "e4m3", sa, sb)
    for i in range(5):
        for j in range(7):
            acc = sum(_int_value(int(A[i, k]), "e5m2") * _int_value(int(B[j, k]), "e4m3") for k in range(33))
            want = Fraction(acc) * UNIT["e5m2"] * UNIT["e4m3"] * Fraction(0.375) * Fraction(3.0)
            assert abs(Fraction(ref[i, j]) - want) <= abs(want) * Fraction(1, 2 ** 50)


def test_triple_loop_non_square():
    rng = np.random.default_rng(2)
    from oracle.codec import decode
    A = _finite_codes(rng, (3, 11), "e5m2")
    B = _finite_codes(rng, (4, 11), "e4m3")
    ref = gemm_ref(A, "e5m2", B, "e4m3", 2.0, 0.5)
    for i in range(3):
        for j in range(4):
            s = 0.0
            for k in range(11):
                s += decode(A[i, k], "e5m2") * decode(B[j, k], "e4m3")
            assert ref[i, j] == pytest.approx(s, rel=1e-15, abs=1e-300)
            r, b = gemm_entry(A, "e5m2", B, "e4m3", 2.0, 0.5, i, j)
            assert r == pytest.approx(ref[i, j], rel=1e-15, abs=1e-300)


def test_abs_sum_and_entry_match_exact_rational_triple_loop():
    """sum_k |a_k b_k| (gemm_abs_ref and gemm_entry's second value) against a triple loop in exact
    rationals over the codes' integer values, with negative and non-power-of-two inverse scales, so
    that a missing abs on either operand or on a scale, a dropped term or a transposed pairing fails."""
    rng = np.random.default_rng(5)
    for af, bf, (m, n, k) in [("e5m2", "e4m3", (4, 5, 23)), ("e4m3", "e4m3", (3, 6, 40)),
                              ("e4m3", "e5m2", (5, 2, 17))]:
        A = _finite_codes(rng, (m, k), af)
        B = _finite_codes(rng, (n, k), bf)
        sa, sb = np.float32(-0.3), np.float32(1.75)
        absr = gemm_abs_ref(A, af, B, bf, sa, sb)
        ref = gemm_ref(A, af, B, bf, sa, sb)
        fa, fb = Fraction(float(sa)), Fraction(float(sb))
        for i in range(m):
            for j in range(n):
                tot = Fraction(0)
                val = Fraction(0)
                for kk in range(k):
                    p = (Fraction(_int_value(int(A[i, kk]), af)) * UNIT[af] *
                         Fraction(_int_value(int(B[j, kk]), bf)) * UNIT[bf])
                    tot += abs(p)
                    val += p
                want_abs = tot * abs(fa) * abs(fb)
                want = val * fa * fb
                assert abs(Fraction(absr[i, j]) - want_abs) <= want_abs * Fraction(1, 2 ** 50)
                r, b = gemm_entry(A, af, B, bf, sa, sb, i, j)
                assert abs(Fraction(b) - want_abs) <= want_abs * Fraction(1, 2 ** 50)
                assert abs(Fraction(r) - want) <= tot * abs(fa * fb) * Fraction(1, 2 ** 50)
                assert abs(Fraction(ref[i, j]) - want) <= tot * abs(fa * fb) * Fraction(1, 2 ** 50)
        # the bound term is never smaller than |y| and is the plain sum when all products are >= 0
        assert (absr >= np.abs(ref) * (1 - 2 ** -50)).all()
    P = np.full((2, 8), 0x40, np.uint8)           # E4M3 2.0
    Q = np.full((3, 8), 0x38, np.uint8)           # E4M3 1.0
    assert np.array_equal(gemm_abs_ref(P, "e4m3", Q, "e4m3", 0.5, 3.0), np.full((2, 3), 24.0))
    assert np.array_equal(gemm_abs_ref(P, "e4m3", Q, "e4m3", 0.5, 3.0),
                          np.abs(gemm_ref(P, "e4m3", Q, "e4m3", 0.5, 3.0)))


def test_ratio_hand_values_and_counts():
    """gemm_ratio on hand-computed entries: the bound 2**-7 |y_ref| + c * sum|ab| evaluated by hand,
    zero bounds, NaN and infinite references, and the count of planted violations."""
    y_ref = np.array([[100.0, 100.0, 0.0, 0.0, np.nan, np.inf, -np.inf, 3.0]])
    absr = np.array([[200.0, 200.0, 0.0, 0.0, 1.0, 1.0, 1.0, 1e7]])
    # BF16 bits: 101.0, 100.0, 0.0, 1.0, NaN, +Inf, +Inf, 0.0
    y = np.array([[0x42CA, 0x42C8, 0x0000, 0x3F80, 0x7FC0, 0x7F80, 0x7F80, 0x0000]], np.uint16)
    r = gemm_ratio(y, y_ref, absr)
    want0 = 1.0 / (2.0 ** -7 * 100.0 + SUM_COEF * 200.0)
    assert r[0, 0] == pytest.approx(want0, rel=1e-15)
    assert r[0, 1] == 0.0 and r[0, 2] == 0.0 and r[0, 3] == np.inf
    assert r[0, 4] == 0.0 and r[0, 5] == 0.0 and r[0, 6] == np.inf
    assert r[0, 7] == pytest.approx(3.0 / (2.0 ** -7 * 3.0 + 10.0), rel=1e-15)
    assert int((r > 1).sum()) == 3
    ok, worst = gemm_check(y, y_ref, absr)
    assert not ok and worst == np.inf
    # a larger sum coefficient only lowers the ratio of finite entries
    r2 = gemm_ratio(y, y_ref, absr, 2.0 ** -9)
    assert r2[0, 0] == pytest.approx(1.0 / (2.0 ** -7 * 100.0 + 2.0 ** -9 * 200.0), rel=1e-15)
    rng = np.random.default_rng(6)
    A = _finite_codes(rng, (20, 64), "e4m3")
    B = _finite_codes(rng, (30, 64), "e4m3")
    ref = gemm_ref(A, "e4m3", B, "e4m3", 0.5, 0.25)
    ab = gemm_abs_ref(A, "e4m3", B, "e4m3", 0.5, 0.25)
    bits = _to_bf16_bits(ref)
    assert (gemm_ratio(bits, ref, ab) <= 1.0).all()
    bad = bits.copy()
    pos = [(0, 0), (7, 13), (19, 29)]
    for i, j in pos:
        bad[i, j] ^= 0x8000 if ref[i, j] != 0 else 0x3F80   # flip the sign (or plant 1.0 for a zero)
    rr = gemm_ratio(bad, ref, ab)
    assert sorted(map(tuple, np.argwhere(rr > 1.0).tolist())) == pos


def _to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 (via float32) for the tolerance checks."""
    u = y.astype(np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def test_tolerance_accepts_rounded_and_rejects_wrong_results():
    rng = np.random.default_rng(3)
    K = 512
    A = _finite_codes(rng, (16, K), "e4m3")
    B = _finite_codes(rng, (24, K), "e4m3")
    sa, sb = np.float32(1 / 64), np.float32(1 / 32)
    ref = gemm_ref(A, "e4m3", B, "e4m3", sa, sb)
    absr = gemm_abs_ref(A, "e4m3", B, "e4m3", sa, sb)
    ok, worst = gemm_check(_to_bf16_bits(ref), ref, absr)
    assert ok and worst < 0.6
    # dropping the last k term
    ref_drop = gemm_ref(A[:, :-1], "e4m3", B[:, :-1], "e4m3", sa, sb)
    big = np.abs(ref - ref_drop) > 2 * (2.0 ** -7 * np.abs(ref) + 1e-6 * absr)
    assert big.any()
    assert not gemm_check(_to_bf16_bits(ref_drop), ref, absr)[0]
    # transposed operand pairing (B . A^T has a different shape; use a square case)
    Bs = _finite_codes(rng, (16, K), "e4m3")
    ref_s = gemm_ref(A, "e4m3", Bs, "e4m3", sa, sb)
    abs_s = gemm_abs_ref(A, "e4m3", Bs, "e4m3", sa, sb)
    assert not gemm_check(_to_bf16_bits(ref_s.T), ref_s, abs_s)[0]
    # a wrong scale (one inverse scale applied twice)
    assert not gemm_check(_to_bf16_bits(ref * float(sa)), ref, absr)[0]
    # sign flip
    assert not gemm_check(_to_bf16_bits(-ref), ref, absr)[0]


def test_nan_codes_propagate_and_are_graded():
    A = np.array([[0x7F, 0x38]], np.uint8)      # NaN, 1.0 (E4M3)
    B = np.array([[0x38, 0x38]], np.uint8)
    ref = gemm_ref(A, "e4m3", B, "e4m3", 1.0, 1.0)
    assert np.isnan(ref).all()
    nan_bits = np.array([[0x7FC0]], np.uint16)
    absr = gemm_abs_ref(A, "e4m3", B, "e4m3", 1.0, 1.0)
    assert gemm_check(nan_bits, ref, absr)[0]
    assert not gemm_check(np.array([[0x3F80]], np.uint16), ref, absr)[0]


def test_bf16_output_widening():
    assert bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000], np.uint16)).tolist() == [1.0, -2.0, 0.0]


def _aligned_block_gemm(A, af, B, bf, sa, sb, block=64, frac_bits=16):
    """A model of a reduced-precision matrix instruction: each block of `block` products is aligned
    to the binade of its largest |product|, truncated toward zero to frac_bits bits below it and summed
    exactly; the block sums are added in FP32; the result is scaled in FP32. Written here from that
    description (not from the oracle) to exercise the fast-accumulation bound."""
    from oracle.codec import decode_table
    da = decode_table(FMT[af].name)[A].astype(np.float64)
    db = decode_table(FMT[bf].name)[B].astype(np.float64)
    m, k = da.shape
    n = db.shape[0]
    out = np.zeros((m, n), np.float32)
    for i in range(m):
        p = da[i][None, :] * db            # n x k exact products
        acc = np.zeros(n, np.float32)
        for k0 in range(0, k, block):
            blk = p[:, k0:k0 + block]
            mx = np.abs(blk).max(axis=1)
            e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
            q = np.ldexp(1.0, (e - frac_bits).astype(int))[:, None]
            s = (np.trunc(blk / q) * q).sum(axis=1)
            acc = (acc.astype(np.float64) + s).astype(np.float32)
        out[i] = acc * (np.float32(sa) * np.float32(sb))
    return out.astype(np.float64)


def test_fast_accumulation_bound_holds_for_the_aligned_block_model():
    """The fast-accumulation bound (2**-9 * sum|ab|) accepts the aligned-block reduction on
    full-range random codes and on blocks with one dominant product, while the FP32 bound rejects the
    latter; exact sums come out when every product of a block has one magnitude."""
    from oracle.gemm import FAST_ACCUM_SUM_COEF
    rng = np.random.default_rng(11)
    for af, bf in [("e4m3", "e4m3"), ("e5m2", "e4m3")]:
        A = _finite_codes(rng, (12, 256), af)
        B = _finite_codes(rng, (10, 256), bf)
        sa, sb = np.float32(1 / 16), np.float32(3.0)
        y = _aligned_block_gemm(A, af, B, bf, sa, sb)
        ref = gemm_ref(A, af, B, bf, sa, sb)
        absr = gemm_abs_ref(A, af, B, bf, sa, sb)
        assert gemm_check(_to_bf16_bits(y), ref, absr, FAST_ACCUM_SUM_COEF)[0]
    # one dominant product per block, +448*448 in the first and -448*448 in the second so they cancel,
    # and 63 products of 1.5 per block that the alignment (quantum 2 at 448*448) truncates to zero
    A = np.full((4, 128), 0x38, np.uint8)     # E4M3 1.0
    B = np.full((3, 128), 0x3C, np.uint8)     # E4M3 1.5
    A[:, ::64] = 0x7E
    B[:, 0] = 0x7E
    B[:, 64] = 0xFE
    B[1, 1::2] |= 0x80                          # mixed signs among the small products
    y = _aligned_block_gemm(A, "e4m3", B, "e4m3", 1.0, 1.0)
    ref = gemm_ref(A, "e4m3", B, "e4m3", 1.0, 1.0)
    absr = gemm_abs_ref(A, "e4m3", B, "e4m3", 1.0, 1.0)
    assert not np.array_equal(y, ref)
    assert gemm_check(_to_bf16_bits(y), ref, absr, FAST_ACCUM_SUM_COEF)[0]
    assert not gemm_check(_to_bf16_bits(y), ref, absr)[0]
    # equal magnitudes within each block: the model is exact
    A = (np.full((5, 192), 0x30, np.uint8) | (rng.integers(0, 2, (5, 192)) << 7).astype(np.uint8))
    B = (np.full((6, 192), 0x48, np.uint8) | (rng.integers(0, 2, (6, 192)) << 7).astype(np.uint8))
    assert np.array_equal(_aligned_block_gemm(A, "e4m3", B, "e4m3", 1.0, 1.0),
                          gemm_ref(A, "e4m3", B, "e4m3", 1.0, 1.0))


def test_fast_accumulation_bound_rejects_wrong_results():
    """Under the looser bound a transposed pairing, a doubled inverse scale and a sign flip still fail."""
    from oracle.gemm import FAST_ACCUM_SUM_COEF
    rng = np.random.default_rng(12)
    K = 256
    A = _finite_codes(rng, (16, K), "e4m3")
    Bs = _finite_codes(rng, (16, K), "e4m3")
    sa, sb = np.float32(1 / 64), np.float32(1 / 32)
    ref = gemm_ref(A, "e4m3", Bs, "e4m3", sa, sb)
    absr = gemm_abs_ref(A, "e4m3", Bs, "e4m3", sa, sb)
    c = FAST_ACCUM_SUM_COEF
    assert gemm_check(_to_bf16_bits(ref), ref, absr, c)[0]
    assert not gemm_check(_to_bf16_bits(ref.T), ref, absr, c)[0]
    assert not gemm_check(_to_bf16_bits(ref * float(sa)), ref, absr, c)[0]
    assert not gemm_check(_to_bf16_bits(-ref), ref, absr, c)[0]
