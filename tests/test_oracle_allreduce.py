"""Pins of the shared-scale all-reduce oracle: the min-scale / max-amax identity, exact integer
sums of the decoded codes, the single-rank case, and the bound's rejection of plausible mistakes."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.codec import FMT


def _rand_hist(rng, n_ranks, L):
    return [np.exp2(rng.uniform(-20, 20, L)).astype(np.float32) for _ in range(n_ranks)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("margin", [0, 3])
def test_min_of_rank_scales_is_update_of_max_amax(fmt, margin):
    rng = np.random.default_rng(margin + (fmt == "e5m2"))
    for _ in range(200):
        hs = _rand_hist(rng, int(rng.integers(2, 9)), int(rng.integers(1, 17)))
        s, si = oracle.shared_scale(hs, [1.0] * len(hs), [1.0] * len(hs), fmt, margin)
        top = max(float(h.max()) for h in hs)
        s2, si2, _ = oracle.update_scale(np.array([top], np.float32), np.float32(1), np.float32(1), fmt, margin)
        assert np.float32(s).view(np.uint32) == np.float32(s2).view(np.uint32)
        assert np.float32(si).view(np.uint32) == np.float32(si2).view(np.uint32)
        # and it is the smallest rank scale, by the rational definition of each rank's quotient
        fmax = Fraction(float(oracle.decode_table(fmt)[FMT[fmt].max_code]))
        exact = [fmax / Fraction(float(h.max())) / 2 ** margin for h in hs]
        assert Fraction(float(s)) <= min(exact) * (1 + Fraction(1, 2 ** 23))


def test_hand_example_two_ranks():
    """E4M3 codes 0x38 = 1.0, 0x40 = 2.0, 0xB8 = -1.0: ranks [1, 2] and [2, -1] sum to [3, 1]; scale_inv 0.5."""
    q = np.array([[0x38, 0x40], [0x40, 0xB8]], np.uint8)
    assert np.array_equal(oracle.reduce_ref(q, "e4m3", 0.5), [1.5, 0.5])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_sum_matches_exact_integer_arithmetic(fmt):
    """Every finite code is an integer multiple of the smallest subnormal (2**-9 / 2**-16)."""
    rng = np.random.default_rng(4)
    top = FMT[fmt].max_code
    q = (rng.integers(0, top + 1, (7, 300)) | (rng.integers(0, 2, (7, 300)) << 7)).astype(np.uint8)
    unit = 2 ** (9 if fmt == "e4m3" else 16)
    tab = oracle.decode_table(fmt)
    ints = np.array([[int(Fraction(float(tab[c])) * unit) for c in row] for row in q], dtype=object)
    want = [Fraction(int(s), unit) * Fraction(float(np.float32(0.25))) for s in ints.sum(axis=0)]
    got = oracle.reduce_ref(q, fmt, 0.25)
    assert all(Fraction(float(g)) == w for g, w in zip(got, want))


def test_single_rank_is_the_dequantised_code():
    q = np.arange(256, dtype=np.uint8)[None, :]
    got = oracle.reduce_ref(q, "e5m2", 3.0)
    want = oracle.decode_table("e5m2") * 3.0
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)])


def test_bound_accepts_fp32_rank_order_and_rejects_mistakes():
    rng = np.random.default_rng(9)
    top = FMT["e5m2"].max_code
    q = (rng.integers(top - 40, top + 1, (8, 4000)) | (rng.integers(0, 2, (8, 4000)) << 7)).astype(np.uint8)
    tab = oracle.decode_table("e5m2").astype(np.float32)
    si = np.float32(1 / 3)
    acc = np.zeros(4000, np.float32)
    for r in range(8):
        acc = (acc + tab[q[r]]).astype(np.float32)
    from workloads import f32_to_bf16_bits
    good = f32_to_bf16_bits((acc * si).astype(np.float32))
    assert oracle.reduce_check(good, q, "e5m2", si, "bf16")[0]
    assert oracle.reduce_check((acc * si).astype(np.float32), q, "e5m2", si, "f32")[0]
    wrong = {
        "a rank dropped": sum(tab[q[r]] for r in range(7)) * si,
        "scale instead of inverse": acc * np.float32(3.0),
        "mean instead of sum": acc * si / 8,
        "sign of one rank flipped": (acc - 2 * tab[q[3]]) * si,
    }
    for name, v in wrong.items():
        assert not oracle.reduce_check(f32_to_bf16_bits(np.asarray(v, np.float32)), q, "e5m2", si, "bf16")[0], name
