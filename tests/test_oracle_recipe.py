"""Pins for the oracle's amax, scaled cast and delayed-scaling recipe.

Each check rests on something other than the oracle's own formula: exact
rational arithmetic, powers of two, properties the pages state for the recipe
knobs (margin trades overflow for underflow, a longer history is more stable),
or invariants of a sliding-window maximum.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.codec import FMT, decode_table
from oracle.recipe import CANONICAL_NAN, DelayedScaling, amax, cast, max_nan, primed_scale

F32 = np.float32


def bits(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def nearest_f32(r: Fraction) -> np.float32:
    """Round a positive rational to binary32, ties to even, using exact comparisons."""
    c = np.float32(float(r))              # within one binary32 ulp of r (float() rounds once)
    best = None
    for cand in (np.nextafter(c, F32(0)), c, np.nextafter(c, F32(np.inf))):
        d = abs(Fraction(float(cand)) - r)
        if best is None or d < best[0] or (d == best[0] and bits(cand) % 2 == 0):
            best = (d, cand)
    return best[1]


def test_amax_values():
    assert amax(np.array([-3.0, 2.0, 1.0], F32)) == F32(3.0)
    z = amax(np.array([-0.0, -0.0], F32))
    assert bits(z) == 0
    assert bits(amax(np.array([1.0, np.nan, -np.inf], F32))) == 0x7FC00000
    neg_nan = np.array([0xFFFFFFFF], np.uint32).view(np.float32)
    assert bits(amax(np.concatenate([np.ones(3, F32), neg_nan]))) == 0x7FC00000
    assert amax(np.array([1.0, -np.inf], F32)) == F32(np.inf)
    # bf16 storage: 0xC0A0 is -5.0, 0x4040 is 3.0
    assert amax(np.array([0xC0A0, 0x4040], np.uint16), "bf16") == F32(5.0)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_scale_for_power_of_two_amax(name):
    """fmax / 2**k is exact, so s and s_inv are known in closed form."""
    fmax = FMT[name].max
    for k in range(-30, 31, 3):
        r = primed_scale(np.array([2.0 ** k, -0.5 * 2.0 ** k], F32), name, "f32", 16)
        assert float(r.scale) == fmax * 2.0 ** -k
        assert r.scale_inv == nearest_f32(Fraction(1) / Fraction(float(r.scale)))


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_scale_is_correctly_rounded_quotient(name):
    rng = np.random.default_rng(3)
    fmax = Fraction(FMT[name].max)
    for a in np.exp2(rng.uniform(-40, 40, 300)).astype(F32):
        r = primed_scale(np.array([a], F32), name, "f32", 4)
        want = nearest_f32(fmax / Fraction(float(a)))
        assert r.scale == want
        assert r.scale_inv == nearest_f32(1 / Fraction(float(want)))


def test_margin_is_an_exact_power_of_two():
    x = np.random.default_rng(0).standard_normal(4096).astype(F32)
    s0 = primed_scale(x, "e4m3", "f32", 8, margin=0).scale
    for m in range(0, 12):
        sm = primed_scale(x, "e4m3", "f32", 8, margin=m).scale
        assert float(sm) == float(s0) * 2.0 ** -m


def test_margin_trades_overflow_for_underflow():
    """A larger margin gives fewer saturated codes and more zero codes (recipe section of the TE guide)."""
    rng = np.random.default_rng(1)
    prime = rng.standard_normal(1 << 14).astype(F32)
    nxt = (prime * F32(3.0)).astype(F32)                 # next step's range has grown
    nxt[:64] *= F32(1e-9)                                # and some tiny entries
    sat, zero = [], []
    for m in range(0, 8):
        rec = primed_scale(prime, "e4m3", "f32", 16, margin=m)
        q = rec.cast_step(nxt, "f32")
        sat.append(int(np.sum((q & 0x7F) == 0x7E)))
        zero.append(int(np.sum((q & 0x7F) == 0)))
    assert sat[0] > 0
    assert all(a >= b for a, b in zip(sat, sat[1:]))
    assert all(a <= b for a, b in zip(zero, zero[1:]))
    assert zero[-1] > zero[0]


def _amax_run(amaxes, L, fmt="e4m3", margin=0):
    rec = DelayedScaling(fmt, L, margin)
    scales = []
    for a in amaxes:
        rec.record(F32(a))
        rec.update()
        scales.append(float(rec.scale))
    return np.array(scales)


def test_history_window_spike_rolls_out_after_L_updates():
    L = 5
    seq = [1.0] * 3 + [100.0] + [1.0] * 12
    s = _amax_run(seq, L)
    assert s[2] == 448.0
    # the spike governs the scale for exactly L updates, then the window forgets it
    assert all(s[3 + i] == float(F32(448.0) / F32(100.0)) for i in range(L))
    assert s[3 + L] == 448.0


def test_longer_history_is_more_stable():
    """scale(L1) <= scale(L2) for L1 >= L2, and the step-to-step variation shrinks with L."""
    rng = np.random.default_rng(4)
    seq = np.exp(rng.normal(0, 0.7, 200)).astype(F32)
    runs = {L: _amax_run(seq, L) for L in (1, 2, 4, 16, 64)}
    Ls = sorted(runs)
    for lo, hi in zip(Ls, Ls[1:]):
        assert np.all(runs[hi] <= runs[lo])
    tv = [np.abs(np.diff(np.log(runs[L]))).sum() for L in Ls]
    assert all(a >= b for a, b in zip(tv, tv[1:]))


def test_window_max_matches_brute_force():
    """After step t the scale comes from the max of the last L amaxes."""
    rng = np.random.default_rng(8)
    seq = np.exp(rng.normal(0, 1.0, 60)).astype(F32)
    for L in (1, 3, 7):
        s = _amax_run(seq, L)
        for t in range(len(seq)):
            window = seq[max(0, t - L + 1): t + 1]
            assert s[t] == nearest_f32(Fraction(448) / Fraction(float(max(window))))


def test_delayed_cast_uses_previous_scale():
    rng = np.random.default_rng(2)
    xs = [rng.standard_normal(512).astype(F32) * F32(u) for u in (1.0, 4.0, 0.25, 2.0)]
    rec = DelayedScaling("e4m3", 16, 0)
    assert rec.scale == 1.0 and rec.scale_inv == 1.0 and not rec.history.any()
    prev_scale = rec.scale
    for x in xs:
        q = rec.cast_step(x, "f32")
        # the codes are those of x times the scale in force before this step
        assert np.array_equal(q, cast(x, prev_scale, "e4m3"))
        assert rec.history[0] == np.abs(x).max()
        rec.update()
        prev_scale = rec.scale


def test_scaled_amax_element_hits_the_top_code():
    rng = np.random.default_rng(6)
    for name in ("e4m3", "e5m2"):
        x = (rng.standard_normal(2048) * 7).astype(F32)
        rec = primed_scale(x, name, "f32", 16)
        q = rec.cast_step(x, "f32")
        top = FMT[name].max_code
        i = int(np.argmax(np.abs(x)))
        assert (q[i] & 0x7F) == top
        assert np.all((q & 0x7F) <= top)
        # dequantised values reproduce x to within FP8's half-epsilon
        dq = decode_table(name)[q] * float(rec.scale_inv)
        eps = 2.0 ** -(FMT[name].man_bits + 1)
        normal = np.abs(x) * float(rec.scale) >= 2.0 ** FMT[name].emin
        assert np.all(np.abs(dq - x)[normal] <= 1.01 * eps * np.abs(x)[normal])


def test_hold_rules():
    rec = primed_scale(np.array([2.0], F32), "e4m3", "f32", 3)
    s, si = rec.scale, rec.scale_inv
    assert s == 224.0
    # all-zero steps: max(history) is still 2 for L-1 more updates, then 0 -> scale held
    for _ in range(5):
        rec.record(F32(0.0))
        rec.update()
        assert rec.scale == s and rec.scale_inv == si
    # NaN amax holds the scale until it rolls out of the window
    rec.record(CANONICAL_NAN)
    for t in range(3):
        rec.update()
        assert rec.scale == s
        rec.record(F32(4.0))
    rec.update()
    assert rec.scale == 112.0
    # Inf amax: not finite -> held
    rec2 = primed_scale(np.array([np.inf, 1.0], F32), "e4m3", "f32", 2)
    assert rec2.scale == 1.0 and rec2.scale_inv == 1.0
    # a subnormal amax makes fmax / amax overflow -> held
    rec3 = primed_scale(np.array([1e-45], F32), "e4m3", "f32", 2)
    assert rec3.scale == 1.0
    # a margin that underflows the scale to zero -> held
    rec4 = primed_scale(np.array([1e30], F32), "e4m3", "f32", 2, margin=200)
    assert rec4.scale == 1.0
    # a subnormal scale whose inverse overflows binary32 cannot dequantise -> held
    rec5 = primed_scale(np.array([1.0], F32), "e4m3", "f32", 2, margin=140)
    assert rec5.scale == 1.0 and rec5.scale_inv == 1.0
    # a tiny but normal scale is accepted, with its exact power-of-two inverse
    rec6 = primed_scale(np.array([7.0], F32), "e4m3", "f32", 2, margin=100)
    assert float(rec6.scale) == 64.0 * 2.0 ** -100 and float(rec6.scale_inv) == 2.0 ** 94


def test_history_roll_and_state_round_trip():
    rng = np.random.default_rng(9)
    steps = [rng.standard_normal(256).astype(F32) * F32(u) for u in rng.uniform(0.5, 2, 16)]
    full = DelayedScaling("e4m3", 4, 0)
    out_full = []
    for x in steps:
        out_full.append(full.cast_step(x))
        full.update()
    a = DelayedScaling("e4m3", 4, 0)
    out = []
    for x in steps[:8]:
        out.append(a.cast_step(x))
        a.update()
    saved = a.state()
    b = DelayedScaling("e4m3", 4, 0)
    b.load_state(*saved)
    for x in steps[8:]:
        out.append(b.cast_step(x))
        b.update()
    assert all(np.array_equal(p, q) for p, q in zip(out, out_full))
    assert np.array_equal(b.history.view(np.uint32), full.history.view(np.uint32))
    assert b.scale == full.scale and b.scale_inv == full.scale_inv


def test_max_nan():
    assert max_nan([]) == 0.0
    assert bits(max_nan([np.float32(1), CANONICAL_NAN])) == 0x7FC00000
    assert max_nan([F32(-1), F32(2)]) == 2.0


def test_nan_product_sign_rule():
    """A NaN product's code carries sign(x) xor sign(s); Inf * 0 and NaN scales included."""
    neg_nan = np.array([0xFFC00000], np.uint32).view(np.float32)[0]
    x = np.array([np.nan, neg_nan, np.inf, -np.inf, 1.0, -2.0], F32)
    q = cast(x, F32(0.0), "e4m3")
    assert q.tolist() == [0x7F, 0xFF, 0x7F, 0xFF, 0x00, 0x80]
    q = cast(x, F32(-0.0), "e5m2")
    assert q.tolist() == [0xFF, 0x7F, 0xFF, 0x7F, 0x80, 0x00]
    q = cast(x, F32(np.nan), "e4m3")
    assert q.tolist() == [0x7F, 0xFF, 0x7F, 0xFF, 0x7F, 0xFF]
    q = cast(x, F32(-2.0), "e4m3")
    assert q.tolist() == [0xFF, 0x7F, 0xFE, 0x7E, 0xC0, 0x48]
