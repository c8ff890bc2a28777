"""Pins for the oracle's FP8 codec: page constants, textbook formats, libraries, brute force."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.codec import FMT, decode, decode_table, encode
from tests.conftest import read_golden

CODES = np.arange(256, dtype=np.uint8)


def test_format_constants_from_pages():
    """Bit split and largest finite values are the ones the pages print."""
    rows = read_golden("fp8_formats.txt")
    assert {r[0] for r in rows} == {"e4m3", "e5m2"}
    for name, eb, mb, fmax in rows:
        f = FMT[name]
        assert f.exp_bits == int(eb) and f.man_bits == int(mb)
        assert 1 + f.exp_bits + f.man_bits == 8
        assert f.max == float(fmax)
        t = decode_table(name)
        assert np.nanmax(t[np.isfinite(t)]) == float(fmax)
        assert decode(f.max_code, name) == float(fmax)


def test_precision_table_reads_as_epsilon():
    """The table's largest values match the formats; its error column is 2**-mantissa_bits."""
    for name, s, e, m, fmax, rel in read_golden("precision_table.txt"):
        eps = 2.0 ** -int(m)
        assert 0.5 <= eps / float(rel) <= 1.6, name
        if name in FMT:
            assert FMT[name].max == float(fmax)
        elif name == "fp16":
            assert float(np.finfo(np.float16).max) == float(fmax)
        else:
            big = float(np.finfo(np.float32).max) if name == "fp32" else (2 - 2.0 ** -7) * 2.0 ** 127
            assert abs(big - float(fmax)) / big < 0.01


def test_e5m2_is_fp16_top_byte():
    """E5M2 has FP16's exponent, so each code is the binary16 whose top byte it is."""
    h = (CODES.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    t = decode_table("e5m2")
    assert np.array_equal(np.isnan(h), np.isnan(t))
    fin = ~np.isnan(h)
    assert np.array_equal(h[fin], t[fin])
    assert np.array_equal(np.signbit(h[fin]), np.signbit(t[fin]))


def test_e4m3_values_are_fp16_values():
    t = decode_table("e4m3")
    fin = np.isfinite(t)
    assert np.array_equal(t[fin].astype(np.float16).astype(np.float64), t[fin])


@pytest.mark.parametrize("name,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_decode_matches_torch(name, tdt):
    tv = torch.from_numpy(CODES.copy()).view(tdt).to(torch.float64).numpy()
    t = decode_table(name)
    assert np.array_equal(np.isnan(tv), np.isnan(t))
    fin = ~np.isnan(t)
    assert np.array_equal(tv[fin], t[fin])


def test_code_classes_and_order():
    t4, t5 = decode_table("e4m3"), decode_table("e5m2")
    assert np.isnan(t4).sum() == 2 and np.isfinite(t4).sum() == 254 and np.isinf(t4).sum() == 0
    assert np.isnan(t5).sum() == 6 and np.isfinite(t5).sum() == 248 and np.isinf(t5).sum() == 2
    for name, t in (("e4m3", t4), ("e5m2", t5)):
        top = FMT[name].max_code
        pos = t[: top + 1]
        assert np.all(np.diff(pos) > 0)
        assert np.array_equal(t[128: 128 + top + 1], -pos)
        assert math.copysign(1.0, t[128]) == -1.0
    assert t4[1] == 2.0 ** -9 and t4[8] == 2.0 ** -6
    assert t5[1] == 2.0 ** -16 and t5[4] == 2.0 ** -14


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encode_roundtrip_all_codes(name):
    t = decode_table(name)
    fin = np.isfinite(t)
    assert np.array_equal(encode(t[fin].astype(np.float32), name), CODES[fin])


def test_hand_cases():
    for name, val, code, *_ in read_golden("codec_hand_cases.txt"):
        v = np.float32(float(val))
        assert oracle.encode_scalar(v, name) == int(code, 16), (name, val)
    nneg = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)
    assert encode(nneg, "e4m3")[0] == 0xFF and encode(nneg, "e5m2")[0] == 0xFF


def _brute_force(v: np.ndarray, name: str) -> np.ndarray:
    """Nearest finite value by exhaustive search, ties to the even code; sign copied.

    Beyond the largest finite value the nearest finite value is the largest one,
    so saturation needs no rule of its own here (Inf and NaN are excluded).
    """
    t = decode_table(name)
    top = FMT[name].max_code
    vals = t[: top + 1]                               # +0 .. largest, increasing
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.arange(top + 1)[None, :]
    even_pick = np.where(cand & (idx % 2 == 0), idx, 10 ** 6).min(axis=1)
    any_pick = np.where(cand, idx, 10 ** 6).min(axis=1)
    pick = np.where(cand.sum(axis=1) > 1, even_pick, any_pick)
    sign = (v.view(np.uint32) >> 31).astype(np.uint8) << 7
    return pick.astype(np.uint8) | sign


def _probe_values(name, n_random=40000, seed=0):
    rng = np.random.default_rng(seed)
    t = decode_table(name)
    top = FMT[name].max_code
    vals = t[: top + 1]
    mids = (vals[:-1] + vals[1:]) / 2
    pieces = [vals, mids, vals[-1] + np.array([1.0, 8.0, 16.0, 1e3, 1e6]) * (vals[-1] - vals[-2]) / 16]
    m32 = mids.astype(np.float32)
    pieces += [np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))]
    e = rng.uniform(-24 if name == "e4m3" else -34, 20, n_random)
    pieces.append(np.exp2(e))
    bits = rng.integers(0, 2 ** 32, n_random, dtype=np.uint64).astype(np.uint32)
    rb = np.abs(bits.view(np.float32))
    # float64 distances stay exact enough to order the candidates below 2**40
    pieces.append(rb[np.isfinite(rb) & (rb < 2.0 ** 40)])
    v = np.concatenate([np.asarray(p, dtype=np.float32) for p in pieces])
    sgn = np.where(rng.random(v.size) < 0.5, -1, 1).astype(np.float32)
    return (v * sgn).astype(np.float32)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encode_matches_brute_force(name):
    v = _probe_values(name)
    for i in range(0, v.size, 8192):
        c = v[i: i + 8192]
        assert np.array_equal(encode(c, name), _brute_force(c, name))


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encode_far_above_range_exact_nearest(name):
    """Huge finite values: nearest finite code found with exact rational distances."""
    from fractions import Fraction
    rng = np.random.default_rng(7)
    top = FMT[name].max_code
    cands = [Fraction(decode(c, name)) for c in range(top + 1)]
    bits = rng.integers(0x43000000, 0x7F800000, 300, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    got = encode(v, name)
    for x, g in zip(v, got):
        fx = Fraction(float(x))
        d = [abs(fx - c) for c in cands]
        best = min(d)
        picks = [i for i, di in enumerate(d) if di == best]
        want = picks[0] if len(picks) == 1 else [i for i in picks if i % 2 == 0][0]
        assert g == want, (x, g, want)


@pytest.mark.parametrize("name,tdt,limit", [("e4m3", torch.float8_e4m3fn, 464.0),
                                             ("e5m2", torch.float8_e5m2, 61440.0)])
def test_encode_matches_torch_below_overflow(name, tdt, limit):
    """torch's float8 cast rounds to nearest even but does not saturate: compare below its overflow."""
    v = _probe_values(name, seed=1)
    v = v[np.abs(v) < limit]
    tb = torch.from_numpy(v.copy()).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(encode(v, name), tb)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_relative_error_bound(name):
    """In the normal range the rounding error is at most half an epsilon (precision table)."""
    f = FMT[name]
    rng = np.random.default_rng(5)
    v = np.exp2(rng.uniform(f.emin, math.log2(f.max), 100000)).astype(np.float32)
    v = v[v < f.max]
    err = np.abs(decode_table(name)[encode(v, name)] - v.astype(np.float64))
    assert np.all(err <= 2.0 ** -(f.man_bits + 1) * v.astype(np.float64))
    sub = (np.exp2(rng.uniform(-40, f.emin, 10000))).astype(np.float32)
    err = np.abs(decode_table(name)[encode(sub, name)] - sub.astype(np.float64))
    assert np.all(err <= 2.0 ** (f.emin - f.man_bits - 1))


def test_bf16_widening_matches_torch():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f32(b)
    tv = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(mine.view(np.uint32)[~np.isnan(mine)], tv.view(np.uint32)[~np.isnan(tv)])
    assert np.array_equal(np.isnan(mine), np.isnan(tv))
