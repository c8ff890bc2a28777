"""FP8 codec of the oracle: decode from bit fields, saturating round-to-nearest-even encode.

Test infrastructure only (see the package docstring).

Formats ([TE] §TEとFP8混合精度とは and [TRT] §FP8量子化の技術的優位性と背景 give the
bit split; [MPT] §定義, precision table, gives the largest values 448 and
57344 and says E5M2 spans FP16's range):
  E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. Exponent
        field 15 with mantissa 7 is NaN; there is no infinity (OCP "fn").
  E5M2: sign bit 7, exponent bits 6..2 (bias 15), mantissa bits 1..0. Exponent
        field 31 is Inf (mantissa 0) or NaN, as in IEEE binary16.
Exponent field 0 encodes subnormals m * 2**(1 - bias - mantissa_bits).
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class FP8Format:
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    ieee_specials: bool   # True: all-ones exponent is Inf/NaN (E5M2); False: only S.1111.111 is NaN (E4M3)

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal binade."""
        return 1 - self.bias

    def is_nan_fields(self, e: int, m: int) -> bool:
        all_ones = (1 << self.exp_bits) - 1
        if self.ieee_specials:
            return e == all_ones and m != 0
        return e == all_ones and m == (1 << self.man_bits) - 1

    def is_inf_fields(self, e: int, m: int) -> bool:
        return self.ieee_specials and e == (1 << self.exp_bits) - 1 and m == 0

    @property
    def max(self) -> float:
        """Largest finite value, found by scanning the positive codes."""
        return _largest_finite(self)[1]

    @property
    def max_code(self) -> int:
        """Code of the largest finite value."""
        return _largest_finite(self)[0]


@functools.lru_cache(maxsize=None)
def _largest_finite(f: FP8Format):
    best = (0, 0.0)
    for c in range(128):
        v = decode(c, f)
        if math.isfinite(v) and v > best[1]:
            best = (c, v)
    return best


FMT = {
    "e4m3": FP8Format("e4m3", 4, 3, 7, ieee_specials=False),
    "e5m2": FP8Format("e5m2", 5, 2, 15, ieee_specials=True),
}


def _fmt(fmt) -> FP8Format:
    return FMT[fmt] if isinstance(fmt, str) else fmt


def decode(code: int, fmt) -> float:
    """Value of one FP8 code, read field by field (float64; exact)."""
    f = _fmt(fmt)
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> f.man_bits) & ((1 << f.exp_bits) - 1)
    m = code & ((1 << f.man_bits) - 1)
    if f.is_nan_fields(e, m):
        return math.nan
    if f.is_inf_fields(e, m):
        return sign * math.inf
    if e == 0:
        return sign * math.ldexp(m, f.emin - f.man_bits)
    return sign * math.ldexp((1 << f.man_bits) + m, e - f.bias - f.man_bits)


def decode_table(fmt) -> np.ndarray:
    """float64[256]: the value of every code."""
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def encode(v, fmt) -> np.ndarray:
    """Saturating round-to-nearest-even encode of float32 values to FP8 codes (uint8).

    Steps, for a = |v| taken exactly in float64:
      1. NaN -> sign | 0x7F.
      2. a >= largest finite value (Inf included) -> sign | largest finite code.
      3. Otherwise the quantum of a's binade is q = 2**(max(floor(log2 a), emin) - M);
         n = a / q rounded to an integer, ties to even; the result is n * q, which
         is never above the largest finite value because a is below it.
      4. Write the fields of n * q: a carry to n = 2**(M+1) moves up one binade;
         n < 2**M can only happen in the subnormal binade (exponent field 0).
    """
    f = _fmt(fmt)
    v = np.ascontiguousarray(v, dtype=np.float32)
    bits = v.view(np.uint32)
    sign = ((bits >> np.uint32(31)).astype(np.uint8) << np.uint8(7)).astype(np.uint8)
    a = np.abs(v.astype(np.float64))
    fmax = f.max
    out = np.zeros(v.shape, dtype=np.uint8)

    nan = np.isnan(a)
    sat = ~nan & (a >= fmax)
    rest = ~nan & ~sat

    out[nan] = 0x7F
    out[sat] = f.max_code

    ar = a[rest]
    _, e2 = np.frexp(ar)                        # ar = frac * 2**e2, frac in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, f.emin)
    q = np.ldexp(np.ones_like(ar), (e - f.man_bits).astype(np.int32))
    n = np.rint(ar / q)                         # numpy rint: half to even; ar / q is exact
    n = n.astype(np.int64)
    top = 1 << (f.man_bits + 1)
    carry = n == top
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 1 << f.man_bits, n)
    normal = n >= (1 << f.man_bits)
    exp_field = np.where(normal, e + f.bias, 0)
    man_field = np.where(normal, n - (1 << f.man_bits), n)
    out[rest] = ((exp_field << f.man_bits) | man_field).astype(np.uint8)
    return out | sign


def encode_scalar(x: float, fmt) -> int:
    return int(encode(np.array([x], dtype=np.float32), fmt)[0])


def bf16_to_f32(b) -> np.ndarray:
    """BF16 bit patterns (uint16) to float32: the bits become the top half (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
