"""amax, scaled cast and the delayed-scaling recipe of the oracle.

Test infrastructure only (see the package docstring).

[TE] §TEとFP8混合精度とは: each tensor's value range is watched and its scaling
factor is adjusted so the values fit FP8's range. [TE] §動的スケーリングとFP8レシピの設定:
the default recipe is DelayedScaling with margin (default 0; larger means fewer
overflows and more underflows), fp8_format (HYBRID = E4M3 forward, E5M2
backward) and amax_history_len (default 1024; the length of the history the
scale is computed from). [MPT] §横断的知見 "テンソルスケーリングが FP8 実用化の鍵"
names delayed and just-in-time per-tensor scaling. The scale formula
s = fmax / max(history) / 2**margin and the round-to-nearest-even saturating
cast are the readings listed in the package docstring.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .codec import _fmt, bf16_to_f32, encode

CANONICAL_NAN = np.array([0x7FC00000], dtype=np.uint32).view(np.float32)[0]


def _as_f32(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(x)
    raise ValueError(dtype)


def max_nan(values) -> np.float32:
    """Largest of float32 values, NaN if any is NaN (returned as the canonical NaN)."""
    v = np.asarray(values, dtype=np.float32).ravel()
    if v.size == 0:
        return np.float32(0.0)
    if np.isnan(v).any():
        return CANONICAL_NAN
    return np.float32(v.max())


def amax(x, dtype: str = "f32") -> np.float32:
    """a = max |x| over the whole tensor, in float32 (exact); -0 counts as 0."""
    return max_nan(np.abs(_as_f32(x, dtype)))


def cast(x, scale, fmt, dtype: str = "f32") -> np.ndarray:
    """q = enc(fp32(x) * s): one binary32 multiply (round to nearest even), then one FP8 rounding.

    IEEE 754 leaves the sign of a NaN result open; it is read here as the sign
    the product would have, sign(x) xor sign(s), so a NaN product's code is
    0x7F with that sign.
    """
    xf = _as_f32(x, dtype)
    s = np.float32(scale)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = xf * s                    # numpy float32 multiply: IEEE binary32, RNE, no flushing
    q = encode(prod, fmt)
    nan = np.isnan(prod)
    if nan.any():
        sx = (np.ascontiguousarray(xf).view(np.uint32) >> np.uint32(31)).astype(np.uint8)
        ss = np.uint8(int(np.array([s], np.float32).view(np.uint32)[0]) >> 31)
        q[nan] = np.uint8(0x7F) | ((sx[nan] ^ ss) << np.uint8(7))
    return q


def update_scale(history: np.ndarray, scale: np.float32, scale_inv: np.float32,
                 fmt, margin: int):
    """One delayed-scaling update for an FP8 format (see update_scale_fmax)."""
    return update_scale_fmax(history, scale, scale_inv, _fmt(fmt).max, margin)


def update_scale_fmax(history: np.ndarray, scale: np.float32, scale_inv: np.float32,
                      fmax: float, margin: int):
    """One delayed-scaling update towards a format whose largest value is fmax.
    Returns (scale, scale_inv, rolled history).

    a_max = max over every history entry (NaN propagates). If a_max is finite
    and positive, s' = fp32(fp32(fmax / a_max) * 2**-margin), and if s' and
    fp32(1 / s') are both finite and positive they become scale and scale_inv.
    In every other case the previous scale and scale_inv are kept. Then the
    history rolls by one: entry i takes entry i-1's value and entry 0 becomes 0,
    ready to receive the next step's amax.
    """
    h = np.asarray(history, dtype=np.float32).copy()
    a_max = max_nan(h)
    new_scale, new_inv = np.float32(scale), np.float32(scale_inv)
    if math.isfinite(float(a_max)) and a_max > 0:
        with np.errstate(over="ignore"):
            ratio = np.float32(fmax) / a_max                   # binary32 division, correctly rounded
            s = np.float32(math.ldexp(float(ratio), -int(margin)))  # exact power-of-two step, one rounding
            inv = np.float32(1.0) / s if s > 0 else np.float32(np.inf)
        # a scale is usable only if it and its inverse are finite and positive
        if math.isfinite(float(s)) and s > 0 and math.isfinite(float(inv)):
            new_scale = s
            new_inv = inv
    h[1:] = h[:-1].copy()
    h[0] = np.float32(0.0)
    return new_scale, new_inv, h


class DelayedScaling:
    """Per-tensor recipe state: history[L], scale, scale_inv (cold start: 0, 1, 1)."""

    def __init__(self, fmt, history_len: int = 1024, margin: int = 0):
        if history_len < 1 or margin < 0:
            raise ValueError("history_len >= 1 and margin >= 0 required")
        self.fmt = _fmt(fmt)
        self.margin = int(margin)
        self.history = np.zeros(history_len, dtype=np.float32)
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)

    def record(self, a) -> None:
        """Fold this step's amax into the newest history entry."""
        self.history[0] = max_nan([self.history[0], a])

    def cast_step(self, x, dtype: str = "f32", record: bool = True) -> np.ndarray:
        """Cast with the current (previous step's) scale and record this tensor's amax."""
        q = cast(x, self.scale, self.fmt, dtype)
        if record:
            self.record(amax(x, dtype))
        return q

    def update(self) -> None:
        self.scale, self.scale_inv, self.history = update_scale(
            self.history, self.scale, self.scale_inv, self.fmt, self.margin)

    def state(self):
        return self.history.copy(), np.float32(self.scale), np.float32(self.scale_inv)

    def load_state(self, history, scale, scale_inv) -> None:
        self.history = np.asarray(history, dtype=np.float32).copy()
        self.scale = np.float32(scale)
        self.scale_inv = np.float32(scale_inv)


def transpose_codes(q: np.ndarray) -> np.ndarray:
    """The transposed copy of a code matrix (a pure relayout)."""
    return np.ascontiguousarray(np.asarray(q).T)


def nan_bits_equal(a, b) -> bool:
    """Bitwise equality of float32 arrays (NaNs must match bit for bit)."""
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


def primed_scale(x, fmt, dtype: str, history_len: int = 1024, margin: int = 0,
                 rec: Optional[DelayedScaling] = None) -> DelayedScaling:
    """Single-shot workloads: one amax-only priming step, then one update.

    The returned recipe holds s = fp32(fmax / amax(x)) * 2**-margin (when that is
    finite and positive), ready for the checked fused amax+cast step.
    """
    rec = rec or DelayedScaling(fmt, history_len, margin)
    rec.record(amax(x, dtype))
    rec.update()
    return rec
