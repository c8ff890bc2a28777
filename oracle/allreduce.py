"""FP64 reference for the FP8 gradient all-reduce with one shared scale.

Test infrastructure only (see the package docstring).

[MPT] §横断的知見 "テンソルスケーリングが FP8 実用化の鍵": for an FP8 all-reduce every
GPU uses one shared scalar, the smallest of the ranks' scales, s'_g =
min(s'_1, ..., s'_N), so the codes of all ranks mean the same thing and can be
summed. The pages stop there; the readings taken:

  * shared scale: each rank's scale is the delayed-scaling update of its own
    amax history; since that update is a non-increasing function of the
    history's max (a rounded quotient fmax / a, times an exact 2**-margin), the
    smallest scale is the update of the largest amax over all ranks. So one
    MAX all-reduce of the amax slots, followed by the ordinary update on each
    rank, gives every rank s'_g (when every rank's update succeeds; a rank
    that would hold its scale is not covered by the identity);
  * reduction: rank r contributes q_r = enc(g_r * s'_g); the reduced gradient
    is (sum_r dec(q_r)) * (1 / s'_g), the sum taken over the decoded values
    and dequantised once.
"""
from __future__ import annotations

import numpy as np

from .codec import _fmt, bf16_to_f32, decode_table
from .recipe import update_scale


def shared_scale(histories, scales, scale_invs, fmt, margin: int = 0):
    """min over ranks of each rank's updated scale (the reading's definition), with its inverse."""
    outs = [update_scale(np.asarray(h, np.float32), np.float32(s), np.float32(si), fmt, margin)
            for h, s, si in zip(histories, scales, scale_invs)]
    k = int(np.argmin([float(o[0]) for o in outs]))
    return outs[k][0], outs[k][1]


def reduce_ref(q_stack, fmt, scale_inv) -> np.ndarray:
    """(sum_r dec(q_r)) * scale_inv in float64; q_stack is [ranks, ...] codes."""
    d = decode_table(_fmt(fmt))[np.asarray(q_stack, dtype=np.uint8)]
    with np.errstate(invalid="ignore", over="ignore"):
        return d.sum(axis=0) * float(np.float32(scale_inv))


def reduce_bound(q_stack, fmt, scale_inv, out_dtype: str) -> np.ndarray:
    """Tolerance for an FP32 sum in rank order, dequantised once, then rounded to out_dtype.

    The FP32 running sum of N decoded values errs by at most (N - 1) 2**-24
    sum_r |dec(q_r)|; the multiply adds 2**-24 of the result; the output
    rounding adds half a unit of out_dtype (2**-9 relative for BF16, 2**-24
    for FP32). One full unit is allowed for the output rounding, since the
    FP32 error can move a value across a rounding boundary.
    """
    d = decode_table(_fmt(fmt))[np.asarray(q_stack, dtype=np.uint8)]
    n = d.shape[0]
    si = abs(float(np.float32(scale_inv)))
    with np.errstate(invalid="ignore", over="ignore"):
        ref = np.abs(d.sum(axis=0)) * si
        mag = np.abs(d).sum(axis=0) * si
    unit = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -23
    return unit * ref + (n + 1) * 2.0 ** -24 * mag


def reduce_check(out, q_stack, fmt, scale_inv, out_dtype: str):
    """(ok, worst ratio); out is BF16 bits (uint16) or float32 values; NaN must match NaN, Inf must match Inf."""
    y = bf16_to_f32(np.asarray(out, np.uint16)) if out_dtype == "bf16" else np.asarray(out, np.float32)
    y = y.astype(np.float64)
    ref = reduce_ref(q_stack, fmt, scale_inv)
    b = reduce_bound(q_stack, fmt, scale_inv, out_dtype)
    same_special = np.array_equal(np.isnan(y), np.isnan(ref)) and np.array_equal(np.isinf(y), np.isinf(ref))
    fin = np.isfinite(ref)
    if fin.any():
        # an FP32 sum that overflows where the exact one does not is outside the method's range
        if not np.isfinite(y[fin]).all():
            return False, float("inf")
        ratio = np.abs(y[fin] - ref[fin]) / np.maximum(b[fin], 1e-300)
        worst = float(ratio.max())
    else:
        worst = 0.0
    return same_special and worst <= 1.0, worst
