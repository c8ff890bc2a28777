"""FP64 reference for LayerNorm followed by the amax and FP8 cast of its output.

Test infrastructure only (see the package docstring).

[TE] §基本的なFP8トレーニングコードの構成: besides the linear layer, the LayerNorm module
is swapped for its FP8-aware counterpart, which hands the following linear
layer its input. The pages name the layer but not its formula; the textbook
LayerNorm over the last (contiguous) dimension is taken, in the order the
definition states it:

    mu_i      = (1/n) sum_j x_ij
    var_i     = (1/n) sum_j (x_ij - mu_i)**2          (biased: divides by n)
    rstd_i    = 1 / sqrt(var_i + eps)                  (eps inside the root)
    y_ij      = (x_ij - mu_i) * rstd_i * gamma_j + beta_j

The GPU result is the BF16 rounding of an FP32 evaluation, so it is compared
within `layer_norm_bound`; the amax and codes of that BF16 output are then
compared bit for bit with `recipe.amax` and `recipe.cast` applied to it.
"""
from __future__ import annotations

import numpy as np

from .codec import bf16_to_f32


def _rows_f64(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def layer_norm_ref(x, gamma, beta, eps, dtype: str = "bf16"):
    """(y, mu, rstd) in float64; gamma and beta are fp32 vectors (beta may be None)."""
    xf = _rows_f64(x, dtype)
    n = xf.shape[1]
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    b = np.zeros(n) if beta is None else np.asarray(beta, dtype=np.float32).astype(np.float64)
    mu = xf.sum(axis=1) / n
    d = xf - mu[:, None]
    var = (d * d).sum(axis=1) / n
    with np.errstate(divide="ignore", invalid="ignore"):
        rstd = 1.0 / np.sqrt(var + float(np.float32(eps)))
        y = d * rstd[:, None] * g[None, :] + b[None, :]
    return y, mu, rstd


def layer_norm_bound(x, gamma, beta, eps, dtype: str = "bf16") -> np.ndarray:
    """Elementwise tolerance for a BF16 output of an FP32 evaluation.

    2**-8 |y_ref| is one BF16 unit in the last place: the final rounding
    (half a unit) plus a rounding decision the FP32 error can flip. The second
    term bounds the FP32 evaluation: each row sum is formed from n terms in at
    most n/64 + 8 sequential steps (per-lane runs, then a tree), so the mean
    and the variance carry a relative error of at most c_n = (n/64 + 8) 2**-24
    of the sums of magnitudes that form them; the three final operations add a
    few more units. Eight c_n, applied to every magnitude that enters y_ij,
    covers both.
    """
    xf = _rows_f64(x, dtype)
    n = xf.shape[1]
    y, mu, rstd = layer_norm_ref(x, gamma, beta, eps, dtype)
    g = np.abs(np.asarray(gamma, dtype=np.float32).astype(np.float64))
    b = np.zeros(n) if beta is None else np.abs(np.asarray(beta, dtype=np.float32).astype(np.float64))
    c_n = (n / 64.0 + 8.0) * 2.0 ** -24
    spread = np.abs(xf - mu[:, None]).mean(axis=1) + np.abs(mu)       # per row
    mag = g[None, :] * rstd[:, None] * (np.abs(xf - mu[:, None]) + spread[:, None]) + b[None, :]
    return 2.0 ** -8 * np.abs(y) + 8.0 * c_n * mag


def layer_norm_check(y_bits, x, gamma, beta, eps, dtype: str = "bf16"):
    """(ok, worst ratio) for BF16 output bits against the reference; NaN must match NaN."""
    y = bf16_to_f32(np.asarray(y_bits, dtype=np.uint16)).astype(np.float64)
    ref, _, _ = layer_norm_ref(x, gamma, beta, eps, dtype)
    bound = layer_norm_bound(x, gamma, beta, eps, dtype)
    nan_ok = np.array_equal(np.isnan(y), np.isnan(ref))
    fin = np.isfinite(ref)
    with np.errstate(invalid="ignore"):
        ratio = np.abs(y[fin] - ref[fin]) / np.maximum(bound[fin], 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    return nan_ok and worst <= 1.0, worst
