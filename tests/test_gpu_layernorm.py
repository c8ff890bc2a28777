"""GPU parity of fp8_layernorm_amax_cast.

The BF16 output is compared with the oracle's FP64 LayerNorm within
`layer_norm_bound`; the amax and codes of that BF16 output are compared bit for
bit with the oracle's amax and cast of it (the call's definition). Register
and generic paths, ragged and long rows, strided layouts, fp32 sources, no
BF16 output, NaN rows and zero/infinite scales.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import banner, dev, f32, first_diff, host, require_gpu

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu


def _bits(v):
    return np.array([v], np.float32).view(np.uint32)[0]


def _inputs(seed, rows, cols, offset=3.0):
    x = wl.small_normal(seed, (rows, cols), std=1.5, outlier_factor=20.0)
    xf = oracle.bf16_to_f32(x) + np.float32(offset)          # a row mean to remove
    x = wl.f32_to_bf16_bits(xf)
    rng = np.random.default_rng(seed)
    g = rng.normal(1.0, 0.2, cols).astype(np.float32)
    b = rng.normal(0.0, 0.2, cols).astype(np.float32)
    return x, g, b


def _run(x, g, b, eps, fmt, s, ld_pad=(0, 0, 0), dtype="bf16", want_y=True, amax0=0.0):
    rows, cols = x.shape
    if dtype == "bf16":
        xs = torch.zeros(rows, cols + ld_pad[0], dtype=torch.int16, device="cuda")
        xs[:, :cols] = dev(x)
    else:
        xs = torch.zeros(rows, cols + ld_pad[0], dtype=torch.float32, device="cuda")
        xs[:, :cols] = dev(oracle.bf16_to_f32(x))
    xt = xs[:, :cols]
    ys = torch.full((rows, cols + ld_pad[1]), 0x1234, dtype=torch.int16, device="cuda")
    qs = torch.full((rows, cols + ld_pad[2]), 0x5A, dtype=torch.uint8, device="cuda")
    am = f32(amax0)
    mu = torch.empty(rows, dtype=torch.float32, device="cuda")
    rs = torch.empty(rows, dtype=torch.float32, device="cuda")
    fp8.fp8_layernorm_amax_cast(xt, dev(g), None if b is None else dev(b), eps, fmt,
                                ys[:, :cols] if want_y else None, f32(s), qs[:, :cols], am, mu, rs)
    yh, qh = host(ys), host(qs)
    if ld_pad[1]:
        assert (yh[:, cols:] == 0x1234).all(), "wrote past cols in y"
    if ld_pad[2]:
        assert (qh[:, cols:] == 0x5A).all(), "wrote past cols in q"
    return yh[:, :cols], qh[:, :cols], host(am)[0], host(mu), host(rs)


def _check(x, g, b, eps, fmt, s, y, q, am, mu, rs, amax0=0.0):
    ok, worst = oracle.layer_norm_check(y, x, g, b, eps)
    assert ok, f"LayerNorm output: worst |err|/bound = {worst}"
    want_q = oracle.cast(y, np.float32(s), fmt, "bf16")
    assert np.array_equal(q, want_q), first_diff(q, want_q)
    want_a = oracle.max_nan([np.float32(amax0), oracle.amax(y, "bf16")])
    assert _bits(am) == _bits(want_a), (am, want_a)
    _, mu_ref, rs_ref = oracle.layer_norm_ref(x, g, b, eps)
    n = x.shape[1]
    c_n = (n / 64 + 8) * 2.0 ** -24
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    fin = np.isfinite(mu_ref)
    assert np.all(np.abs(mu[fin] - mu_ref[fin]) <= 8 * c_n * np.abs(xf[fin]).mean(axis=1) + 1e-30)
    fin = np.isfinite(rs_ref)
    assert np.all(np.abs(rs[fin] - rs_ref[fin]) <= 16 * c_n * rs_ref[fin] * (1 + np.abs(mu_ref[fin]) * rs_ref[fin]))


SHAPES = [(1, 8), (4, 8), (37, 16), (64, 520), (129, 4096), (33, 5120), (16, 8192), (8, 16384),
          (5, 100), (7, 20000), (3, 1)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", SHAPES)
def test_layernorm_shapes(fmt, shape):
    require_gpu()
    rows, cols = shape
    x, g, b = _inputs(rows * 7 + cols, rows, cols)
    for eps, beta, s in ((1e-5, b, 4.0), (0.0, None, 100.0), (0.5, b, 1e-3)):
        banner("layernorm", fmt, shape, eps, beta is None, s)
        res = _run(x, g, beta, eps, fmt, s)
        _check(x, g, beta, eps, fmt, s, *res)


@pytest.mark.parametrize("cols", [2056, 3072, 4096, 4104, 6144, 8192, 16384])
def test_layernorm_output_modes_agree(cols):
    """BF16 only, codes only and both: each width and mode picks its own launch shape; y is the same
    bits in every mode and matches the oracle, the codes and amax are the oracle's cast of that y."""
    require_gpu()
    rows = 24
    x, g, b = _inputs(cols + 1, rows, cols)
    s, fmt = 8.0, "e4m3"
    banner("layernorm modes", rows, cols)
    y_both, q_both, am_both, mu, rs = _run(x, g, b, 1e-5, fmt, s)
    _check(x, g, b, 1e-5, fmt, s, y_both, q_both, am_both, mu, rs)
    y_only = torch.full((rows, cols), 0x1234, dtype=torch.int16, device="cuda")
    fp8.fp8_layernorm_amax_cast(dev(x), dev(g), dev(b), 1e-5, fmt, y_only)
    assert np.array_equal(host(y_only), y_both), first_diff(host(y_only), y_both)
    q_only = torch.full((rows, cols), 0x5A, dtype=torch.uint8, device="cuda")
    am = f32(0.0)
    fp8.fp8_layernorm_amax_cast(dev(x), dev(g), dev(b), 1e-5, fmt, None, f32(s), q_only, am)
    assert np.array_equal(host(q_only), q_both), first_diff(host(q_only), q_both)
    assert _bits(host(am)[0]) == _bits(am_both)


def test_layernorm_layouts_and_sources():
    """Strided rows (register path), odd strides (generic path), fp32 sources, no BF16 output."""
    require_gpu()
    rows, cols = 48, 1024
    x, g, b = _inputs(5, rows, cols)
    base = None
    for pads, dtype in (((0, 0, 0), "bf16"), ((8, 8, 8), "bf16"), ((3, 5, 5), "bf16"), ((0, 0, 0), "f32"),
                        ((5, 0, 3), "f32")):
        banner("layernorm-layout", pads, dtype)
        res = _run(x, g, b, 1e-5, "e4m3", 2.0, pads, dtype)
        _check(x, g, b, 1e-5, "e4m3", 2.0, *res)
        if pads == (0, 0, 0) and dtype == "bf16":
            base = res
    banner("layernorm-no-y")
    _, q, am, _, _ = _run(x, g, b, 1e-5, "e4m3", 2.0, want_y=False)
    assert np.array_equal(q, base[1]) and _bits(am) == _bits(base[2])


def test_layernorm_amax_accumulates_and_special_values():
    require_gpu()
    rows, cols = 16, 256
    x, g, b = _inputs(9, rows, cols)
    xf = oracle.bf16_to_f32(x)
    xf[3, 10] = np.nan                     # a NaN row
    xf[7, :] = 2.5                         # a constant row: y = beta exactly
    x = wl.f32_to_bf16_bits(xf)
    for s in (1.0, -1.0, 0.0, float("inf")):
        banner("layernorm-special", s)
        res = _run(x, g, b, 1e-5, "e4m3", s)
        _check(x, g, b, 1e-5, "e4m3", s, *res)
        y = res[0]
        assert np.isnan(oracle.bf16_to_f32(y[3])).all()
        assert np.array_equal(oracle.bf16_to_f32(y[7]), oracle.bf16_to_f32(wl.f32_to_bf16_bits(b)))
    x2, g2, b2 = _inputs(10, 8, 64)
    banner("layernorm-amax-prior")
    res = _run(x2, g2, b2, 1e-5, "e5m2", 1.0, amax0=1e4)
    _check(x2, g2, b2, 1e-5, "e5m2", 1.0, *res, amax0=1e4)


def test_layernorm_full_size_activation():
    """The 7B MLP input shape (4096 x 4096): amax over all of y exactly, y and codes on sampled rows."""
    require_gpu()
    inp = wl.load("mlp7b_up_fwd")["X"]
    rows, cols = inp.shape
    rng = np.random.default_rng(77)
    g = rng.normal(1.0, 0.2, cols).astype(np.float32)
    b = rng.normal(0.0, 0.2, cols).astype(np.float32)
    y = torch.empty(rows, cols, dtype=torch.int16, device="cuda")
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    am = f32(0.0)
    banner("layernorm-full", rows, cols)
    fp8.fp8_layernorm_amax_cast(dev(inp), dev(g), dev(b), 1e-5, "e4m3", y, f32(3.0), q, am)
    yh = host(y)
    assert _bits(host(am)[0]) == _bits(oracle.amax(yh, "bf16"))
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 62, replace=False)]))
    ok, worst = oracle.layer_norm_check(yh[sel], inp[sel], g, b, 1e-5)
    assert ok, worst
    qh = host(q[torch.from_numpy(sel).cuda()])
    want = oracle.cast(yh[sel], np.float32(3.0), "e4m3", "bf16")
    assert np.array_equal(qh, want), first_diff(qh, want)


def test_layer_plan_with_layernorm_operand():
    """A layer step whose X operand is LayerNorm(X): its codes and recorded amax are those of the LayerNorm
    output (taken from a separate call that also writes y), under the delayed scale; W takes the plain cast."""
    require_gpu()
    from fp8_mixed_precision_cast_amd.linear import GemmOp, LayerPlan, OperandSpec
    x, g, b = _inputs(31, 256, 512)
    w = wl.small_normal(32, (384, 512), std=0.02)
    inp = {"X": dev(x), "W": dev(w)}
    dg, db = dev(g), dev(b)
    plan = LayerPlan([OperandSpec("X", (256, 512), "e4m3", layernorm=True), OperandSpec("W", (384, 512), "e4m3")],
                     [GemmOp("fwd", "X", False, "W", False)], history_len=4, ln_params={"X": (dg, db, 1e-5)})
    banner("plan-layernorm", "prime")
    plan.prime(inp)
    y = torch.empty(256, 512, dtype=torch.int16, device="cuda")
    fp8.fp8_layernorm_amax_cast(inp["X"], dg, db, 1e-5, "e4m3", y)
    yh = host(y)
    for step in range(2):
        st = plan.state["X"]
        s_before = host(st.scale)[0]
        banner("plan-layernorm", step)
        plan.cast_all(inp)
        want = oracle.cast(yh, s_before, "e4m3", "bf16")
        got = host(plan.q["X"])
        assert np.array_equal(got, want), first_diff(got, want)
        assert _bits(host(st.history)[0]) == _bits(oracle.amax(yh, "bf16"))
        plan.gemm_all()
        plan.update_all()
    assert _bits(host(plan.state["X"].scale)[0]) == _bits(np.float32(448.0) / oracle.amax(yh, "bf16"))
