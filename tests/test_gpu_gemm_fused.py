"""GPU parity of fp8_scaled_gemm_amax_cast.

Its BF16 output must be the plain GEMM's, bit for bit, and within the GEMM
bound of the oracle's FP64 product; its amax and FP8 copy must equal, bit for
bit, the oracle's amax and cast applied to that BF16 output (the definition of
the fused call), across ragged shapes, both output formats, code outputs with
wider row pitches, saturating and underflowing scales and NaN outputs. A code
output whose start or row pitch is not a multiple of 16 bytes is refused.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.codec import FMT
from tests.gpu_util import banner, dev, f32, first_diff, host, pitched, require_gpu

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu


def _codes(rng, shape, fmt, spread=40):
    top = FMT[fmt].max_code
    c = rng.integers(max(0, top - spread), top + 1, shape, dtype=np.int64)
    sign = rng.integers(0, 2, shape, dtype=np.int64) << 7
    return (c | sign).astype(np.uint8)


def _bits(v):
    return np.array([v], np.float32).view(np.uint32)[0]


def _fused(a, af, b, bf, sa, sb, yf, ys, amax0=0.0, ldq_pad=0, want_q=True, want_amax=True):
    """ldq_pad: extra bytes (a multiple of 16) in the row pitch of y_q beyond n rounded up to 16."""
    m, n = a.shape[0], b.shape[0]
    da, db = dev(a), dev(b)
    c_plain, _ = pitched(m, n, torch.int16, fill=0)
    fp8.fp8_scaled_gemm(da, af, db, bf, f32(sa), f32(sb), c_plain)
    c, _ = pitched(m, n, torch.int16, fill=0)
    q, q_store = pitched(m, n, torch.uint8, fill=0x5A, pad_bytes=ldq_pad)
    q = q if want_q else None
    am = f32(amax0) if want_amax else None
    fp8.fp8_scaled_gemm_amax_cast(da, af, db, bf, f32(sa), f32(sb), c, yf, f32(ys) if want_q else None, q, am)
    cb = host(c)
    assert np.array_equal(cb, host(c_plain)), "fused C differs from the plain GEMM: " + first_diff(cb, host(c_plain))
    if want_q:
        qs = host(q_store)
        want = oracle.cast(cb, np.float32(ys), yf, "bf16")
        assert np.array_equal(qs[:, :n], want), first_diff(qs[:, :n], want)
        assert (qs[:, n:] == 0x5A).all(), "wrote past n in y_q"
    if want_amax:
        want_a = oracle.max_nan([np.float32(amax0), oracle.amax(cb, "bf16")])
        assert _bits(host(am)[0]) == _bits(want_a), (host(am)[0], want_a)
    return cb


SHAPES = [(256, 256, 128), (300, 200, 272), (257, 129, 16), (1, 1, 16), (17, 300, 48), (640, 384, 1024)]


@pytest.mark.parametrize("yf", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", SHAPES)
def test_fused_amax_cast_shapes(yf, shape):
    require_gpu()
    m, n, k = shape
    rng = np.random.default_rng(m * 13 + n * 5 + k + (yf == "e5m2"))
    for af, bf in (("e4m3", "e4m3"), ("e5m2", "e4m3")):
        a, b = _codes(rng, (m, k), af), _codes(rng, (n, k), bf)
        sa, sb = np.float32(0.75), np.float32(3.0)
        c = None
        for ys, pad in ((1.0, 0), (37.5, 16), (1e6, 32), (1e-30, 16)):  # plain, wider pitch, saturating, underflow
            banner("fused", af, bf, yf, shape, ys, pad)
            c = _fused(a, af, b, bf, sa, sb, yf, ys, amax0=0.0, ldq_pad=pad)
        ref = oracle.gemm_ref(a, af, b, bf, sa, sb)
        ok, worst = oracle.gemm_check(c, ref, oracle.gemm_abs_ref(a, af, b, bf, sa, sb))
        assert ok, worst


def test_fused_outputs_one_at_a_time_and_amax_accumulates():
    require_gpu()
    rng = np.random.default_rng(7)
    a, b = _codes(rng, (300, 256), "e4m3"), _codes(rng, (520, 256), "e4m3")
    banner("fused", "amax-only")
    c = _fused(a, "e4m3", b, "e4m3", 1.0, 1.0, "e4m3", 2.0, amax0=0.0, want_q=False)
    big = float(oracle.amax(c, "bf16")) * 4
    banner("fused", "amax keeps a larger prior value")
    _fused(a, "e4m3", b, "e4m3", 1.0, 1.0, "e4m3", 2.0, amax0=big, want_q=False)
    banner("fused", "codes-only")
    _fused(a, "e4m3", b, "e4m3", 1.0, 1.0, "e5m2", 0.5, want_amax=False)
    banner("fused", "neither: the plain GEMM")
    _fused(a, "e4m3", b, "e4m3", 1.0, 1.0, "e5m2", 0.5, want_q=False, want_amax=False)


def test_fused_nan_outputs():
    """A NaN code in A makes its output row NaN: the amax is the canonical NaN, the codes follow the sign rule;
    zero and infinite output scales make NaN products out of infinite and zero outputs."""
    require_gpu()
    rng = np.random.default_rng(11)
    a, b = _codes(rng, (64, 128), "e4m3"), _codes(rng, (96, 128), "e4m3")
    a[5, 17] = 0x7F
    a[40, 3] = 0xFF
    a[7, :] = 0                       # a zero output row: 0 * Inf is NaN under an infinite scale
    for ys in (1.0, -1.0, 0.0, float("inf"), float("-inf")):
        banner("fused-nan", ys)
        c = _fused(a, "e4m3", b, "e4m3", 1.0, 1.0, "e4m3", ys)
        assert np.isnan(oracle.gemm.bf16_bits_to_f64(c[5])).all()


def test_fused_full_size_mlp_shape():
    """The 7B MLP up-projection shape: amax over all of C exactly, codes on sampled rows, C on sampled blocks."""
    require_gpu()
    rng = np.random.default_rng(2024)
    m, n, k = 4096, 11008, 4096
    a, b = _codes(rng, (m, k), "e4m3", spread=60), _codes(rng, (n, k), "e4m3", spread=60)
    sa, sb = np.float32(1 / 64), np.float32(1 / 96)
    ys = np.float32(0.37)
    da, db = dev(a), dev(b)
    c = torch.empty(m, n, dtype=torch.int16, device="cuda")
    q = torch.empty(m, n, dtype=torch.uint8, device="cuda")
    am = f32(0.0)
    banner("fused-full", m, n, k)
    fp8.fp8_scaled_gemm_amax_cast(da, "e4m3", db, "e4m3", f32(sa), f32(sb), c, "e4m3", f32(ys), q, am)
    cb = host(c)
    assert _bits(host(am)[0]) == _bits(oracle.amax(cb, "bf16"))
    rows = np.unique(np.concatenate([[0, 255, 256, m - 1], rng.choice(m, 60, replace=False)]))
    qs = host(q[torch.from_numpy(rows).cuda()])
    want = oracle.cast(cb[rows], ys, "e4m3", "bf16")
    assert np.array_equal(qs, want), first_diff(qs, want)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 62, replace=False)]))
    ref = oracle.gemm_ref(a[rows], "e4m3", b[cols], "e4m3", sa, sb)
    absr = oracle.gemm_abs_ref(a[rows], "e4m3", b[cols], "e4m3", sa, sb)
    ok, worst = oracle.gemm_check(cb[rows][:, cols], ref, absr)
    assert ok, worst


@pytest.mark.parametrize("accum", ["exact", "fast"])
def test_layer_plan_output_cast_fused_equals_separate(accum):
    """A chained layer step: the fused output cast, the separate second pass and the fused cast without
    the BF16 output give the same codes, histories and scales, and the codes are the oracle's cast of
    the BF16 output with the delayed scale; under either GEMM accumulation."""
    require_gpu()
    from fp8_mixed_precision_cast_amd.linear import GemmOp, LayerPlan, OperandSpec
    import workloads as wl
    x = wl.small_normal(3, (300, 256), std=1.0, outlier_factor=20.0)
    w = wl.small_normal(4, (520, 256), std=0.02)
    inp = {"X": dev(x), "W": dev(w)}
    ops = [OperandSpec("X", (300, 256), "e4m3"), OperandSpec("W", (520, 256), "e4m3")]
    gem = [GemmOp("fwd", "X", False, "W", False)]
    plans = {mode: LayerPlan(ops, gem, history_len=8, output_cast=mode, gemm_accum=accum)
             for mode in ("fused", "separate", "fused_codes")}
    plans["fused_codes"].out["fwd"].view(torch.int16).fill_(0x1234)   # never stored in that mode
    for mode, plan in plans.items():
        banner("plan-output-cast", mode)
        plan.prime(inp)
    for step in range(3):
        for mode, plan in plans.items():
            ys = plan.ystate["fwd"]
            s_before = host(ys.scale)[0]
            banner("plan-output-cast", accum, mode, step)
            plan.step(inp)
            if mode == "fused_codes":
                assert (host(plan.out["fwd"].view(torch.int16)) == 0x1234).all(), "BF16 output stored"
                continue
            cb = host(plan.out["fwd"].view(torch.int16))
            want = oracle.cast(cb, s_before, "e4m3", "bf16")
            got = host(plan.yq["fwd"])
            assert np.array_equal(got, want), (mode, step, first_diff(got, want))
        f = plans["fused"]
        for other in ("separate", "fused_codes"):
            s = plans[other]
            assert np.array_equal(host(f.yq["fwd"]), host(s.yq["fwd"])), other
            for attr in ("history", "scale", "scale_inv"):
                a = host(getattr(f.ystate["fwd"], attr)).view(np.uint32)
                b = host(getattr(s.ystate["fwd"], attr)).view(np.uint32)
                assert np.array_equal(a, b), (other, attr)


def test_fused_without_bf16_output():
    """c = NULL: the codes and the amax are still those of the (unstored) BF16 output."""
    require_gpu()
    rng = np.random.default_rng(21)
    for m, n, k in ((512, 768, 256), (300, 200, 64)):
        a, b = _codes(rng, (m, k), "e4m3"), _codes(rng, (n, k), "e5m2")
        banner("fused-no-c", m, n, k)
        cb = _fused(a, "e4m3", b, "e5m2", 0.5, 2.0, "e4m3", 3.0)      # reference run with c
        q, _ = pitched(m, n, torch.uint8)
        am = f32(0.0)
        fp8.fp8_scaled_gemm_amax_cast(dev(a), "e4m3", dev(b), "e5m2", f32(0.5), f32(2.0), None, "e4m3", f32(3.0), q, am)
        want = oracle.cast(cb, np.float32(3.0), "e4m3", "bf16")
        assert np.array_equal(host(q), want), first_diff(host(q), want)
        assert _bits(host(am)[0]) == _bits(oracle.amax(cb, "bf16"))


def test_fused_refuses_misaligned_code_outputs():
    require_gpu()
    a = torch.zeros(32, 64, dtype=torch.uint8, device="cuda")
    c = torch.zeros(32, 32, dtype=torch.int16, device="cuda")
    store = torch.full((32, 64), 0x5A, dtype=torch.uint8, device="cuda")
    for name, yq in (("offset by 8 bytes", store[:, 8:40]), ("pitch of 40 bytes", store[:, :40].contiguous()[:, :32])):
        with pytest.raises(fp8.Fp8mpError) as ei:
            fp8.fp8_scaled_gemm_amax_cast(a, "e4m3", a, "e4m3", f32(1.0), f32(1.0), c, "e4m3", f32(1.0), yq, None)
        assert ei.value.status == 1, name
    assert (host(store) == 0x5A).all()


# The FP32-accumulation GEMM with the fused cast walks several tiles per workgroup here (more tiles than CUs),
# storing each tile's BF16 output and codes while the next one runs; one shape switches to narrow tiles for
# its last round. The amax is folded over all of a workgroup's tiles before it is committed.
WALK_SHAPES = [(4100, 4100, 256), (8192, 8448, 144)]


@pytest.mark.parametrize("shape", WALK_SHAPES)
def test_fused_on_workgroups_walking_several_tiles(shape):
    require_gpu()
    m, n, k = shape
    rng = np.random.default_rng(m + 7 * n + 3 * k)
    a, b = _codes(rng, (m, k), "e4m3"), _codes(rng, (n, k), "e5m2")
    for yf, ys, pad in (("e4m3", 1.0, 0), ("e5m2", 1e6, 16)):
        banner("fused walk", shape, yf, ys)
        _fused(a, "e4m3", b, "e5m2", 0.5, 1 / 3.0, yf, ys, amax0=0.0, ldq_pad=pad)
