"""GPU parity of the shared-scale FP8 all-reduce pieces on one GPU.

fp8_reduce_shared_scale against the oracle's FP64 sum of decoded codes within
its bound (exactly, for every code on one rank); the shared scale obtained by
a MAX of the ranks' amax slots followed by fp8_scale_update against the
oracle's minimum of the ranks' own updates, bit for bit; and the whole chain
(shared scale, cast of each rank's gradient, reduction).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle.codec import FMT
from tests.gpu_util import banner, dev, f32, first_diff, host, require_gpu

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu


def _bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


def _reduce(q, fmt, si, out_dtype, stride_pad=0):
    n, numel = q.shape
    qs = torch.zeros(n, numel + stride_pad, dtype=torch.uint8, device="cuda")
    qs[:, :numel] = dev(q)
    out = torch.empty(numel, dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device="cuda")
    fp8.fp8_reduce_shared_scale(qs[:, :numel], fmt, f32(si), out)
    o = host(out.view(torch.int16)) if out_dtype == "bf16" else host(out)
    return o


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_code_on_one_rank_is_exact(fmt):
    require_gpu()
    q = np.tile(np.arange(256, dtype=np.uint8), 9)[None, :]         # 2304 codes: vector path plus a tail
    for out_dtype in ("f32", "bf16"):
        banner("reduce-codes", fmt, out_dtype)
        o = _reduce(q, fmt, 1.0, out_dtype)
        got = oracle.bf16_to_f32(o) if out_dtype == "bf16" else o
        want = oracle.decode_table(fmt)[q[0]].astype(np.float32)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        fin = ~np.isnan(want)
        assert np.array_equal(_bits(got[fin]), _bits(want[fin])), first_diff(_bits(got[fin]), _bits(want[fin]))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("n_ranks", [1, 2, 3, 8])
def test_reduce_shapes(fmt, n_ranks):
    require_gpu()
    rng = np.random.default_rng(n_ranks * 10 + (fmt == "e5m2"))
    top = FMT[fmt].max_code
    for numel in (1, 15, 16, 17, 4101, 100000):
        q = (rng.integers(0, top + 1, (n_ranks, numel)) | (rng.integers(0, 2, (n_ranks, numel)) << 7)).astype(np.uint8)
        for out_dtype, pad, si in (("bf16", 0, 0.37), ("f32", 16, 1.0 / 3), ("bf16", 3, 2.0 ** -10), ("f32", 5, 7.0)):
            banner("reduce", fmt, n_ranks, numel, out_dtype, pad)
            o = _reduce(q, fmt, si, out_dtype, pad)
            ok, worst = oracle.reduce_check(o, q, fmt, si, out_dtype)
            assert ok, (numel, out_dtype, pad, worst)


def test_reduce_special_codes():
    require_gpu()
    q = np.zeros((3, 64), np.uint8)
    q[0, 0] = 0x7F            # E5M2 NaN
    q[0, 1], q[1, 1] = 0x7C, 0x7C      # +Inf + +Inf
    q[0, 2], q[2, 2] = 0x7C, 0xFC      # +Inf + -Inf = NaN
    q[1, 3] = 0x7B            # largest finite
    for out_dtype in ("bf16", "f32"):
        banner("reduce-special", out_dtype)
        o = _reduce(q, "e5m2", 1.0, out_dtype)
        ok, worst = oracle.reduce_check(o, q, "e5m2", 1.0, out_dtype)
        assert ok, worst


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_shared_scale_is_min_of_rank_scales(fmt):
    """Over T steps, every rank records its own amax, the slots are MAX-reduced across ranks (simulated on one
    GPU), and each rank runs fp8_scale_update: after every step every rank holds the smallest of the scales the
    ranks would have computed from their own histories (the oracle's delayed recipe per rank)."""
    require_gpu()
    rng = np.random.default_rng(5 + (fmt == "e5m2"))
    for trial in range(6):
        n, L, T = int(rng.integers(2, 9)), int(rng.integers(1, 9)), 12
        amaxes = np.exp2(rng.uniform(-20, 20, (T, n))).astype(np.float32)
        refs = [oracle.DelayedScaling(fmt, L, 1) for _ in range(n)]
        hist = [torch.zeros(L, dtype=torch.float32, device="cuda") for _ in range(n)]
        sc = [(f32(1.0), f32(1.0)) for _ in range(n)]
        for t in range(T):
            for r in range(n):
                refs[r].record(amaxes[t, r])
                refs[r].update()
                hist[r][0] = float(amaxes[t, r])
            top = torch.stack([h[0] for h in hist]).amax()      # stands in for the RCCL MAX all-reduce
            for h in hist:
                h[0] = top
            banner("shared-scale", fmt, trial, n, L, t)
            want = min(refs, key=lambda d: float(d.scale))
            for r in range(n):
                fp8.fp8_scale_update(hist[r], fmt, 1, sc[r][0], sc[r][1])
                assert _bits(host(sc[r][0]))[0] == _bits(want.scale), (t, r)
                assert _bits(host(sc[r][1]))[0] == _bits(want.scale_inv), (t, r)


def test_shared_scale_gradient_chain():
    """Each of 4 ranks casts its BF16 gradient with the shared scale (E5M2); the reduction of the codes
    matches the oracle's sum of its own codes, and those codes are bit-identical to the GPU's."""
    require_gpu()
    n, shape = 4, (256, 384)
    grads = [wl.small_normal(40 + r, shape, std=1e-3, dist="student_t3") for r in range(n)]
    hists = [np.array([oracle.amax(g, "bf16")], np.float32) for g in grads]
    s, si = oracle.shared_scale(hists, [1.0] * n, [1.0] * n, "e5m2", 0)
    codes = np.stack([oracle.cast(g, s, "e5m2", "bf16") for g in grads])
    q = torch.empty(n, shape[0] * shape[1], dtype=torch.uint8, device="cuda")
    ds = f32(s)
    for r in range(n):
        banner("chain-cast", r)
        fp8.fp8_amax_cast(dev(grads[r]), "e5m2", ds, q[r].view(shape), None, None)
    assert np.array_equal(host(q), codes.reshape(n, -1)), "shared-scale casts differ"
    out = torch.empty(shape[0] * shape[1], dtype=torch.float32, device="cuda")
    banner("chain-reduce")
    fp8.fp8_reduce_shared_scale(q, "e5m2", f32(si), out)
    ok, worst = oracle.reduce_check(host(out), codes.reshape(n, -1), "e5m2", si, "f32")
    assert ok, worst
    # and the reduced gradient is close to the exact sum of the BF16 gradients (FP8 quantisation error only)
    gf = [oracle.bf16_to_f32(g).astype(np.float64).ravel() for g in grads]
    exact = sum(gf)
    err = np.abs(host(out) - exact)
    assert np.all(err <= n * 2.0 ** -3 * max(np.abs(x).max() for x in gf))


def test_reduce_full_size_wgrad():
    """8 ranks of the 7B up-projection's weight gradient (11008 x 4096, E5M2) into BF16, sampled check."""
    require_gpu()
    n, numel = 8, 11008 * 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(123)
    q = torch.randint(0, 256, (n, numel), dtype=torch.uint8, device="cuda", generator=g)
    q[(q & 0x7F) >= 0x7C] = 0x3C        # finite codes only
    out = torch.empty(numel, dtype=torch.bfloat16, device="cuda")
    banner("reduce-full", n, numel)
    fp8.fp8_reduce_shared_scale(q, "e5m2", f32(2.0 ** -12), out)
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([[0, numel - 1], rng.choice(numel, 4000, replace=False)]))
    ti = torch.from_numpy(idx).cuda()
    qs = host(q[:, ti])
    ok, worst = oracle.reduce_check(host(out.view(torch.int16)[ti]), qs, "e5m2", 2.0 ** -12, "bf16")
    assert ok, worst
