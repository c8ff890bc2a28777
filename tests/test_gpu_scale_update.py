"""GPU parity of fp8_scale_update against the oracle: scale, scale_inv and history bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from oracle.recipe import CANONICAL_NAN, update_scale
from tests.gpu_util import banner, dev, f32, f32_bits, host, require_gpu

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu

F32 = np.float32


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _one(hist, fmt, margin, scale=1.0, scale_inv=1.0):
    h = dev(np.asarray(hist, np.float32))
    s, si = f32(scale), f32(scale_inv)
    fp8.fp8_scale_update(h, fmt, margin, s, si)
    want_s, want_si, want_h = update_scale(np.asarray(hist, np.float32), F32(scale), F32(scale_inv), fmt, margin)
    got_h = host(h)
    assert f32_bits(s)[0] == _bits(want_s), (float(host(s)[0]), float(want_s))
    assert f32_bits(si)[0] == _bits(want_si), (float(host(si)[0]), float(want_si))
    assert np.array_equal(_bits(got_h), _bits(want_h))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("L", [1, 2, 5, 16, 255, 256, 257, 1024, 1500, 8192, 8193, 10000])
def test_random_histories(fmt, L):
    require_gpu()
    rng = np.random.default_rng(L)
    for margin in (0, 1, 3):
        hist = np.exp2(rng.uniform(-30, 30, L)).astype(F32)
        banner("scale-update", fmt, L, margin)
        _one(hist, fmt, margin, scale=2.5, scale_inv=0.4)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quotients_over_many_amaxes(fmt):
    """Correct rounding of fmax / a and 1 / s over many single-entry histories."""
    require_gpu()
    rng = np.random.default_rng(99)
    bits = rng.integers(0x00800000, 0x7F800000, 2000, dtype=np.uint64).astype(np.uint32)
    for a in bits.view(np.float32)[:400]:
        _one([a], fmt, 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_hold_rules(fmt):
    require_gpu()
    cases = [
        ("all-zero", [0.0] * 8, 0),
        ("nan", [1.0, float(CANONICAL_NAN), 2.0], 0),
        ("inf", [np.inf, 1.0], 0),
        ("subnormal-amax", [1e-45, 0.0], 0),
        ("margin-underflow", [1e30], 200),
        ("margin-subnormal-scale", [1.0], 140),          # inverse overflows -> held
        ("margin-subnormal-ok", [448.0 if fmt == "e4m3" else 57344.0], 127),   # s = 2^-127, 1/s finite
        ("huge-margin", [3.0], 2 ** 31 - 1),
        ("tiny-normal-scale", [7.0], 100),
    ]
    for name, hist, margin in cases:
        banner("hold", fmt, name)
        _one(np.array(hist, F32), fmt, margin, scale=3.0, scale_inv=F32(1) / F32(3))


def test_sixteen_step_recipe_and_resume():
    """A cast+update loop on the GPU equals the oracle's, and survives a state round trip."""
    require_gpu()
    import workloads as wl
    w = wl.BY_NAME["tiny_fwd_256"]
    x = wl.load(w.name)["X"]
    xs = wl.tiny_step_inputs(x, wl.step_factors(w.config_id, w.steps))
    ref = oracle.DelayedScaling("e4m3", w.history_len, 0)
    st = fp8.DelayedScalingState("e4m3", w.history_len, 0)
    q = torch.empty(256, 256, dtype=torch.uint8, device="cuda")
    for t, xt in enumerate(xs):
        banner("recipe-step", t)
        if t == 8:     # checkpoint, reset, restore
            sd = {k: v.cpu() for k, v in st.state_dict().items()}
            st = fp8.DelayedScalingState("e4m3", w.history_len, 0)
            st.load_state_dict({k: v.cuda() for k, v in sd.items()})
        st.cast(dev(xt), q)
        want = ref.cast_step(xt, "f32")
        assert np.array_equal(host(q), want)
        st.update()
        ref.update()
        assert np.array_equal(_bits(host(st.history)), _bits(ref.history))
        assert f32_bits(st.scale)[0] == _bits(ref.scale) and f32_bits(st.scale_inv)[0] == _bits(ref.scale_inv)


def test_batched_update_equals_oracle_per_tensor():
    """20 tensors (two launches of up to 16) with mixed formats, lengths, margins and hold cases."""
    require_gpu()
    from oracle.adam import update_fp16_scale
    rng = np.random.default_rng(123)
    fmts = ["e4m3", "e5m2", "fp16"]
    cases = []
    for t in range(20):
        L = int(rng.choice([1, 3, 256, 1024, 8192, 8193, 10000]))
        fmt = fmts[t % 3]
        margin = int(rng.integers(0, 4))
        hist = np.exp2(rng.uniform(-30, 30, L)).astype(F32)
        if t == 5:
            hist[:] = 0                       # held
        if t == 7:
            hist[L // 2] = CANONICAL_NAN      # held while the NaN is in the window
        cases.append((fmt, margin, hist, F32(rng.uniform(0.5, 4)), None))

    class St:
        pass
    states = []
    for fmt, margin, hist, s0, _ in cases:
        st = St()
        st.history, st.fmt, st.margin = dev(hist), fp8.FORMATS[fmt], margin
        st.scale, st.scale_inv = f32(s0), f32(F32(1) / s0)
        states.append(st)
    banner("batched-update", len(states))
    fp8.fp8_scale_update_batched(states)
    for (fmt, margin, hist, s0, _), st in zip(cases, states):
        si0 = F32(1) / s0
        if fmt == "fp16":
            ws, wsi, wh = update_fp16_scale(hist, s0, si0, margin)
        else:
            ws, wsi, wh = update_scale(hist, s0, si0, fmt, margin)
        assert f32_bits(st.scale)[0] == _bits(ws) and f32_bits(st.scale_inv)[0] == _bits(wsi), (fmt, margin, hist.size)
        assert np.array_equal(_bits(host(st.history)), _bits(wh))
