"""GPU parity of fp8_adam_step against the oracle's binary32 step, bit for bit.

Codes of the first moment, FP16 bits of the second moment and of the scaled
master weights, both amaxes and the dequantisation factors written for the
next step; vector and scalar paths, BF16 and FP32 gradients, saturation, NaN,
and a multi-step run of the AdamFP8State recipe against the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import banner, dev, f32, first_diff, host, require_gpu
from workloads import f32_to_bf16_bits

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _state(rng, n, g_dtype):
    g32 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g = f32_to_bf16_bits(g32) if g_dtype == "bf16" else g32
    m_q = oracle.cast((rng.standard_normal(n) * 1e-3).astype(np.float32), np.float32(2.0 ** 14), "e4m3")
    v = oracle.f16_encode(np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32))
    w = oracle.f16_encode((rng.standard_normal(n) * 0.02 * 1024).astype(np.float32))
    return g, m_q, v, w


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01, step=7)


def _ref_hp(hp):
    """The oracle takes the bias corrections of the step; the library forms them from the step number."""
    c1, c2 = oracle.bias_corrections(hp["beta1"], hp["beta2"], hp["step"])
    return {**{k: v for k, v in hp.items() if k != "step"}, "c1": c1, "c2": c2}


def _gpu_step(g, g_dtype, m_q, v, w, m_dq, m_scale, w_dq, w_scale, hp, offset=0):
    n = m_q.size

    def place(a, dtype):
        t = torch.zeros(n + offset, dtype=dtype, device="cuda")
        t[offset:] = dev(a).view(dtype) if a.dtype != np.float32 else dev(a)
        return t[offset:]
    dg = place(g, torch.int16 if g_dtype == "bf16" else torch.float32)
    dm, dv, dw = place(m_q, torch.uint8), place(v, torch.int16), place(w, torch.int16)
    scal = {k: f32(x) for k, x in dict(mdi=m_dq, ms=m_scale, msi=np.float32(1) / np.float32(m_scale), wdi=w_dq,
                                       ws=w_scale, wsi=np.float32(1) / np.float32(w_scale)).items()}
    mdo, wdo, ma, wa = f32(-1.0), f32(-1.0), f32(0.0), f32(0.0)
    fp8.fp8_adam_step(dg, dm, scal["mdi"], mdo, scal["ms"], scal["msi"], ma, dv, dw, scal["wdi"], wdo, scal["ws"],
                      scal["wsi"], wa, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"], hp["step"])
    return (host(dm), host(dv), host(dw), host(ma)[0], host(wa)[0], host(mdo)[0], host(wdo)[0],
            host(scal["msi"])[0], host(scal["wsi"])[0])


def _compare(ref, got):
    m_q, v, w, ma, wa = ref
    gm, gv, gw, gma, gwa, mdo, wdo, msi, wsi = got
    assert np.array_equal(gm, m_q), "m codes: " + first_diff(gm, m_q)
    assert np.array_equal(gv, v), "v bits: " + first_diff(gv, v)
    assert np.array_equal(gw, w), "w bits: " + first_diff(gw, w)
    assert _bits(gma) == _bits(ma) and _bits(gwa) == _bits(wa)
    assert _bits(mdo) == _bits(msi) and _bits(wdo) == _bits(wsi)


@pytest.mark.parametrize("g_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 4099, 100000])
def test_adam_step_bit_exact(g_dtype, n):
    require_gpu()
    rng = np.random.default_rng(n + (g_dtype == "f32"))
    g, m_q, v, w = _state(rng, n, g_dtype)
    for offset, (m_scale, w_scale) in ((0, (2.0 ** 14, 1024.0)), (1, (3000.0, 777.0)), (0, (1e6, 5e6))):
        m_dq, w_dq = np.float32(2.0 ** -14), np.float32(1 / 1024)
        banner("adam", g_dtype, n, offset, m_scale, w_scale)
        ref = oracle.adam_step_ref(g, g_dtype, m_q, m_dq, m_scale, v, w, w_dq, w_scale, **_ref_hp(HP))
        got = _gpu_step(g, g_dtype, m_q, v, w, m_dq, m_scale, w_dq, w_scale, HP, offset)
        _compare(ref, got)


def test_adam_special_values():
    """NaN and infinite gradients, saturation of both stores, zero state."""
    require_gpu()
    rng = np.random.default_rng(3)
    n = 64
    g, m_q, v, w = _state(rng, n, "f32")
    g[3], g[4], g[5] = np.nan, np.inf, -np.inf
    m_q[10:14] = 0
    v[10:14] = 0
    ref = oracle.adam_step_ref(g, "f32", m_q, 2.0 ** -14, 2.0 ** 14, v, w, 1 / 1024, 1e9, **_ref_hp(HP))
    banner("adam-special")
    got = _gpu_step(g, "f32", m_q, v, w, np.float32(2.0 ** -14), 2.0 ** 14, np.float32(1 / 1024), 1e9, HP)
    gm, gv, gw = got[0], got[1], got[2]
    fin = np.ones(n, bool)
    fin[3:6] = False
    assert np.array_equal(gm, ref[0])                           # codes carry the NaN sign rule
    assert np.array_equal(gv[fin], ref[1][fin]) and np.array_equal(gw[fin], ref[2][fin])
    assert np.isnan(oracle.f16_decode(gv[3:6])).all() == np.isnan(oracle.f16_decode(ref[1][3:6])).all()
    assert (gw[fin] & 0x7FFF).max() == 0x7BFF                   # saturated at 65504 by the huge scale
    assert _bits(got[3]) == _bits(ref[3]) and _bits(got[4]) == _bits(ref[4])   # NaN amaxes are canonical


def _gpu_step_wq(g, g_dtype, m_q, v, w, m_dq, m_scale, w_dq, w_scale, hp, fmt, wq_scale, offset=0, codes=True):
    """fp8_adam_step_weight_cast; the codes buffer sits `offset` bytes past an aligned start."""
    n = m_q.size
    dg = dev(g).view(torch.int16) if g_dtype == "bf16" else dev(g)
    dm, dv, dw = dev(m_q), dev(v).view(torch.int16), dev(w).view(torch.int16)
    scal = {k: f32(x) for k, x in dict(mdi=m_dq, ms=m_scale, msi=np.float32(1) / np.float32(m_scale), wdi=w_dq,
                                       ws=w_scale, wsi=np.float32(1) / np.float32(w_scale), qs=wq_scale).items()}
    mdo, wdo, ma, wa, qa = f32(-1.0), f32(-1.0), f32(0.0), f32(0.0), f32(0.0)
    wq = None
    if codes:
        buf = torch.full((n + offset + 1,), 0x5A, dtype=torch.uint8, device="cuda")
        wq = buf[offset:offset + n]
    fp8.fp8_adam_step(dg, dm, scal["mdi"], mdo, scal["ms"], scal["msi"], ma, dv, dw, scal["wdi"], wdo, scal["ws"],
                      scal["wsi"], wa, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"], hp["step"],
                      wq=wq, wq_fmt=fmt, wq_scale=scal["qs"], wq_amax=qa)
    if codes:
        hb = host(buf)
        assert (hb[:offset] == 0x5A).all() and hb[offset + n] == 0x5A, "wrote outside the codes"
    got = (host(dm), host(dv), host(dw), host(ma)[0], host(wa)[0], host(mdo)[0], host(wdo)[0],
           host(scal["msi"])[0], host(scal["wsi"])[0])
    return got, (host(wq) if codes else None), host(qa)[0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("n", [1, 9, 4099, 100000])
def test_adam_weight_codes_bit_exact(fmt, n):
    """The fused step's every other output is the plain step's; the codes and amax are the oracle's cast of
    the master weights as this step stored them."""
    require_gpu()
    rng = np.random.default_rng(100 + n)
    g, m_q, v, w = _state(rng, n, "bf16")
    m_dq, w_dq = np.float32(2.0 ** -14), np.float32(1 / 1024)
    for offset, w_scale, q_scale in ((0, 1024.0, 448.0 / 0.08), (3, 777.0, 60.0), (0, 1024.0, 1e9)):
        banner("adam-wq", fmt, n, offset, w_scale, q_scale)
        ref = oracle.adam_step_ref(g, "bf16", m_q, m_dq, 2.0 ** 14, v, w, w_dq, w_scale, **_ref_hp(HP))
        got, wq, qa = _gpu_step_wq(g, "bf16", m_q, v, w, m_dq, 2.0 ** 14, w_dq, w_scale, HP, fmt, q_scale, offset)
        _compare(ref, got)
        want_q, want_a = oracle.adam_weight_codes_ref(got[2], got[8], q_scale, fmt)
        assert np.array_equal(wq, want_q), "weight codes: " + first_diff(wq, want_q)
        assert _bits(qa) == _bits(oracle.max_nan([np.float32(0), want_a]))
    got, wq, qa = _gpu_step_wq(g, "bf16", m_q, v, w, m_dq, 2.0 ** 14, w_dq, 1024.0, HP, fmt, 1.0, codes=False)
    _compare(oracle.adam_step_ref(g, "bf16", m_q, m_dq, 2.0 ** 14, v, w, w_dq, 1024.0, **_ref_hp(HP)), got)
    assert _bits(qa) == _bits(oracle.max_nan([np.float32(0), oracle.adam_weight_codes_ref(got[2], got[8], 1.0,
                                                                                          fmt)[1]]))


def test_adam_fp8_state_recipe_over_steps():
    """AdamFP8State for 12 steps against the oracle's step plus delayed updates (E4M3 for m, FP16 for w),
    with the next forward's E4M3 weight codes and their own delayed scale."""
    require_gpu()
    rng = np.random.default_rng(11)
    n, L = 5003, 4
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.1)
    st = fp8.AdamFP8State(torch.from_numpy(w0).cuda(), history_len=L, weight_codes="e4m3", weight_history_len=L,
                          **hp)
    q_s = q_si = np.float32(1)
    q_h = np.zeros(L, np.float32)
    # oracle state
    m_q = np.zeros(n, np.uint8)
    v = np.zeros(n, np.uint16)
    w = oracle.f16_encode(w0)
    m_dq = w_dq = np.float32(1)
    m_s = m_si = w_s = w_si = np.float32(1)
    m_h, w_h = np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in range(1, 13):
        g = f32_to_bf16_bits((rng.standard_normal(n) * 1e-2 * t).astype(np.float32))
        c1, c2 = oracle.bias_corrections(hp["beta1"], hp["beta2"], t)
        m_q, v, w, ma, wa = oracle.adam_step_ref(g, "bf16", m_q, m_dq, m_s, v, w, w_dq, w_s, hp["lr"], hp["beta1"],
                                                 hp["beta2"], hp["eps"], hp["weight_decay"], c1, c2)
        m_dq, w_dq = m_si, w_si
        wq, qa = oracle.adam_weight_codes_ref(w, w_si, q_s, "e4m3")   # cast with the forward weight's scale in force
        q_h[0] = oracle.max_nan([q_h[0], qa])
        q_s, q_si, q_h = oracle.update_scale(q_h, q_s, q_si, "e4m3", 0)
        m_h[0] = oracle.max_nan([m_h[0], ma])
        w_h[0] = oracle.max_nan([w_h[0], wa])
        m_s, m_si, m_h = oracle.update_scale(m_h, m_s, m_si, "e4m3", 0)
        w_s, w_si, w_h = oracle.update_fp16_scale(w_h, w_s, w_si, 0)
        banner("adam-recipe", t)
        st.step(dev(g).view(torch.int16))
        assert np.array_equal(host(st.m_q), m_q), (t, first_diff(host(st.m_q), m_q))
        assert np.array_equal(host(st.v.view(torch.int16)), v), t
        assert np.array_equal(host(st.w.view(torch.int16)), w), t
        assert _bits(host(st.m_state.scale))[0] == _bits(m_s) and _bits(host(st.w_state.scale))[0] == _bits(w_s)
        assert _bits(host(st.m_dq)[st.cur]) == _bits(m_dq) and _bits(host(st.w_dq)[st.cur]) == _bits(w_dq)
        assert np.array_equal(host(st.wq), wq), (t, first_diff(host(st.wq), wq))
        assert _bits(host(st.wq_state.scale))[0] == _bits(q_s)
    # the master weights moved against the mean gradient sign, as Adam does
    assert np.isfinite(host(st.master_weights())).all()


def test_adam_full_size_weight():
    """The 7B up-projection weight (11008 x 4096 parameters), sampled against the oracle."""
    require_gpu()
    n = 11008 * 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    grad = (torch.randn(n, device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    m_q = torch.randint(0, 0x7E, (n,), dtype=torch.uint8, device="cuda", generator=g)
    v = (torch.rand(n, device="cuda", generator=g) * 1e-5).to(torch.float16)
    w = (torch.randn(n, device="cuda", generator=g) * 0.02 * 4096).to(torch.float16)
    rng = np.random.default_rng(6)
    idx = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 4000, replace=False)]))
    ti = torch.from_numpy(idx).cuda()
    before = [host(x[ti]) for x in (grad.view(torch.int16), m_q, v.view(torch.int16), w.view(torch.int16))]
    scal = [f32(x) for x in (2.0 ** -20, 2.0 ** 20, 2.0 ** -20, 1 / 4096, 4096.0, 1 / 4096)]
    mdo, wdo, ma, wa = f32(0), f32(0), f32(0), f32(0)
    banner("adam-full", n)
    fp8.fp8_adam_step(grad, m_q, scal[0], mdo, scal[1], scal[2], ma, v.view(torch.int16), w.view(torch.int16),
                      scal[3], wdo, scal[4], scal[5], wa, **{k: v_ for k, v_ in zip(
                          ("lr", "beta1", "beta2", "eps", "weight_decay", "step"), (1e-4, 0.9, 0.95, 1e-8, 0.1, 3))})
    ref = oracle.adam_step_ref(before[0], "bf16", before[1], 2.0 ** -20, 2.0 ** 20, before[2], before[3], 1 / 4096,
                               4096.0, 1e-4, 0.9, 0.95, 1e-8, 0.1, *oracle.bias_corrections(0.9, 0.95, 3))
    assert np.array_equal(host(m_q[ti]), ref[0])
    assert np.array_equal(host(v.view(torch.int16)[ti]), ref[1])
    assert np.array_equal(host(w.view(torch.int16)[ti]), ref[2])
