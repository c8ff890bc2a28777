"""Just-in-time (current) per-tensor scaling through the C-ABI, against the oracle.

The scale comes from the tensor's own amax in the same step: an amax-only pass,
the update on a one-entry history, then the cast with the fresh scale.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle.recipe import update_scale
from tests.gpu_util import banner, dev, host, pitched, require_gpu

import fp8_mixed_precision_cast_amd as fp8
from fp8_mixed_precision_cast_amd.linear import plan_from_workload

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _jit_scale(x, dtype, fmt, margin, prev=(1.0, 1.0)):
    s, si, _ = update_scale(np.array([oracle.amax(x, dtype)], np.float32), np.float32(prev[0]),
                            np.float32(prev[1]), fmt, margin)
    return s, si


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("margin", [0, 2])
def test_current_scaling_codes_and_scales(fmt, margin):
    require_gpu()
    for shape, std in (((300, 200), 1.0), ((1024, 512), 0.02), ((64, 4096), 1e-3)):
        x = wl.small_normal(shape[0] + margin, shape, std=std, outlier_factor=20.0)
        banner("current", fmt, margin, shape)
        st = fp8.CurrentScalingState(fmt, margin)
        q, _ = pitched(shape[0], shape[1], torch.uint8)
        qt, _ = pitched(shape[1], shape[0], torch.uint8)
        st.cast(dev(x), q, qt)
        s, si = _jit_scale(x, "bf16", fmt, margin)
        assert _bits(host(st.scale))[0] == _bits(s) and _bits(host(st.scale_inv))[0] == _bits(si)
        want = oracle.cast(x, s, fmt, "bf16")
        assert np.array_equal(host(q), want)
        assert np.array_equal(host(qt), want.T)
        assert host(st.slot)[0] == 0.0          # the one-entry history was rolled
        codes = want & 0x7F
        assert codes.max() == oracle.FMT[fmt].max_code or margin > 0


def test_current_scaling_holds_on_zero_tensor():
    require_gpu()
    st = fp8.CurrentScalingState("e4m3")
    x = torch.randn(64, 64, device="cuda").to(torch.bfloat16)
    q = torch.empty(64, 64, dtype=torch.uint8, device="cuda")
    st.cast(x, q)
    s_prev = host(st.scale)[0]
    st.cast(torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda"), q)
    assert host(st.scale)[0] == s_prev and not host(q).any()


def test_current_scaling_layer_step_full_size():
    require_gpu()
    w = wl.BY_NAME["mlp7b_up_fwd"]
    inp = wl.load(w.name)
    plan = plan_from_workload(w, recipe="current")
    dinp = {k: dev(v) for k, v in inp.items()}
    banner("current layer step")
    plan.step(dinp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    sc = {}
    for t in w.tensors:
        s, si = _jit_scale(inp[t.name], "bf16", "e4m3", 0)
        sc[t.name] = (s, si)
        assert _bits(host(plan.state[t.name].scale))[0] == _bits(s)
    ii = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 62, replace=False)]))
    jj = np.unique(np.concatenate([[0, 11007], rng.choice(11008, 62, replace=False)]))
    qa = oracle.cast(inp["X"][ii], sc["X"][0], "e4m3", "bf16")
    qb = oracle.cast(inp["W"][jj], sc["W"][0], "e4m3", "bf16")
    assert np.array_equal(host(plan.q["X"][torch.from_numpy(ii).cuda()]), qa)
    ref = oracle.gemm_ref(qa, "e4m3", qb, "e4m3", sc["X"][1], sc["W"][1])
    absr = oracle.gemm_abs_ref(qa, "e4m3", qb, "e4m3", sc["X"][1], sc["W"][1])
    y = plan.out["fwd"].view(torch.int16)[torch.from_numpy(ii).cuda()][:, torch.from_numpy(jj).cuda()]
    ok, worst = oracle.gemm_check(host(y), ref, absr)
    assert ok, worst
