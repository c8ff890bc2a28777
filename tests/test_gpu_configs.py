"""The five workloads end to end through the C-ABI, in the launch configuration the benchmark times.

Every workload runs the hot path as the benchmark does (LayerPlan: fused
amax+cast(+transpose) of every operand, the GEMMs, the scale updates). The
tiny workload is checked in full for all 16 delayed-scaling steps. The large
ones are checked at full size on what the oracle can compute piece by piece:
amax, scales and history exactly; sampled rows and columns of the codes
exactly; q_t == q^T on the device for every element; and a sampled block of
every GEMM's output against the oracle's FP64 result on the oracle's own codes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import banner, dev, host, require_gpu

import fp8_mixed_precision_cast_amd as fp8
from fp8_mixed_precision_cast_amd.linear import plan_from_workload

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _state_equal(st, rec, tag):
    assert np.array_equal(_bits(host(st.history)), _bits(rec.history)), f"{tag}: history"
    assert _bits(host(st.scale))[0] == _bits(rec.scale), f"{tag}: scale"
    assert _bits(host(st.scale_inv))[0] == _bits(rec.scale_inv), f"{tag}: scale_inv"


def test_tiny_forward_sixteen_steps():
    require_gpu()
    w = wl.BY_NAME["tiny_fwd_256"]
    inp = wl.load(w.name)
    xs = wl.tiny_step_inputs(inp["X"], wl.step_factors(w.config_id, w.steps))
    plan = plan_from_workload(w)
    recs = {n: oracle.DelayedScaling(w.formats[n], w.history_len, w.margin) for n in ("X", "W")}
    wd = dev(inp["W"])
    saturated_steps = []
    for t, xt in enumerate(xs):
        banner("tiny step", t)
        plan.step({"X": dev(xt), "W": wd})
        qx = recs["X"].cast_step(xt, "f32")
        qw = recs["W"].cast_step(inp["W"], "f32")
        sx_inv, sw_inv = recs["X"].scale_inv, recs["W"].scale_inv
        assert np.array_equal(host(plan.q["X"]), qx), f"step {t}: X codes"
        if ((qx & 0x7F) == 0x7E).any():
            saturated_steps.append(t)
        assert np.array_equal(host(plan.q["W"]), qw), f"step {t}: W codes"
        ref = oracle.gemm_ref(qx, "e4m3", qw, "e4m3", sx_inv, sw_inv)
        absr = oracle.gemm_abs_ref(qx, "e4m3", qw, "e4m3", sx_inv, sw_inv)
        ok, worst = oracle.gemm_check(host(plan.out["fwd"].view(torch.int16)), ref, absr)
        assert ok, f"step {t}: gemm worst {worst}"
        for r in recs.values():
            r.update()
        _state_equal(plan.state["X"], recs["X"], f"step {t} X")
        _state_equal(plan.state["W"], recs["W"], f"step {t} W")
    # steps whose u_t exceeds every earlier factor overflow the delayed scale and saturate
    assert saturated_steps == [1, 4, 6]


def _sample(n, k, rng):
    idx = rng.choice(n, min(k, n), replace=False)
    return np.unique(np.concatenate([[0, n - 1], idx]))


BIG = ["mlp7b_up_fwd", "mlp7b_bwd_hybrid", "proj13b_fwd", "slice70b_fwd"]


@pytest.mark.parametrize("name", BIG)
def test_full_size_workload(name):
    require_gpu()
    w = wl.BY_NAME[name]
    banner("generate", name)
    inp = wl.load(w.name)
    plan = plan_from_workload(w)
    dinp = {k: dev(v) for k, v in inp.items()}
    banner("run", name)
    plan.prime(dinp)
    plan.step(dinp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.config_id)

    used = {}
    for t in w.tensors:
        fmt = w.formats[t.name]
        x = inp[t.name]
        banner("check", name, t.name)
        rec = oracle.primed_scale(x, fmt, "bf16", w.history_len, w.margin)
        used[t.name] = (rec.scale, rec.scale_inv)
        a = oracle.amax(x, "bf16")
        rec.record(a)
        rec.update()
        _state_equal(plan.state[t.name], rec, f"{name}/{t.name}")
        rows = _sample(x.shape[0], 48, rng)
        q = plan.q[t.name]
        got = host(q[torch.from_numpy(rows).cuda()])
        want = oracle.cast(x[rows], used[t.name][0], fmt, "bf16")
        assert np.array_equal(got, want), f"{t.name} sampled rows"
        if plan.qt[t.name] is not None:
            qt = plan.qt[t.name]
            assert torch.equal(qt, q.t()), f"{t.name}: q_t != q^T"
            cols = _sample(x.shape[1], 16, rng)
            got_t = host(qt[torch.from_numpy(cols).cuda()])
            want_t = oracle.cast(np.ascontiguousarray(x[:, cols].T), used[t.name][0], fmt, "bf16")
            assert np.array_equal(got_t, want_t), f"{t.name} sampled columns"

    for g in w.gemms:
        banner("gemm-check", name, g.name)
        y = plan.out[g.name]
        assert y.shape == (g.m, g.n)
        ii = _sample(g.m, 62, rng)
        jj = _sample(g.n, 62, rng)

        def operand_rows(tname, transposed, idx):
            x = inp[tname]
            src = np.ascontiguousarray(x[:, idx].T) if transposed else x[idx]
            return oracle.cast(src, used[tname][0], w.formats[tname], "bf16")

        qa = operand_rows(g.a, g.a_transposed, ii)
        qb = operand_rows(g.b, g.b_transposed, jj)
        ref = oracle.gemm_ref(qa, g.a_fmt, qb, g.b_fmt, used[g.a][1], used[g.b][1])
        absr = oracle.gemm_abs_ref(qa, g.a_fmt, qb, g.b_fmt, used[g.a][1], used[g.b][1])
        yi = y.view(torch.int16)[torch.from_numpy(ii).cuda()][:, torch.from_numpy(jj).cuda()]
        ok, worst = oracle.gemm_check(host(yi), ref, absr)
        assert ok, f"{name}/{g.name}: worst |err|/bound {worst}"
        assert torch.isfinite(y.float()).all(), f"{name}/{g.name}: non-finite output"
