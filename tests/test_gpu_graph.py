"""GPU test of a layer step captured as a HIP graph (LayerPlan.capture).

Replays of the captured step must leave exactly the state an eager plan reaches
with the same calls: codes, BF16 outputs, amax histories, scales and inverse
scales, bit for bit, after every replay. The inputs change in place between
steps (the graph reads them at fixed addresses), and unrelated eager work and
synchronizations run between the replays.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import banner, dev, first_diff, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("accum", ["exact", "fast"])
@pytest.mark.parametrize("output_cast", [None, "fused"])
def test_graph_replays_match_eager_steps(accum, output_cast):
    require_gpu()
    import workloads as wl
    from fp8_mixed_precision_cast_amd.linear import GemmOp, LayerPlan, OperandSpec
    xs = [wl.small_normal(30 + t, (300, 256), std=1.0, outlier_factor=20.0) for t in range(6)]
    w = wl.small_normal(29, (520, 256), std=0.02)
    ops = [OperandSpec("X", (300, 256), "e4m3"), OperandSpec("W", (520, 256), "e4m3")]
    gem = [GemmOp("fwd", "X", False, "W", False)]
    plans = {k: LayerPlan(ops, gem, history_len=8, output_cast=output_cast, gemm_accum=accum)
             for k in ("eager", "graph")}
    inp = {k: {"X": dev(xs[0]), "W": dev(w)} for k in plans}
    for k, p in plans.items():
        p.prime(inp[k])
        p.step(inp[k])
    banner("graph capture", accum, output_cast)
    g = plans["graph"].capture(inp["graph"])
    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for t in range(1, len(xs)):
        for k in plans:
            inp[k]["X"].copy_(dev(xs[t]))
        banner("graph replay", accum, output_cast, t)
        plans["eager"].step(inp["eager"])
        g.replay()
        scratch.fill_(float(t))                 # unrelated eager work between replays
        torch.cuda.synchronize()
        e, r = plans["eager"], plans["graph"]
        for name in ("X", "W"):
            a, b = host(e.q[name]), host(r.q[name])
            assert np.array_equal(a, b), (t, name, first_diff(a, b))
            for attr in ("history", "scale", "scale_inv"):
                a = host(getattr(e.state[name], attr)).view(np.uint32)
                b = host(getattr(r.state[name], attr)).view(np.uint32)
                assert np.array_equal(a, b), (t, name, attr)
        a, b = host(e.out["fwd"].view(torch.int16)), host(r.out["fwd"].view(torch.int16))
        assert np.array_equal(a, b), (t, "C", first_diff(a, b))
        if output_cast:
            assert np.array_equal(host(e.yq["fwd"]), host(r.yq["fwd"])), (t, "y codes")
            for attr in ("history", "scale", "scale_inv"):
                a = host(getattr(e.ystate["fwd"], attr)).view(np.uint32)
                b = host(getattr(r.ystate["fwd"], attr)).view(np.uint32)
                assert np.array_equal(a, b), (t, "y", attr)


@pytest.mark.parametrize("accum", ["exact", "fast"])
def test_multi_step_graph_matches_eager_steps(accum):
    """A graph of three consecutive steps (capture(steps=3)): each replay leaves the state of three eager
    steps, bit for bit; the history, whose oldest entries the steps roll out, tells three from two or
    four."""
    require_gpu()
    import workloads as wl
    from fp8_mixed_precision_cast_amd.linear import GemmOp, LayerPlan, OperandSpec
    xs = [wl.small_normal(60 + t, (300, 256), std=1.0 + 0.5 * t, outlier_factor=20.0) for t in range(4)]
    w = wl.small_normal(59, (520, 256), std=0.02)
    ops = [OperandSpec("X", (300, 256), "e4m3"), OperandSpec("W", (520, 256), "e4m3")]
    gem = [GemmOp("fwd", "X", False, "W", False)]
    plans = {k: LayerPlan(ops, gem, history_len=16, gemm_accum=accum) for k in ("eager", "graph")}
    inp = {k: {"X": dev(xs[0]), "W": dev(w)} for k in plans}
    for k, p in plans.items():
        p.prime(inp[k])
        p.step(inp[k])
    banner("graph capture, 3 steps", accum)
    g = plans["graph"].capture(inp["graph"], steps=3)
    for t in range(1, len(xs)):
        for k in plans:
            inp[k]["X"].copy_(dev(xs[t]))
        banner("3-step graph replay", accum, t)
        for _ in range(3):
            plans["eager"].step(inp["eager"])
        g.replay()
        torch.cuda.synchronize()
        e, r = plans["eager"], plans["graph"]
        for name in ("X", "W"):
            assert np.array_equal(host(e.q[name]), host(r.q[name])), (t, name)
            for attr in ("history", "scale", "scale_inv"):
                a = host(getattr(e.state[name], attr)).view(np.uint32)
                b = host(getattr(r.state[name], attr)).view(np.uint32)
                assert np.array_equal(a, b), (t, name, attr)
        a, b = host(e.out["fwd"].view(torch.int16)), host(r.out["fwd"].view(torch.int16))
        assert np.array_equal(a, b), (t, "C", first_diff(a, b))
