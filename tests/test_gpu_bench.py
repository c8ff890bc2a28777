"""bench.py end to end on the GPU with few steps, in this process: the one JSON line and its contract
fields, and the diagnostic modes at small sizes."""
import json
import os
import sys

import pytest

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(monkeypatch, capsys, *args):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    bench.main()
    out = capsys.readouterr().out
    return [json.loads(line) for line in out.splitlines() if line.startswith("{")]


def test_bench_line_contract(monkeypatch, capsys):
    require_gpu()
    (line,) = _run(monkeypatch, capsys, "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert line["config"]["settle_steps"] >= 10 and line["config"]["settle_s"] == 2.0
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "components"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 2 and line["warmup"] == 1
    assert line["config"]["workload"] == "mlp7b_up_fwd" and line["value"] > 0
    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["peak"] == 5000.0 and roof["instruction_peak"] == 2500.0
    assert line["components"]["gemm_fast_accum_tflops"] > 0
    par = line["parity"]
    assert par["ok"] and len(par["checked"]) == 3, par
    assert par["checked"][-1]["fp32_bound_ok"]
    clk = line["clocks"]
    assert clk is not None and ("sclk_mhz" in clk or "error" in clk)
    assert line["config"]["step_launch"] == "hip_graph" and line["config"]["steps_per_graph"] == 2
    assert 0 < line["ms_per_step"] and 0 < line["components"]["eager_ms_per_step"]
    (eager,) = _run(monkeypatch, capsys, "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-graph")
    assert eager["config"]["step_launch"] == "eager"
    assert eager["ms_per_step"] == eager["components"]["eager_ms_per_step"]
    pc = line["percentiles_ms"]["step"]
    assert 0 < pc["p10"] <= pc["p50"] <= pc["p90"] and line["rocm"]["hip"]
    (fast,) = _run(monkeypatch, capsys, "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--gemm-accum", "fast")
    assert fast["config"]["gemm_accum"] == "fast" and fast["roofline"]["peak"] == 5000.0
    assert fast["roofline"]["instruction_peak"] == 5000.0 and fast["parity"]["ok"]
    assert fast["parity"]["checked"][-1]["fast_bound_ok"]
    assert fast["components"]["gemm_exact_accum_tflops"] > 0


def test_bench_diagnostic_modes(monkeypatch, capsys):
    require_gpu()
    lines = _run(monkeypatch, capsys, "--gemm-data", "512x768x256")
    kinds = {l.get("gemm_data") for l in lines if "gemm_data" in l}
    assert kinds == {"zero", "one", "uniform", "normal"}
    assert {l.get("accum") for l in lines if "gemm_data" in l} == {"exact", "fast"}
    assert all(l["tflops"] > 0 for l in lines if "gemm_data" in l)
    (copy,) = _run(monkeypatch, capsys, "--copy-reference", str(1 << 24))
    assert copy["copy_reference_bytes"] == 1 << 24 and copy["copy_gbps"] > 0
