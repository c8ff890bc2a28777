#!/usr/bin/env python3
"""Benchmark of the per-tensor-scaled FP8 linear layer's hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: the
fused amax+cast of X and of W with the delayed scales, the scaled FP8 GEMM
into BF16, and the two scale updates, all through the C-ABI library. The
default workload is the 7B-class MLP up-projection (X[4096x4096] BF16 with
0.1% outliers x20, W[11008x4096] BF16 N(0, 0.02); GEMM M=4096, N=11008,
K=4096; amax history 1024, margin 0).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload mlp7b_up_fwd]

Prints one JSON line. After W warm-up steps, --steps-per-graph consecutive
steps (10 by default, fewer when that does not divide K) are captured as one
HIP graph, as a training loop captures an iteration of many layers, and
replayed untimed for --settle-seconds (the GPU's power management dips a few
milliseconds into a burst and settles within a second or two); then K steps of
replays are timed, synchronized on both sides: `value` is the step's GEMM
FLOPs divided by that step time (TFLOP/s, higher is better; `--no-graph` times
eager steps instead). K eager steps follow directly, with HIP events around
every phase on the launch stream: they give `roofline` (the dominant kernel,
the GEMM, per launch) and the per-phase `components`. `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_MFMA_TFLOPS = 2500.0  # dense
PEAK_FP8_MFMA_TFLOPS = 5000.0   # dense


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="before the warm-up steps, repeat the step untimed for this long so the GPU's clock and "
                         "power management have settled (reported in config.settle_s)")
    ap.add_argument("--workload", default="mlp7b_up_fwd")
    ap.add_argument("--recipe", default="delayed", choices=["delayed", "current"],
                    help="delayed scaling (the pages' default recipe) or just-in-time scaling")
    ap.add_argument("--output-cast", default="none", choices=["none", "fused", "fused_codes", "separate"],
                    help="also cast the GEMM output to E4M3 for a next layer: in the GEMM epilogue (fused_codes: "
                         "without storing the BF16 output) or as a second pass")
    ap.add_argument("--layernorm", action="store_true",
                    help="X is LayerNorm(X) (gamma ~ N(1, 0.2), beta ~ N(0, 0.2), eps 1e-5), normalised and cast in one pass")
    ap.add_argument("--gemm-accum", default="exact", choices=["exact", "fast"],
                    help="exact: FP32 accumulation (BF16 MFMA on exactly widened FP8); fast: the FP8 MFMA's own "
                         "reduced-precision accumulation (within 2^-9 of sum|a*b|)")
    ap.add_argument("--steps-per-graph", type=int, default=10,
                    help="consecutive steps captured in one HIP graph (the largest divisor of --steps up to this "
                         "is used; 1 replays a one-step graph per step)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager steps only (by default the timed steps are replays of the step captured "
                         "as a HIP graph, after the eager steps that give the per-kernel figures)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clocks", action="store_true", help="skip the clock window (amdsmi)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per GEMM launch from rocprofv3 counters (JSON), if present")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES three times (calibrates HBM counters) and "
                         "report its rate")
    ap.add_argument("--gemm-data", default="", metavar="MxNxK",
                    help="only time fp8_scaled_gemm (and its fast-accumulation form) at this shape on E4M3 "
                         "operands of several kinds "
                         "(all zero, all 1.0, uniform random codes, cast N(0,1) values): one JSON line per kind")
    return ap.parse_args()


GEMM_SOURCES = ("gemm_kernels.h", "gemm_parts.h", "gemm.hip", "gemm_exact_a4.hip", "gemm_exact_a5.hip", "gemm_fast.hip")


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: what the compiler sees."""
    import re
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] in "\"'":
            q, j = src[i], i + 1
            while j < n and src[j] != q:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_digest() -> str:
    """Digest of the GEMM sources' code (in this order, comments and whitespace left out); counter readings are
    valid only for the code they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "fp8_mixed_precision_cast_amd", "csrc", name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def copy_reference(nbytes: int) -> None:
    """Three device copies of nbytes; prints the fastest one's rate (bytes read + written per second)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    print(json.dumps({"copy_reference_bytes": nbytes, "copy_ms": round(best, 4),
                      "copy_gbps": round(2 * nbytes / best / 1e6, 1)}), flush=True)


def gemm_data(shape: str, iters: int = 20) -> None:
    """fp8_scaled_gemm at one shape on operands of different content. The instruction stream does not
    depend on the data, but the power it draws does: on a power-limited chip the clock, and with it
    the rate, falls as the operands' bits toggle more."""
    import torch
    import fp8_mixed_precision_cast_amd as fp8
    m, n, k = (int(v) for v in shape.lower().split("x"))
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    c = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    one = torch.ones(1, device="cuda")

    def codes(kind, rows):
        if kind == "zero":
            return torch.zeros(rows, k, dtype=torch.uint8, device="cuda")
        if kind == "one":
            return torch.full((rows, k), 0x38, dtype=torch.uint8, device="cuda")   # E4M3 1.0
        if kind == "uniform":
            q = torch.randint(0, 256, (rows, k), dtype=torch.uint8, device="cuda", generator=g)
            q[(q & 0x7F) == 0x7F] = 0x7E   # no NaN codes
            return q
        x = torch.randn(rows, k, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
        q = torch.empty(rows, k, dtype=torch.uint8, device="cuda")
        fp8.fp8_amax_cast(x, "e4m3", torch.full((1,), 448.0 / 4.5, device="cuda"), q)
        return q

    for kind in ("zero", "one", "uniform", "normal"):
        a, b = codes(kind, m), codes(kind, n)
        for accum, call in (("exact", fp8.fp8_scaled_gemm), ("fast", fp8.fp8_scaled_gemm_fast_accum)):
            for _ in range(5):
                call(a, "e4m3", b, "e4m3", one, one, c)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                call(a, "e4m3", b, "e4m3", one, one, c)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            print(json.dumps({"gemm_data": kind, "accum": accum, "shape": [m, n, k], "us": round(ms * 1e3, 1),
                              "tflops": round(2 * m * n * k / ms / 1e9, 1)}), flush=True)
        del a, b
    # Context: the vendor library through torch at the same shape on N(0,1) data, BF16 x BF16 (the
    # same MFMA path as ours) and FP8 x FP8 (the FP8 MFMA, whose accumulation is coarser than the
    # tolerance this library is held to).
    a = torch.randn(m, k, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, k, device="cuda", generator=g).to(torch.bfloat16)
    refs = {"torch_bf16_mm": lambda: a @ b.t()}
    if hasattr(torch, "_scaled_mm"):
        a8, b8 = (a * 0.25).to(torch.float8_e4m3fn), (b * 0.25).to(torch.float8_e4m3fn)
        refs["torch_fp8_scaled_mm"] = lambda: torch._scaled_mm(a8, b8.t(), scale_a=one[0], scale_b=one[0],
                                                                 out_dtype=torch.bfloat16)
    for name, f in refs.items():
        try:
            for _ in range(5):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                f()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            print(json.dumps({"library": name, "shape": [m, n, k], "us": round(ms * 1e3, 1),
                              "tflops": round(2 * m * n * k / ms / 1e9, 1)}), flush=True)
        except RuntimeError as e:
            print(json.dumps({"library": name, "error": str(e)[:120]}), flush=True)


def cpu_baseline(w, inp, min_seconds: float = 10.0):
    """The oracle's whole step (amax, cast, FP64 GEMM, update) on the workload, repeated
    until at least min_seconds of CPU work have been timed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info})) or "unknown"
    except Exception:
        threads, blas = 1, "unknown"
    g = w.gemms[0]
    x, wt = inp["X"], inp["W"]
    reps, total = 0, 0.0
    stages = {"amax_cast": 0.0, "fp64_gemm": 0.0, "update": 0.0}
    while total < min_seconds and reps < 20:
        t0 = time.perf_counter()
        rx = oracle.DelayedScaling("e4m3", w.history_len, w.margin)
        rw = oracle.DelayedScaling("e4m3", w.history_len, w.margin)
        qx = rx.cast_step(x, "bf16")
        qw = rw.cast_step(wt, "bf16")
        t1 = time.perf_counter()
        y = oracle.gemm_ref(qx, "e4m3", qw, "e4m3", rx.scale_inv, rw.scale_inv)
        t2 = time.perf_counter()
        rx.update()
        rw.update()
        t3 = time.perf_counter()
        stages["amax_cast"] += t1 - t0
        stages["fp64_gemm"] += t2 - t1
        stages["update"] += t3 - t2
        total += t3 - t0
        reps += 1
        del y
    flops = 2.0 * g.m * g.n * g.k
    return {"value": flops * reps / total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "stage_seconds_per_step": {k: round(v / reps, 4) for k, v in stages.items()},
            "sample": f"{reps} full oracle steps (amax, cast of X and W, FP64 GEMM {g.m}x{g.n}x{g.k}, "
                      f"update) in {total:.1f} s; elementwise stages single-threaded, BLAS on {threads} threads"}


def cold_cast_gbps(plan, dinp, reps: int = 5):
    """The casts timed after the 256 MB MALL has been flushed by writing a 1 GiB buffer, so the sources
    and codes come from HBM (GB/s of algorithmic bytes, median over reps)."""
    import torch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plan.cast_all(dinp)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    times.sort()
    ms = times[len(times) // 2]
    return plan.cast_bytes(dinp) / (ms * 1e-3) / 1e9, ms


def settle(run, steps_per_run: int, seconds: float) -> int:
    """Calls run() (steps_per_run steps) untimed for `seconds`; returns the number of steps run. A few
    milliseconds into a burst of work the power controller lowers the clock below where it ends up
    after a second or two (per-dispatch traces show it), so the timed steps follow this directly."""
    import torch
    n = 0
    torch.cuda.synchronize()
    s0 = time.perf_counter()
    while True:   # at least once, so a captured graph has been replayed before it is timed
        run()
        n += steps_per_run
        torch.cuda.synchronize()
        if time.perf_counter() - s0 >= seconds:
            return n


def steps_per_graph(k: int, wanted: int) -> int:
    """The largest divisor of k that is at most `wanted` (at least 1): the timed region then replays
    whole graphs for exactly k steps."""
    return max(d for d in range(1, max(1, min(k, wanted)) + 1) if k % d == 0)


def graph_steps(g, steps: int):
    """Replays the captured graph `steps` times, synchronized on both sides. Returns (wall seconds per
    replay, per-replay milliseconds from HIP events recorded between the replays on the launch
    stream)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def other_gemm_tflops(plan, accum: str, iters: int = 20) -> float:
    """The plan's GEMMs, on the codes of the last step, in the other accumulation mode: TFLOP/s per
    launch from HIP events around iters rounds (outside the timed steps)."""
    import torch
    import fp8_mixed_precision_cast_amd as fp8
    call = fp8.fp8_scaled_gemm_fast_accum if accum == "fast" else fp8.fp8_scaled_gemm
    stream = torch.cuda.current_stream()
    outs = [torch.empty_like(c) for (_, _, _, _, _, _, c) in plan.gemm_operands()]
    for _ in range(3):
        for (a, af, b, bf, sa, sb, _), c in zip(plan.gemm_operands(), outs):
            call(a, af, b, bf, sa, sb, c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        for (a, af, b, bf, sa, sb, _), c in zip(plan.gemm_operands(), outs):
            call(a, af, b, bf, sa, sb, c)
    e1.record(stream)
    torch.cuda.synchronize()
    return plan.gemm_flops() * iters / (e0.elapsed_time(e1) * 1e-3) / 1e12


class ClockSampler:
    """The GPU's graphics clock (SCLK, mean over the XCDs), memory clock (MCLK) and socket power while the
    step runs, read through the amdsmi library from the device's metrics table. The table refreshes
    about once a second, so a background thread polls it every 20 ms and keeps each refreshed reading
    (a new system clock counter) taken after the window began; the mean power between the first and
    last of them comes from the energy accumulator. Reports what it saw, or why it could not."""

    def __init__(self):
        self.readings, self.error, self._stop, self._thread, self._h, self._smi = [], None, False, None, None, None
        self._first = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                raise RuntimeError("no GPU handle")
            self._h = handles[0]
            self._smi = amdsmi
            self._res = float(amdsmi.amdsmi_get_energy_count(self._h).get("counter_resolution", 15.3))
            self._first = self._read()
        except Exception as e:  # the numbers are context; their absence is reported, not fatal
            self.error = f"{type(e).__name__}: {str(e)[:100]}"
            self._smi = None

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        g = m.get("current_gfxclks")
        gfx = [v for v in g if isinstance(v, (int, float)) and 0 < v < 65535] if isinstance(g, (list, tuple)) else []
        num = lambda v: v if isinstance(v, (int, float)) else None
        return {"counter": m.get("system_clock_counter"), "sclk": sum(gfx) / len(gfx) if gfx else None,
                "sclk_per_xcd": gfx, "mclk": num(m.get("current_uclk")),
                "power": num(m.get("current_socket_power")), "energy": num(m.get("energy_accumulator"))}

    def _poll(self):
        last = self._first["counter"]
        while not self._stop:
            try:
                r = self._read()
            except Exception as e:
                self.error = f"{type(e).__name__}: {str(e)[:100]}"
                return
            if r["counter"] != last:
                self.readings.append(r)
                last = r["counter"]
            time.sleep(0.02)

    def __enter__(self):
        if self._smi is not None:
            import threading
            self._thread = threading.Thread(target=self._poll, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self):
        # the first refreshed reading may still average time before the load began
        rs = self.readings[1:] if len(self.readings) > 2 else self.readings
        if not rs:
            return {"error": self.error or "no refreshed reading of the metrics table in the window"}

        def stats(key):
            v = sorted(r[key] for r in rs if r[key] is not None)
            return {"median": v[len(v) // 2], "min": v[0], "max": v[-1]} if v else None
        out = {"readings": len(rs), "sclk_mhz": stats("sclk"), "mclk_mhz": stats("mclk"),
               "socket_power_w": stats("power"), "sclk_per_xcd_mhz_last": rs[-1]["sclk_per_xcd"],
               "source": "amdsmi gpu metrics table (refreshed about once a second), polled during the window"}
        a, b = rs[0], rs[-1]
        if len(rs) > 1 and a["energy"] is not None and b["energy"] is not None and b["counter"] != a["counter"]:
            # system_clock_counter counts nanoseconds
            out["mean_power_w"] = round((b["energy"] - a["energy"]) * self._res * 1e-6 /
                                        ((b["counter"] - a["counter"]) * 1e-9), 1)
        return out


def parity(w, inp, plan, n_updates: int, recorded_after: bool, fast: bool, seed: int = 7):
    """Parity of what the timed steps left in the plan against the oracle, outside the timed region.
    Under the delayed recipe with plain operands, every step casts the same data, so after n_updates
    updates the oracle's recipe (record amax, update, n_updates times; one more record when casts
    ran after the last update) gives the history, scale and scale_inv, which must match bit for bit;
    the codes of sampled rows of every tensor must equal the oracle's cast with that scale; a
    sampled block of every GEMM's output is graded against the oracle's FP64 GEMM on the oracle's
    codes under the FP32-accumulation bound (and, for the fast GEMM, its own bound)."""
    import numpy as np
    import torch
    import oracle
    from oracle.gemm import FAST_ACCUM_SUM_COEF
    rng = np.random.default_rng(seed)
    res = {"checked": [], "ok": True}

    def fail(msg):
        res["ok"] = False
        res.setdefault("failures", []).append(msg)

    used = {}
    for t in w.tensors:
        fmt = w.formats[t.name]
        x = inp[t.name]
        rec = oracle.DelayedScaling(fmt, w.history_len, w.margin)
        a = oracle.amax(x, t.dtype)
        for _ in range(n_updates):
            rec.record(a)
            rec.update()
        if recorded_after:
            rec.record(a)
        used[t.name] = (rec.scale, rec.scale_inv)
        st = plan.state[t.name]
        hist = st.history.cpu().numpy().view(np.uint32)
        if not np.array_equal(hist, rec.history.view(np.uint32)):
            fail(f"{t.name}: history")
        if st.scale.cpu().numpy().view(np.uint32)[0] != np.float32(rec.scale).view(np.uint32):
            fail(f"{t.name}: scale")
        if st.scale_inv.cpu().numpy().view(np.uint32)[0] != np.float32(rec.scale_inv).view(np.uint32):
            fail(f"{t.name}: scale_inv")
        rows = np.unique(np.concatenate([[0, x.shape[0] - 1], rng.choice(x.shape[0], 62, replace=False)]))
        got = plan.q[t.name][torch.from_numpy(rows).cuda()].cpu().numpy()
        if not np.array_equal(got, oracle.cast(x[rows], rec.scale, fmt, t.dtype)):
            fail(f"{t.name}: codes of sampled rows")
        if plan.qt[t.name] is not None and not torch.equal(plan.qt[t.name], plan.q[t.name].t()):
            fail(f"{t.name}: q_t != q^T")
        res["checked"].append(f"{t.name}: history, scale, scale_inv bit-exact; {rows.size} code rows exact")
    for g in w.gemms:
        ii = np.unique(np.concatenate([[0, g.m - 1], rng.choice(g.m, 62, replace=False)]))
        jj = np.unique(np.concatenate([[0, g.n - 1], rng.choice(g.n, 62, replace=False)]))

        def rows_of(name, transposed, idx):
            x = inp[name]
            src = np.ascontiguousarray(x[:, idx].T) if transposed else x[idx]
            return oracle.cast(src, used[name][0], w.formats[name], w.tensor(name).dtype)

        qa, qb = rows_of(g.a, g.a_transposed, ii), rows_of(g.b, g.b_transposed, jj)
        sa, sb = used[g.a][1], used[g.b][1]
        ref = oracle.gemm_ref(qa, g.a_fmt, qb, g.b_fmt, sa, sb)
        absr = oracle.gemm_abs_ref(qa, g.a_fmt, qb, g.b_fmt, sa, sb)
        y = plan.out[g.name].view(torch.int16)[torch.from_numpy(ii).cuda()][:, torch.from_numpy(jj).cuda()]
        yb = y.cpu().numpy().view(np.uint16)
        ok32, worst32 = oracle.gemm_check(yb, ref, absr)
        entry = {"gemm": g.name, "block": [int(ii.size), int(jj.size)], "fp32_bound_ok": ok32,
                 "fp32_bound_worst": round(worst32, 4)}
        if fast:
            okf, worstf = oracle.gemm_check(yb, ref, absr, FAST_ACCUM_SUM_COEF)
            entry.update({"fast_bound_ok": okf, "fast_bound_worst": round(worstf, 4)})
            if not okf:
                fail(f"{g.name}: outside the fast-accumulation bound")
        elif not ok32:
            fail(f"{g.name}: outside the FP32-accumulation bound")
        res["checked"].append(entry)
    return res


def main():
    args = parse()
    if args.copy_reference:
        copy_reference(args.copy_reference)
        return
    if args.gemm_data:
        gemm_data(args.gemm_data)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this path measures one MI355X "
              "and does not shard across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    import fp8_mixed_precision_cast_amd as fp8
    from fp8_mixed_precision_cast_amd.linear import plan_from_workload

    w = wl.BY_NAME[args.workload]
    if w.steps != 1:
        raise SystemExit("bench.py times the single-step workloads")
    info = fp8.fp8mp_device_info()
    inp = wl.load(w.name)
    dinp = {k: torch.from_numpy(v.view("int16")).cuda() for k, v in inp.items()}
    ln_params = None
    if args.layernorm:
        import numpy as np
        rng = np.random.default_rng(20261202)
        cols = inp["X"].shape[1]
        ln_params = {"X": (torch.from_numpy(rng.normal(1.0, 0.2, cols).astype(np.float32)).cuda(),
                           torch.from_numpy(rng.normal(0.0, 0.2, cols).astype(np.float32)).cuda(), 1e-5)}
    plan = plan_from_workload(w, recipe=args.recipe,
                              output_cast=None if args.output_cast == "none" else args.output_cast,
                              layernorm=("X",) if args.layernorm else (), ln_params=ln_params,
                              gemm_accum=args.gemm_accum)
    stream = torch.cuda.current_stream()
    plan.prime(dinp)
    n_updates = 1
    for _ in range(args.warmup):
        plan.step(dinp)
    n_updates += args.warmup
    torch.cuda.synchronize()

    K = args.steps
    # The timed steps: K replays of the step captured as a HIP graph (value, ms_per_step), right after
    # the settle replays; with --no-graph, K eager steps after eager settle steps. The K eager steps
    # with HIP events around every phase (roofline, components) follow directly.
    spg = steps_per_graph(K, args.steps_per_graph)
    if args.no_graph:
        graph = None
        settle_steps = settle(lambda: [plan.step(dinp) for _ in range(10)], 10, args.settle_seconds)
    else:
        graph = plan.capture(dinp, steps=spg)
        reps = max(1, 10 // spg)
        settle_steps = settle(lambda: [graph.replay() for _ in range(reps)], reps * spg, args.settle_seconds)
        graph_replay_s, graph_replay_ms = graph_steps(graph, K // spg)
        graph_step_s = graph_replay_s / spg
        graph_ms = [t / spg for t in graph_replay_ms]
    n_updates += settle_steps + (0 if args.no_graph else K)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        plan.cast_all(dinp)
        e[1].record(stream)
        plan.gemm_all()
        e[2].record(stream)
        plan.output_cast_all()
        e[3].record(stream)
        plan.update_all()
        e[4].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_updates += K

    step_s = (t1 - t0) / K
    cast_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    gemm_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    ocast_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    upd_ms = sum(e[3].elapsed_time(e[4]) for e in ev) / K

    def pct(vals):
        v = sorted(vals)
        at = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
        return {"p10": round(at(0.1), 4), "p50": round(at(0.5), 4), "p90": round(at(0.9), 4)}

    step_pct = pct([e[0].elapsed_time(e[4]) for e in ev])
    gemm_pct = pct([e[1].elapsed_time(e[2]) for e in ev])
    cast_pct = pct([e[0].elapsed_time(e[1]) for e in ev])

    flops = plan.gemm_flops()
    n_gemm = len(plan.gemms)
    gemm_launch_ms = gemm_ms / n_gemm
    flops_per_launch = flops / n_gemm
    gemm_tflops = flops_per_launch / (gemm_launch_ms * 1e-3) / 1e12
    cast_bytes = plan.cast_bytes(dinp)
    cast_gbps = cast_bytes / (cast_ms * 1e-3) / 1e9

    eager_step_s = step_s
    if args.no_graph:
        graph_pct = None
    else:
        step_s = graph_step_s
        graph_pct = pct(graph_ms)
    # Clocks: the step repeated for about three seconds (outside the timed region) while the
    # sampler polls the device's metrics table.
    clocks = None
    if not args.no_clocks:
        sampler = ClockSampler()
        reps = max(1, int(3.0 / max(step_s, 1e-4)))
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        with sampler:
            for _ in range(reps):
                plan.step(dinp)
            torch.cuda.synchronize()
        w1 = time.perf_counter()
        n_updates += reps
        clocks = sampler.summary()
        clocks["steps"] = reps
        # eager steps back to back for seconds: the rate once power management has settled
        clocks["window_ms_per_step"] = round((w1 - w0) / reps * 1e3, 4)
    cold_gbps, cold_ms = cold_cast_gbps(plan, dinp)
    other = "fast" if args.gemm_accum == "exact" else "exact"
    other_tflops = other_gemm_tflops(plan, other)

    traffic = None
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            t = json.load(f).get(w.name if args.gemm_accum == "exact" else w.name + ":fast", {})
        if t.get("gemm_source") == source_digest():
            traffic = t.get("gemm_bytes_per_launch")
    fast = args.gemm_accum == "fast"
    # The roofline is the FP8 dense MFMA peak in both modes. The exact mode runs the BF16 MFMA on
    # exactly widened codes, whose own ceiling (half of it) is reported beside it.
    peak = PEAK_FP8_MFMA_TFLOPS

    g = w.gemms[0]

    def describe(t):
        dist = "N(0,{:g})".format(t.scale) if t.dist == "normal" else "t3 x{:g}".format(t.scale)
        tail = " +0.1% x{:g}".format(t.outlier_factor) if t.outlier_factor else ""
        return "{} {}x{} {}{} -> {}".format(t.dtype, t.shape[0], t.shape[1], dist, tail, w.formats[t.name])

    out = {
        "metric": "FP8 scaled-GEMM TFLOP/s (7B MLP shape) + amax/cast GB/s, % of roofline",
        "value": round(flops / step_s / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 operands; fp8 MFMA (fast accumulation, within 2^-9 of sum|ab|), bf16 out" if fast else
                  "fp8-e4m3 operands; bf16 MFMA (exact on FP8 values), f32 accumulate, bf16 out"),
        "data": "synthetic",
        "config": {"workload": w.name, "m": g.m, "n": g.n, "k": g.k,
                   "gemms": ["{} {}x{}x{} {}x{}".format(x.name, x.m, x.n, x.k, x.a_fmt, x.b_fmt) for x in w.gemms],
                   "tensors": {t.name: describe(t) for t in w.tensors},
                   "transposed_casts": list(w.transposed), "history_len": w.history_len, "margin": w.margin,
                   "recipe": args.recipe, "output_cast": args.output_cast, "layernorm_x": bool(args.layernorm),
                   "gemm_accum": args.gemm_accum,
                   "step_launch": "eager" if args.no_graph else "hip_graph",
                   "steps_per_graph": None if args.no_graph else spg,
                   "settle_s": args.settle_seconds, "settle_steps": settle_steps,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": traffic,
                     "kernel": (("gemm_fp8_kernel" if args.output_cast.startswith("fused") else
                                 "gemm_persistent_kernel") + " (fp8 MFMA, fast accumulation)" if fast else
                                "gemm_persistent_kernel (bf16 MFMA on widened FP8)"),
                     "instruction_peak": PEAK_FP8_MFMA_TFLOPS if fast else PEAK_BF16_MFMA_TFLOPS,
                     "frac_of_instruction_peak": round(gemm_tflops / (PEAK_FP8_MFMA_TFLOPS if fast else
                                                                      PEAK_BF16_MFMA_TFLOPS), 4)},
        "components": {
            "gemm_ms": round(gemm_ms, 4), "gemm_tflops": round(gemm_tflops, 2),
            "cast_ms": round(cast_ms, 4), "cast_bytes": cast_bytes, "cast_gbps": round(cast_gbps, 1),
            "cast_frac_of_hbm": round(cast_gbps / PEAK_HBM_GBPS, 4),
            "scale_update_ms": round(upd_ms, 4),
            "cast_cold_ms": round(cold_ms, 4), "cast_cold_gbps": round(cold_gbps, 1),
            "eager_ms_per_step": round(eager_step_s * 1e3, 4),
            "eager_step_tflops": round(flops / eager_step_s / 1e12, 3),
            f"gemm_{other}_accum_tflops": round(other_tflops, 2),
            f"gemm_{other}_accum_frac_of_peak": round(other_tflops / (PEAK_FP8_MFMA_TFLOPS if other == "fast"
                                                                      else PEAK_BF16_MFMA_TFLOPS), 4),
        },
        "percentiles_ms": {"step": graph_pct or step_pct, "eager_step": step_pct, "gemm": gemm_pct, "cast": cast_pct},
        "device": info,
        "clocks": clocks,
        "rocm": {"hip": torch.version.hip, "torch": torch.__version__},
    }
    if args.output_cast != "none":
        out["components"]["output_cast"] = args.output_cast
        out["components"]["output_cast_bytes"] = plan.output_cast_bytes()
        out["components"]["separate_output_cast_ms"] = round(ocast_ms, 4)
    ok = True
    if args.recipe == "delayed" and not args.layernorm and args.output_cast == "none":
        out["parity"] = parity(w, inp, plan, n_updates, True, fast)
        ok = out["parity"]["ok"]
    else:
        out["parity"] = {"skipped": "checked for the delayed recipe on plain operands; the other options "
                                    "are covered by the GPU tests"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)
    if not ok:
        print("parity check failed: " + "; ".join(out["parity"].get("failures", [])), file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
