"""The C-ABI's calls are thread-safe and keep no state between launches: host threads that each drive
their own stream (the binding passes the calling thread's current torch stream) get, launch for
launch, the same bits as one thread running the same work in order.

Each thread runs its own problem several times over: an amax+cast of a BF16 operand, the scale update,
and the FP32-accumulation GEMM (plain, and with the fused output cast); the reference is the same
sequence on one stream, one problem after another.
"""
import threading

import numpy as np
import pytest
import torch

from tests.gpu_util import banner, host, require_gpu

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu

PROBLEMS = [(1024, 1536, 512), (777, 640, 272), (2048, 1024, 1024), (300, 2112, 96)]   # N: 16-byte rows of codes
ROUNDS = 4


def _inputs(idx):
    m, n, k = PROBLEMS[idx]
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + idx)
    x = torch.randn(m, k, device="cuda", generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(n, k, device="cuda", generator=g)).to(torch.bfloat16)
    return x, w


def _run(idx, x, w):
    """One thread's work: ROUNDS of (cast X and W under their current scales, GEMM, fused GEMM + cast of
    its output, updates). Returns every output it made, on the current stream."""
    m, n, k = PROBLEMS[idx]
    dev = x.device
    sx, sw = fp8.DelayedScalingState("e4m3", 16, device=dev), fp8.DelayedScalingState("e4m3", 16, device=dev)
    sy = fp8.DelayedScalingState("e4m3", 16, device=dev)
    qx = torch.empty(m, k, dtype=torch.uint8, device=dev)
    qw = torch.empty(n, k, dtype=torch.uint8, device=dev)
    c = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    c2 = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    qy = torch.empty(m, n, dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(ROUNDS):
        sx.cast(x, q=qx)
        sw.cast(w, q=qw)
        fp8.fp8_scaled_gemm(qx, "e4m3", qw, "e4m3", sx.scale_inv, sw.scale_inv, c)
        fp8.fp8_scaled_gemm_amax_cast(qx, "e4m3", qw, "e4m3", sx.scale_inv, sw.scale_inv, c2, "e4m3",
                                      y_scale=sy.scale, y_q=qy, y_amax=sy.amax_slot)
        for s in (sx, sw, sy):
            s.update()
        outs += [qx.clone(), qw.clone(), c.view(torch.int16).clone(), c2.view(torch.int16).clone(), qy.clone(),
                 sx.history.clone(), sw.history.clone(), sy.history.clone(), sx.scale.clone(), sy.scale.clone()]
    return outs


def test_threads_on_their_own_streams_match_one_thread():
    require_gpu()
    banner("concurrency", len(PROBLEMS), "threads")
    inputs = [_inputs(i) for i in range(len(PROBLEMS))]
    torch.cuda.synchronize()
    ref = [_run(i, *inputs[i]) for i in range(len(PROBLEMS))]
    torch.cuda.synchronize()
    ref = [[host(t) for t in outs] for outs in ref]

    got = [None] * len(PROBLEMS)
    errors = []
    start = threading.Barrier(len(PROBLEMS))

    def worker(i):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()   # default priority
            with torch.cuda.stream(s):
                start.wait()
                outs = _run(i, *inputs[i])
            s.synchronize()
            got[i] = [host(t) for t in outs]
        except Exception as e:   # reported below; a thread's exception would otherwise be lost
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(PROBLEMS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(PROBLEMS)):
        assert len(got[i]) == len(ref[i])
        for j, (a, b) in enumerate(zip(got[i], ref[i])):
            a8, b8 = np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8)
            assert np.array_equal(a8, b8), f"problem {PROBLEMS[i]}, output {j}: threads differ from one thread"
