"""Python binding of libfp8mp: the per-tensor-scaled FP8 linear layer on gfx950.

Argument marshalling only. Every step of the path runs in the HIP library
(``libfp8mp.so``, built in-tree by ``fp8_mixed_precision_cast_amd.build``);
torch supplies device memory and the current stream. The functions carry the
C-ABI names and raise ``Fp8mpError`` on any non-OK status. There is no CPU
fallback: without the built library, importing the binding's entry points
raises.

Tensors:
  * sources: 2-D float32 or bfloat16 (or int16/uint16 BF16 bit patterns), unit
    column stride; the row stride is the leading dimension;
  * FP8 codes: uint8 tensors; scales, inverse scales and amax: float32 tensors
    (their first element is used; a history's first element is its amax slot);
  * GEMM output: bfloat16 (or int16/uint16) tensor.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

__all__ = [
    "E4M3", "E5M2", "F32", "BF16", "Fp8mpError", "lib_path", "load_library",
    "fp8_amax_cast", "fp8_amax_cast_batched", "CastBatch", "fp8_scale_update", "fp8_scale_update_batched", "ScaleUpdateBatch", "fp8_scaled_gemm", "fp8_scaled_gemm_fast_accum", "fp8_scaled_gemm_amax_cast", "fp8_scaled_gemm_amax_cast_fast_accum", "fp8_layernorm_amax_cast", "fp8_reduce_shared_scale", "fp8_adam_step", "AdamFP8State",
    "fp8mp_status_string",
    "fp8mp_device_info", "exported_symbols", "DelayedScalingState", "CurrentScalingState",
]

E4M3, E5M2, FP16 = 0, 1, 2
F32, BF16 = 0, 1
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2, "fp16": FP16, FP16: FP16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_lib = None


class Fp8mpError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {fp8mp_status_string(status)} (status {status})")


def lib_path() -> str:
    return os.path.join(_HERE, "libfp8mp.so")


def load_library() -> ctypes.CDLL:
    """Load libfp8mp.so from this package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp8_mixed_precision_cast_amd.build`")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.fp8_amax_cast.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, vp, vp, i64, vp, i64, vp, vp]
    lib.fp8_amax_cast.restype = ctypes.c_int
    lib.fp8_amax_cast_batched.argtypes = [i32, vp, vp]
    lib.fp8_amax_cast_batched.restype = ctypes.c_int
    lib.fp8_scale_update.argtypes = [vp, i32, ctypes.c_int, i32, vp, vp, vp]
    lib.fp8_scale_update.restype = ctypes.c_int
    lib.fp8_scale_update_batched.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fp8_scale_update_batched.restype = ctypes.c_int
    for name in ("fp8_scaled_gemm", "fp8_scaled_gemm_fast_accum"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, ctypes.c_int, i64, vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, i64, vp]
        fn.restype = ctypes.c_int
    for name in ("fp8_scaled_gemm_amax_cast", "fp8_scaled_gemm_amax_cast_fast_accum"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, ctypes.c_int, i64, vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, i64, ctypes.c_int,
                       vp, vp, i64, vp, vp]
        fn.restype = ctypes.c_int
    lib.fp8_layernorm_amax_cast.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, ctypes.c_float, vp, i64,
                                            ctypes.c_int, vp, vp, i64, vp, vp, vp, vp]
    lib.fp8_layernorm_amax_cast.restype = ctypes.c_int
    lib.fp8_reduce_shared_scale.argtypes = [vp, ctypes.c_int, i32, i64, i64, vp, vp, ctypes.c_int, vp]
    lib.fp8_reduce_shared_scale.restype = ctypes.c_int
    fl = ctypes.c_float
    lib.fp8_adam_step.argtypes = [i64, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  fl, fl, fl, fl, fl, i64, vp]
    lib.fp8_adam_step.restype = ctypes.c_int
    lib.fp8_adam_step_weight_cast.argtypes = [i64, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp, fl, fl, fl, fl, fl, i64, ctypes.c_int, vp, vp, vp, vp]
    lib.fp8_adam_step_weight_cast.restype = ctypes.c_int
    lib.fp8mp_status_string.argtypes = [ctypes.c_int]
    lib.fp8mp_status_string.restype = ctypes.c_char_p
    lib.fp8mp_device_info.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
    lib.fp8mp_device_info.restype = ctypes.c_int
    _lib = lib
    return lib


def exported_symbols() -> list:
    """Function names declared in include/fp8mp.h."""
    with open(os.path.join(_ROOT, "include", "fp8mp.h")) as f:
        text = f.read()
    return re.findall(r"^\s*(?:fp8mp_status|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def fp8mp_status_string(status: int) -> str:
    return load_library().fp8mp_status_string(int(status)).decode()


def fp8mp_device_info() -> str:
    buf = ctypes.create_string_buffer(256)
    st = load_library().fp8mp_device_info(buf, 256)
    if st != 0:
        raise Fp8mpError(st, "fp8mp_device_info")
    return buf.value.decode()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(st: int, call: str) -> None:
    if st != 0:
        raise Fp8mpError(st, call)


def _src_dtype(x) -> int:
    import torch
    if x.dtype == torch.float32:
        return F32
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise TypeError(f"source dtype {x.dtype} is not float32 or bfloat16")


def _rows_ld(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.shape[0], t.shape[1], max(t.stride(0), t.shape[1])


def fp8_amax_cast(x, fmt, scale=None, q=None, q_t=None, amax=None, stream=None) -> None:
    """One pass over x: *amax = max(*amax, max|x|), q = enc(x*scale), q_t = q^T."""
    rows, cols, ld_x = _rows_ld(x, "x")
    ld_q = _rows_ld(q, "q")[2] if q is not None else 0
    ld_qt = _rows_ld(q_t, "q_t")[2] if q_t is not None else 0
    if q is not None and tuple(q.shape) != (rows, cols):
        raise ValueError("q must be rows x cols")
    if q_t is not None and tuple(q_t.shape) != (cols, rows):
        raise ValueError("q_t must be cols x rows")
    st = load_library().fp8_amax_cast(_ptr(x), _src_dtype(x), rows, cols, ld_x, FORMATS[fmt], _ptr(scale),
                                      _ptr(q), ld_q, _ptr(q_t), ld_qt, _ptr(amax), _stream(stream))
    _check(st, "fp8_amax_cast")


class _CastItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("numel", ctypes.c_int64), ("fmt", ctypes.c_int),
                ("scale", ctypes.c_void_p), ("q", ctypes.c_void_p), ("amax", ctypes.c_void_p)]


class CastBatch:
    """The host-side item array of fp8_amax_cast_batched for fixed tensors, built once.

    items: (x, fmt, scale, q, amax) with x contiguous float32/bfloat16, q a contiguous uint8 tensor of
    x's size or None, amax a float32 tensor or None."""

    def __init__(self, items):
        self._keep = list(items)
        arr = (_CastItem * len(items))()
        for k, (x, fmt, scale, q, amax) in enumerate(items):
            if not x.is_contiguous() or (q is not None and (not q.is_contiguous() or q.numel() != x.numel())):
                raise ValueError("batched casts take contiguous tensors of equal size")
            arr[k] = _CastItem(x.data_ptr(), _src_dtype(x), x.numel(), FORMATS[fmt], _ptr(scale), _ptr(q), _ptr(amax))
        self.n = len(items)
        self.items = arr


def fp8_amax_cast_batched(batch, stream=None) -> None:
    """fp8_amax_cast of every item of a CastBatch (or a list of items), one launch per 8 BF16 tensors."""
    if not isinstance(batch, CastBatch):
        batch = CastBatch(batch)
    st = load_library().fp8_amax_cast_batched(batch.n, ctypes.cast(batch.items, ctypes.c_void_p), _stream(stream))
    _check(st, "fp8_amax_cast_batched")


def fp8_scale_update(history, fmt, margin, scale, scale_inv, stream=None) -> None:
    """Delayed-scaling update of (scale, scale_inv) from history, then roll the history."""
    st = load_library().fp8_scale_update(_ptr(history), int(history.numel()), FORMATS[fmt], int(margin),
                                         _ptr(scale), _ptr(scale_inv), _stream(stream))
    _check(st, "fp8_scale_update")


class ScaleUpdateBatch:
    """The host-side argument arrays of fp8_scale_update_batched for a fixed list of recipe states
    (objects with history, fmt, margin, scale, scale_inv), built once."""

    def __init__(self, states):
        n = len(states)
        self.n = n
        self._keep = list(states)
        self.hist = (ctypes.c_void_p * n)(*[st.history.data_ptr() for st in states])
        self.lens = (ctypes.c_int32 * n)(*[int(st.history.numel()) for st in states])
        self.fmts = (ctypes.c_int * n)(*[int(st.fmt) for st in states])
        self.margins = (ctypes.c_int32 * n)(*[int(st.margin) for st in states])
        self.scales = (ctypes.c_void_p * n)(*[st.scale.data_ptr() for st in states])
        self.scale_invs = (ctypes.c_void_p * n)(*[st.scale_inv.data_ptr() for st in states])


def fp8_scale_update_batched(batch, stream=None) -> None:
    """fp8_scale_update for every state of a ScaleUpdateBatch (or a list of states), in one launch per 16."""
    if not isinstance(batch, ScaleUpdateBatch):
        batch = ScaleUpdateBatch(batch)
    st = load_library().fp8_scale_update_batched(batch.n, batch.hist, batch.lens, batch.fmts, batch.margins,
                                                 batch.scales, batch.scale_invs, _stream(stream))
    _check(st, "fp8_scale_update_batched")


def _gemm(call, a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, stream) -> None:
    m, k, lda = _rows_ld(a, "a")
    n, kb, ldb = _rows_ld(b, "b")
    if kb != k:
        raise ValueError("a and b must share k")
    mc, nc, ldc = _rows_ld(c, "c")
    if (mc, nc) != (m, n):
        raise ValueError("c must be m x n")
    st = getattr(load_library(), call)(_ptr(a), FORMATS[a_fmt], lda, _ptr(b), FORMATS[b_fmt], ldb, m, n, k,
                                       _ptr(a_scale_inv), _ptr(b_scale_inv), _ptr(c), ldc, _stream(stream))
    _check(st, call)


def fp8_scaled_gemm(a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, stream=None) -> None:
    """c = (a . b^T) * a_scale_inv * b_scale_inv; a[m,k], b[n,k] uint8 codes; c[m,n] BF16; FP32 accumulation."""
    _gemm("fp8_scaled_gemm", a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, stream)


def fp8_scaled_gemm_fast_accum(a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, stream=None) -> None:
    """fp8_scaled_gemm on the FP8 MFMA's reduced-precision accumulation (within 2^-9 of sum|a*b|)."""
    _gemm("fp8_scaled_gemm_fast_accum", a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, stream)


def _gemm_amax_cast(call, a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, y_fmt, y_scale, y_q, y_amax,
                    stream) -> None:
    m, k, lda = _rows_ld(a, "a")
    n, kb, ldb = _rows_ld(b, "b")
    if kb != k:
        raise ValueError("a and b must share k")
    ldc = 0
    if c is not None:
        mc, nc, ldc = _rows_ld(c, "c")
        if (mc, nc) != (m, n):
            raise ValueError("c must be m x n")
    ld_yq = 0
    if y_q is not None:
        mq, nq, ld_yq = _rows_ld(y_q, "y_q")
        if (mq, nq) != (m, n):
            raise ValueError("y_q must be m x n")
    st = getattr(load_library(), call)(
        _ptr(a), FORMATS[a_fmt], lda, _ptr(b), FORMATS[b_fmt], ldb, m, n, k, _ptr(a_scale_inv), _ptr(b_scale_inv),
        _ptr(c), ldc, FORMATS[y_fmt], _ptr(y_scale), _ptr(y_q), ld_yq, _ptr(y_amax), _stream(stream))
    _check(st, call)


def fp8_scaled_gemm_amax_cast(a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, y_fmt, y_scale=None, y_q=None,
                              y_amax=None, stream=None) -> None:
    """fp8_scaled_gemm, and in the same kernel y_amax = max(y_amax, max|c|), y_q = enc(c * y_scale);
    c may be None when y_q or y_amax is given (the BF16 output is then not stored)."""
    _gemm_amax_cast("fp8_scaled_gemm_amax_cast", a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, y_fmt, y_scale,
                    y_q, y_amax, stream)


def fp8_scaled_gemm_amax_cast_fast_accum(a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, y_fmt, y_scale=None,
                                         y_q=None, y_amax=None, stream=None) -> None:
    """fp8_scaled_gemm_amax_cast on the FP8 MFMA's reduced-precision accumulation."""
    _gemm_amax_cast("fp8_scaled_gemm_amax_cast_fast_accum", a, a_fmt, b, b_fmt, a_scale_inv, b_scale_inv, c, y_fmt,
                    y_scale, y_q, y_amax, stream)


def fp8_layernorm_amax_cast(x, gamma, beta, eps, fmt, y=None, scale=None, q=None, amax=None, mean=None, rstd=None,
                            stream=None) -> None:
    """y = LayerNorm(x) * gamma + beta in BF16; in the same pass amax = max(amax, max|y|), q = enc(y * scale)."""
    rows, cols, ld_x = _rows_ld(x, "x")
    ld_y = ld_q = 0
    if y is not None:
        ry, cy, ld_y = _rows_ld(y, "y")
        if (ry, cy) != (rows, cols):
            raise ValueError("y must be rows x cols")
    if q is not None:
        rq, cq, ld_q = _rows_ld(q, "q")
        if (rq, cq) != (rows, cols):
            raise ValueError("q must be rows x cols")
    st = load_library().fp8_layernorm_amax_cast(
        _ptr(x), _src_dtype(x), rows, cols, ld_x, _ptr(gamma), _ptr(beta), float(eps), _ptr(y), ld_y, FORMATS[fmt],
        _ptr(scale), _ptr(q), ld_q, _ptr(amax), _ptr(mean), _ptr(rstd), _stream(stream))
    _check(st, "fp8_layernorm_amax_cast")


def fp8_reduce_shared_scale(q, fmt, scale_inv, out, stream=None) -> None:
    """out = (sum over the leading dimension of dec(q)) * scale_inv; q is [ranks, numel] uint8 (row stride
    is the rank stride), out a contiguous float32 or bfloat16 tensor of numel elements."""
    if q.dim() != 2 or (q.shape[1] > 1 and q.stride(1) != 1):
        raise ValueError("q must be [ranks, numel] with unit element stride")
    n_ranks, numel = q.shape
    if out.numel() != numel or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of numel elements")
    st = load_library().fp8_reduce_shared_scale(_ptr(q), FORMATS[fmt], int(n_ranks), int(numel),
                                                int(max(q.stride(0), numel)), _ptr(scale_inv), _ptr(out),
                                                _src_dtype(out), _stream(stream))
    _check(st, "fp8_reduce_shared_scale")


def fp8_adam_step(grad, m_q, m_dq_in, m_dq_out, m_scale, m_scale_inv, m_amax, v, w, w_dq_in, w_dq_out, w_scale,
                  w_scale_inv, w_amax, lr, beta1, beta2, eps, weight_decay, step, stream=None,
                  wq=None, wq_fmt="e4m3", wq_scale=None, wq_amax=None) -> None:
    """Adam step number `step` (1, 2, ...) over FP8 m (codes), FP16 v and tensor-scaled FP16 w (all
    updated in place); the library forms the bias corrections from beta1, beta2 and step.

    With wq and/or wq_amax (fp8_adam_step_weight_cast): also wq = enc(W * wq_scale) and
    wq_amax = max(wq_amax, max |W|) for the stored master weights W = fp16 w * w_scale_inv."""
    n = grad.numel()
    for t, name in ((m_q, "m_q"), (v, "v"), (w, "w")) + (((wq, "wq"),) if wq is not None else ()):
        if t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with as many elements as grad")
    if not grad.is_contiguous():
        raise ValueError("grad must be contiguous")
    args = (n, _ptr(grad), _src_dtype(grad), _ptr(m_q), _ptr(m_dq_in), _ptr(m_dq_out), _ptr(m_scale),
            _ptr(m_scale_inv), _ptr(m_amax), _ptr(v), _ptr(w), _ptr(w_dq_in), _ptr(w_dq_out), _ptr(w_scale),
            _ptr(w_scale_inv), _ptr(w_amax), float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
            int(step))
    if wq is None and wq_amax is None:
        _check(load_library().fp8_adam_step(*args, _stream(stream)), "fp8_adam_step")
    else:
        st = load_library().fp8_adam_step_weight_cast(*args, FORMATS[wq_fmt], _ptr(wq_scale), _ptr(wq), _ptr(wq_amax),
                                                      _stream(stream))
        _check(st, "fp8_adam_step_weight_cast")


class AdamFP8State:
    """Adam state with decoupled precisions: m as E4M3 codes, v as FP16, master w as tensor-scaled FP16.

    Both scales follow the delayed recipe (histories of history_len, margin).
    The dequantisation factors of the stored m and w alternate between two
    device floats (the step reads one and writes the other). Cold start: m = 0,
    v = 0, scales 1, w stored with scale 1.
    """

    def __init__(self, w0, history_len: int = 16, margin: int = 0, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                 weight_decay=0.0, weight_codes: Optional[str] = None, weight_history_len: int = 1024):
        """weight_codes ("e4m3" or "e5m2"): every step also writes self.wq, the codes of the updated
        master weights for the next forward, under their own delayed scaling (self.wq_state)."""
        import torch
        dev = w0.device
        self.n = w0.numel()
        self.hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
        self.t = 0
        self.m_q = torch.zeros(self.n, dtype=torch.uint8, device=dev)
        self.v = torch.zeros(self.n, dtype=torch.float16, device=dev)
        self.w = w0.detach().reshape(-1).to(torch.float16).clone()
        self.m_state = DelayedScalingState("e4m3", history_len, margin, dev)
        self.w_state = DelayedScalingState("fp16", history_len, margin, dev)
        self.m_dq = torch.ones(2, dtype=torch.float32, device=dev)
        self.w_dq = torch.ones(2, dtype=torch.float32, device=dev)
        self.cur = 0
        self.wq = self.wq_state = None
        if weight_codes is not None:
            self.wq = torch.zeros(self.n, dtype=torch.uint8, device=dev)
            self.wq_state = DelayedScalingState(weight_codes, weight_history_len, margin, dev)

    def step(self, grad, stream=None) -> None:
        self.t += 1
        b1, b2 = self.hp["beta1"], self.hp["beta2"]
        i, o = self.cur, 1 - self.cur
        ms, ws = self.m_state, self.w_state
        qs = self.wq_state
        fp8_adam_step(grad.reshape(-1), self.m_q, self.m_dq[i:i + 1], self.m_dq[o:o + 1], ms.scale, ms.scale_inv,
                      ms.amax_slot, self.v, self.w, self.w_dq[i:i + 1], self.w_dq[o:o + 1], ws.scale, ws.scale_inv,
                      ws.amax_slot, self.hp["lr"], b1, b2, self.hp["eps"], self.hp["weight_decay"], self.t, stream,
                      wq=self.wq, wq_fmt=qs.fmt if qs else "e4m3", wq_scale=qs.scale if qs else None,
                      wq_amax=qs.amax_slot if qs else None)
        ms.update(stream)
        ws.update(stream)
        if qs is not None:
            qs.update(stream)
        self.cur = o

    def master_weights(self):
        """The master weights as float32 (decoded FP16 times the current dequantisation factor)."""
        return self.w.float() * self.w_dq[self.cur]


class DelayedScalingState:
    """Device buffers of one tensor's recipe state: history[L], scale, scale_inv.

    Cold start: history 0, scale 1, scale_inv 1. ``state_dict``/``load_state_dict``
    copy the three buffers (the checkpointable FP8 state).
    """

    def __init__(self, fmt, history_len: int = 1024, margin: int = 0, device="cuda"):
        import torch
        self.fmt = FORMATS[fmt]
        self.margin = int(margin)
        self.history = torch.zeros(history_len, dtype=torch.float32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=device)

    @property
    def amax_slot(self):
        return self.history[0:1]

    def cast(self, x, q=None, q_t=None, record: bool = True, stream=None) -> None:
        fp8_amax_cast(x, self.fmt, self.scale, q, q_t, self.amax_slot if record else None, stream)

    def update(self, stream=None) -> None:
        fp8_scale_update(self.history, self.fmt, self.margin, self.scale, self.scale_inv, stream)

    def state_dict(self):
        return {"amax_history": self.history.clone(), "scale": self.scale.clone(),
                "scale_inv": self.scale_inv.clone()}

    def load_state_dict(self, sd) -> None:
        self.history.copy_(sd["amax_history"])
        self.scale.copy_(sd["scale"])
        self.scale_inv.copy_(sd["scale_inv"])


class CurrentScalingState:
    """Just-in-time (current) per-tensor scaling through the same three calls.

    [MPT] §横断的知見 "テンソルスケーリングが FP8 実用化の鍵" names just-in-time per-tensor
    scaling beside delayed scaling: the scale comes from the tensor's own amax
    in the same step. Here that is an amax-only pass into a one-entry history,
    the update (scale = fmax / amax / 2**margin, same hold rules; the entry is
    reset to 0), then the cast with the fresh scale: two reads of the source
    instead of one.
    """

    def __init__(self, fmt, margin: int = 0, device="cuda"):
        import torch
        self.fmt = FORMATS[fmt]
        self.margin = int(margin)
        self.slot = torch.zeros(1, dtype=torch.float32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=device)

    def cast(self, x, q=None, q_t=None, stream=None) -> None:
        fp8_amax_cast(x, self.fmt, None, None, None, self.slot, stream)
        fp8_scale_update(self.slot, self.fmt, self.margin, self.scale, self.scale_inv, stream)
        fp8_amax_cast(x, self.fmt, self.scale, q, q_t, None, stream)
