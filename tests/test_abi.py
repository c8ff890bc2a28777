"""The C-ABI library without a GPU: it loads, exports what the header declares, and
rejects bad arguments on the host before touching any device."""
import ctypes
import os
import re

import pytest
import torch

import fp8_mixed_precision_cast_amd as fp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, NO_DEVICE = 0, 1, 2, 3
P = ctypes.c_void_p
A16 = P(4096)   # a fake, 16-byte aligned address; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    return fp8.load_library()


def test_exports_every_declared_symbol(lib):
    names = fp8.exported_symbols()
    assert names == ["fp8_amax_cast", "fp8_amax_cast_batched", "fp8_scale_update", "fp8_scale_update_batched",
                     "fp8_scaled_gemm", "fp8_scaled_gemm_fast_accum",
                     "fp8_scaled_gemm_amax_cast", "fp8_scaled_gemm_amax_cast_fast_accum",
                     "fp8_layernorm_amax_cast", "fp8_reduce_shared_scale", "fp8_adam_step",
                     "fp8_adam_step_weight_cast", "fp8mp_status_string", "fp8mp_device_info"]
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {fp8.lib_path()}").read()
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_status_strings(lib):
    for s in range(6):
        assert fp8.fp8mp_status_string(s)
    assert fp8.fp8mp_status_string(99) == "unknown status"


def test_cast_argument_validation(lib):
    f = lib.fp8_amax_cast
    assert f(None, 1, 4, 4, 4, 0, A16, A16, 4, None, 0, None, None) == INVALID   # x NULL
    assert f(A16, 7, 4, 4, 4, 0, A16, A16, 4, None, 0, None, None) == INVALID    # bad dtype
    assert f(A16, 1, 4, 4, 4, 9, A16, A16, 4, None, 0, None, None) == INVALID    # bad format
    assert f(A16, 1, -1, 4, 4, 0, A16, A16, 4, None, 0, None, None) == INVALID   # negative rows
    assert f(A16, 1, 4, 4, 3, 0, A16, A16, 4, None, 0, None, None) == INVALID    # ld_x < cols
    assert f(A16, 1, 4, 4, 4, 0, None, A16, 4, None, 0, None, None) == INVALID   # q without scale
    assert f(A16, 1, 4, 4, 4, 0, A16, A16, 3, None, 0, None, None) == INVALID    # ld_q < cols
    assert f(A16, 1, 4, 8, 8, 0, A16, None, 0, A16, 3, None, None) == INVALID    # ld_qt < rows
    assert f(P(4097), 1, 4, 4, 4, 0, A16, A16, 4, None, 0, None, None) == INVALID  # misaligned bf16
    # every data pointer starts on a 16-byte boundary
    assert f(P(4096 + 8), 1, 4, 4, 4, 0, A16, A16, 4, None, 0, None, None) == INVALID
    assert f(A16, 1, 4, 4, 4, 0, A16, P(4096 + 4), 4, None, 0, None, None) == INVALID
    assert f(A16, 1, 4, 16, 16, 0, A16, None, 0, P(4096 + 2), 16, None, None) == INVALID
    # a strided (or transposed) BF16 call needs 16-byte row pitches
    assert f(A16, 1, 4, 4, 12, 0, A16, A16, 16, None, 0, None, None) == INVALID  # ld_x of 24 bytes
    assert f(A16, 1, 4, 4, 16, 0, A16, A16, 8, None, 0, None, None) == INVALID   # ld_q of 8 bytes
    assert f(A16, 1, 4, 16, 16, 0, A16, None, 0, A16, 8, None, None) == INVALID  # ld_qt of 8 bytes
    # fp32 sources: contiguous codes only
    assert f(A16, 0, 4, 4, 8, 0, A16, A16, 16, None, 0, None, None) == UNSUPPORTED  # strided fp32
    assert f(A16, 0, 4, 4, 4, 0, A16, None, 0, A16, 16, None, None) == UNSUPPORTED  # fp32 with q_t
    # one row is a contiguous run whatever its leading dimensions
    assert f(A16, 1, 1, 4, 4, 0, None, None, 0, None, 0, None, None) == OK
    assert f(A16, 1, 0, 4, 4, 0, None, None, 0, None, 0, None, None) == OK       # empty
    assert f(A16, 1, 4, 4, 4, 0, None, None, 0, None, 0, None, None) == OK       # nothing requested


def test_scale_update_argument_validation(lib):
    f = lib.fp8_scale_update
    assert f(None, 4, 0, 0, A16, A16, None) == INVALID
    assert f(A16, 0, 0, 0, A16, A16, None) == INVALID
    assert f(A16, 4, 0, -1, A16, A16, None) == INVALID
    assert f(A16, 4, 5, 0, A16, A16, None) == INVALID
    assert f(A16, 4, 0, 0, None, A16, None) == INVALID


def test_batched_cast_validation(lib):
    from fp8_mixed_precision_cast_amd import _CastItem
    f = lib.fp8_amax_cast_batched
    arr = lambda *its: ctypes.cast((_CastItem * len(its))(*its), ctypes.c_void_p)
    good = dict(x=4096, x_dtype=1, numel=64, fmt=0, scale=8192, q=12288, amax=16384)
    item = lambda **kw: _CastItem(**dict(good, **kw))
    assert f(-1, None, None) == INVALID
    assert f(0, None, None) == OK
    assert f(1, None, None) == INVALID
    assert f(1, arr(item(x_dtype=7)), None) == INVALID
    assert f(1, arr(item(fmt=2)), None) == INVALID                 # FP16 storage is not a cast format
    assert f(1, arr(item(numel=-1)), None) == INVALID
    assert f(2, arr(item(), item(x=None)), None) == INVALID       # every item is checked
    assert f(1, arr(item(scale=None)), None) == INVALID           # codes need a scale
    assert f(1, arr(item(x=4097)), None) == INVALID               # misaligned BF16 source
    assert f(1, arr(item(x=4096 + 8)), None) == INVALID           # source not on a 16-byte boundary
    assert f(1, arr(item(q=12288 + 4)), None) == INVALID          # codes not on a 16-byte boundary
    assert f(1, arr(item(x_dtype=0, x=4096 + 4)), None) == INVALID
    assert f(1, arr(item(amax=4098)), None) == INVALID


def test_batched_scale_update_validation(lib):
    f = lib.fp8_scale_update_batched
    n = 2
    ptrs = lambda *v: (ctypes.c_void_p * n)(*v)
    ints = lambda *v: (ctypes.c_int32 * n)(*v)
    fmts = lambda *v: (ctypes.c_int * n)(*v)
    good = dict(h=ptrs(4096, 8192), l=ints(4, 4), f=fmts(0, 1), m=ints(0, 0), s=ptrs(12288, 12292),
                si=ptrs(12296, 12300))
    call = lambda **kw: f(n, *[kw.get(k, good[k]) for k in ("h", "l", "f", "m", "s", "si")], None)
    assert f(-1, None, None, None, None, None, None, None) == INVALID
    assert f(0, None, None, None, None, None, None, None) == OK
    assert call(h=None) == INVALID
    assert call(f=fmts(0, 7)) == INVALID
    assert call(l=ints(4, 0)) == INVALID
    assert call(m=ints(-1, 0)) == INVALID
    assert call(h=ptrs(4096, 0)) == INVALID
    assert call(s=ptrs(12289, 12292)) == INVALID


@pytest.mark.parametrize("name", ["fp8_scaled_gemm", "fp8_scaled_gemm_fast_accum"])
def test_gemm_argument_validation(lib, name):
    f = getattr(lib, name)
    args = lambda **kw: [kw.get("a", A16), kw.get("af", 0), kw.get("lda", 32), kw.get("b", A16), kw.get("bf", 0),
                         kw.get("ldb", 32), kw.get("m", 4), kw.get("n", 8), kw.get("k", 32),
                         kw.get("sa", A16), kw.get("sb", A16), kw.get("c", A16), kw.get("ldc", 8), None]
    assert f(*args(af=3)) == INVALID
    assert f(*args(m=-1)) == INVALID
    assert f(*args(lda=16)) == INVALID
    assert f(*args(ldc=4)) == INVALID
    assert f(*args(c=None)) == INVALID
    assert f(*args(sa=None)) == INVALID
    assert f(*args(k=24, lda=32, ldb=32)) == UNSUPPORTED       # k % 16
    assert f(*args(lda=40)) == INVALID                          # lda not a multiple of 16 bytes
    assert f(*args(ldb=40)) == INVALID
    assert f(*args(a=P(4096 + 8))) == INVALID                   # a not 16-byte aligned
    assert f(*args(b=P(4096 + 1))) == INVALID
    assert f(*args(c=P(4097))) == INVALID                       # c not 2-byte aligned
    assert f(*args(c=P(4096 + 2))) == INVALID                   # c not 16-byte aligned
    assert f(*args(ldc=12)) == INVALID                          # ldc not a multiple of 8 elements
    assert f(*args(m=0)) == OK
    assert f(*args(lda=2**22 + 16)) == UNSUPPORTED              # a tile's rows would pass 32-bit offsets
    assert f(*args(ldb=2**22 + 16)) == UNSUPPORTED


@pytest.mark.parametrize("name", ["fp8_scaled_gemm_amax_cast", "fp8_scaled_gemm_amax_cast_fast_accum"])
def test_fused_gemm_argument_validation(lib, name):
    f = getattr(lib, name)
    args = lambda **kw: [kw.get("a", A16), kw.get("af", 0), kw.get("lda", 32), kw.get("b", A16), kw.get("bf", 0),
                         kw.get("ldb", 32), kw.get("m", 4), kw.get("n", 8), kw.get("k", 32),
                         kw.get("sa", A16), kw.get("sb", A16), kw.get("c", A16), kw.get("ldc", 8),
                         kw.get("yf", 0), kw.get("ys", A16), kw.get("yq", A16), kw.get("ldq", 16),
                         kw.get("ya", A16), None]
    assert f(*args(af=3)) == INVALID                            # the GEMM's own rules apply
    assert f(*args(c=None, yq=None, ya=None)) == INVALID         # c may be NULL only with another output
    assert f(*args(lda=40)) == INVALID
    assert f(*args(k=24, lda=32, ldb=32)) == UNSUPPORTED
    assert f(*args(yq=P(4096 + 8))) == INVALID                 # y_q not 16-byte aligned
    assert f(*args(ldq=24)) == INVALID                          # ld_yq not a multiple of 16
    assert f(*args(yf=2)) == INVALID
    assert f(*args(yf=2, yq=None, ya=None)) == INVALID          # y_fmt checked even without y outputs
    assert f(*args(ys=None)) == INVALID                         # y_q needs a scale
    assert f(*args(ldq=7)) == INVALID                           # ld_yq < n
    assert f(*args(ys=P(4097), yq=None)) == INVALID             # misaligned scale
    assert f(*args(ya=P(4098))) == INVALID                      # misaligned amax
    assert f(*args(m=0)) == OK


def test_layernorm_argument_validation(lib):
    f = lib.fp8_layernorm_amax_cast
    args = lambda **kw: [kw.get("x", A16), kw.get("dt", 1), kw.get("rows", 4), kw.get("cols", 8), kw.get("ldx", 8),
                         kw.get("g", A16), kw.get("b", A16), kw.get("eps", 1e-5), kw.get("y", A16), kw.get("ldy", 8),
                         kw.get("fmt", 0), kw.get("s", A16), kw.get("q", A16), kw.get("ldq", 8), kw.get("am", A16),
                         kw.get("mu", None), kw.get("rs", None), None]
    assert f(*args(dt=5)) == INVALID
    assert f(*args(fmt=7)) == INVALID
    assert f(*args(cols=0)) == INVALID
    assert f(*args(rows=-1)) == INVALID
    assert f(*args(eps=-1.0)) == INVALID
    assert f(*args(eps=float("nan"))) == INVALID
    assert f(*args(eps=float("inf"))) == INVALID
    assert f(*args(x=None)) == INVALID
    assert f(*args(g=None)) == INVALID                           # gamma required
    assert f(*args(ldx=7)) == INVALID
    assert f(*args(ldy=7)) == INVALID
    assert f(*args(s=None)) == INVALID                           # q needs a scale
    assert f(*args(ldq=7)) == INVALID
    assert f(*args(x=P(4097))) == INVALID                        # misaligned bf16
    assert f(*args(dt=0, x=P(4098))) == INVALID                  # misaligned f32
    assert f(*args(g=P(4098))) == INVALID
    assert f(*args(rows=0)) == OK
    assert f(*args(y=None, q=None, am=None)) == OK               # nothing to write


def test_reduce_argument_validation(lib):
    f = lib.fp8_reduce_shared_scale
    args = lambda **kw: [kw.get("q", A16), kw.get("fmt", 1), kw.get("n", 4), kw.get("numel", 64),
                         kw.get("stride", 64), kw.get("si", A16), kw.get("out", A16), kw.get("dt", 1), None]
    assert f(*args(fmt=3)) == INVALID
    assert f(*args(dt=9)) == INVALID
    assert f(*args(n=0)) == INVALID
    assert f(*args(numel=-1)) == INVALID
    assert f(*args(stride=63)) == INVALID                     # ranks would overlap
    assert f(*args(q=None)) == INVALID
    assert f(*args(si=None)) == INVALID
    assert f(*args(out=None)) == INVALID
    assert f(*args(out=P(4097))) == INVALID                   # misaligned BF16 output
    assert f(*args(dt=0, out=P(4098))) == INVALID             # misaligned FP32 output
    assert f(*args(numel=0, stride=0)) == OK


def test_adam_argument_validation(lib):
    f = lib.fp8_adam_step
    B = [P(4096 + 16 * i) for i in range(12)]     # distinct fake aligned addresses
    def args(**kw):
        a = dict(n=64, g=B[0], gd=1, mq=B[1], mdi=B[2], mdo=B[3], ms=B[4], msi=B[5], ma=None, v=B[6], w=B[7],
                 wdi=B[8], wdo=B[9], ws=B[10], wsi=B[11], wa=None, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0,
                 t=7)
        a.update(kw)
        return [a[k] for k in ("n", "g", "gd", "mq", "mdi", "mdo", "ms", "msi", "ma", "v", "w", "wdi", "wdo", "ws",
                               "wsi", "wa", "lr", "b1", "b2", "eps", "wd", "t")] + [None]
    assert f(*args(gd=4)) == INVALID
    assert f(*args(n=-1)) == INVALID
    assert f(*args(g=None)) == INVALID
    assert f(*args(mdo=B[2])) == INVALID                      # dequantisation factor read and written in place
    assert f(*args(wdo=B[8])) == INVALID
    assert f(*args(lr=float("nan"))) == INVALID
    assert f(*args(t=0)) == INVALID                           # step numbers start at 1
    assert f(*args(b1=1.0)) == INVALID                        # 1 - beta^t must not vanish
    assert f(*args(b2=-0.5)) == INVALID
    assert f(*args(b1=float("nan"))) == INVALID
    assert f(*args(v=P(4097))) == INVALID
    assert f(*args(n=0)) == OK
    assert lib.fp8_amax_cast(A16, 1, 4, 4, 4, 2, A16, A16, 4, None, 0, None, None) == INVALID   # not for casts


def _adam_wq_args(B, **kw):
    a = dict(n=64, g=B[0], gd=1, mq=B[1], mdi=B[2], mdo=B[3], ms=B[4], msi=B[5], ma=None, v=B[6], w=B[7],
             wdi=B[8], wdo=B[9], ws=B[10], wsi=B[11], wa=None, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0,
             t=7, qf=0, qs=B[12], q=B[13], qa=B[14])
    a.update(kw)
    return [a[k] for k in ("n", "g", "gd", "mq", "mdi", "mdo", "ms", "msi", "ma", "v", "w", "wdi", "wdo", "ws",
                           "wsi", "wa", "lr", "b1", "b2", "eps", "wd", "t", "qf", "qs", "q", "qa")] + [None]


def test_adam_weight_cast_argument_validation(lib):
    f = lib.fp8_adam_step_weight_cast
    B = [P(4096 + 16 * i) for i in range(15)]
    assert f(*_adam_wq_args(B, gd=4)) == INVALID                  # the Adam step's own checks apply
    assert f(*_adam_wq_args(B, mdo=B[2])) == INVALID
    assert f(*_adam_wq_args(B, qf=2)) == INVALID                  # FP16 is a storage format, not a cast target
    assert f(*_adam_wq_args(B, qf=7)) == INVALID
    assert f(*_adam_wq_args(B, q=None, qa=None)) == INVALID       # nothing to write
    assert f(*_adam_wq_args(B, qs=None)) == INVALID               # codes need the scale
    assert f(*_adam_wq_args(B, qs=P(4098))) == INVALID
    assert f(*_adam_wq_args(B, qa=P(4098))) == INVALID
    assert f(*_adam_wq_args(B, n=0)) == OK
    assert f(*_adam_wq_args(B, n=0, q=None, qs=None)) == OK     # amax only: no scale needed


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a device")
def test_valid_calls_without_device_report_no_device(lib):
    B = [P(4096 + 16 * i) for i in range(15)]
    assert lib.fp8_adam_step_weight_cast(*_adam_wq_args(B)) == NO_DEVICE
    assert lib.fp8_adam_step_weight_cast(*_adam_wq_args(B, qf=1, q=None, qs=None)) == NO_DEVICE
    assert lib.fp8_scale_update(A16, 4, 0, 0, A16, A16, None) == NO_DEVICE
    assert lib.fp8_amax_cast(A16, 1, 4, 4, 4, 0, A16, A16, 4, None, 0, A16, None) == NO_DEVICE
    assert lib.fp8_scaled_gemm(A16, 0, 32, A16, 0, 32, 4, 8, 32, A16, A16, A16, 8, None) == NO_DEVICE
    assert lib.fp8_scaled_gemm_amax_cast(A16, 0, 32, A16, 0, 32, 4, 8, 32, A16, A16, A16, 8, 0, A16, A16, 16, A16,
                                         None) == NO_DEVICE
    assert lib.fp8_scaled_gemm_fast_accum(A16, 0, 32, A16, 0, 32, 4, 8, 32, A16, A16, A16, 8, None) == NO_DEVICE
    assert lib.fp8_scaled_gemm_amax_cast_fast_accum(A16, 0, 32, A16, 0, 32, 4, 8, 32, A16, A16, A16, 8, 0, A16, A16,
                                                    16, A16, None) == NO_DEVICE
    assert lib.fp8_layernorm_amax_cast(A16, 1, 4, 8, 8, A16, None, 1e-5, A16, 8, 0, A16, A16, 8, A16, None, None,
                                       None) == NO_DEVICE
    assert lib.fp8_reduce_shared_scale(A16, 1, 4, 64, 64, A16, A16, 1, None) == NO_DEVICE
    assert lib.fp8_scale_update(A16, 4, 2, 0, A16, A16, None) == NO_DEVICE          # FP16 storage accepted
    one_p, one_i, one_f = (ctypes.c_void_p * 1)(4096), (ctypes.c_int32 * 1)(4), (ctypes.c_int * 1)(2)
    assert lib.fp8_scale_update_batched(1, one_p, one_i, one_f, (ctypes.c_int32 * 1)(0), one_p, one_p,
                                        None) == NO_DEVICE
    # k == 0 with zero leading dimensions passes the host checks (no division by a zero ld)
    assert lib.fp8_scaled_gemm(A16, 0, 0, A16, 0, 0, 4, 8, 0, A16, A16, A16, 8, None) == NO_DEVICE
    buf = ctypes.create_string_buffer(64)
    assert lib.fp8mp_device_info(buf, 64) == NO_DEVICE


def test_binding_has_no_cpu_fallback():
    """The binding's entry points go through the library only."""
    import inspect
    src = inspect.getsource(fp8)
    assert "oracle" not in src and "numpy" not in src
