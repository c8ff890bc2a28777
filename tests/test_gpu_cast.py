"""GPU parity of fp8_amax_cast against the oracle: codes and amax bit for bit.

Exhaustive over all 65536 BF16 inputs at a set of scales, structured fp32
sweeps around every rounding boundary, special values, and every layout path
(flat with a ragged tail, 2-D tiles with ragged edges, strided views,
transposed copy, amax only, empty), and the refusal of layouts the kernels do
not take (misaligned starts or row pitches, strided or transposed fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle.codec import FMT, decode_table
from tests.gpu_util import banner, dev, f32, f32_bits, first_diff, host, pitched, require_gpu

import fp8_mixed_precision_cast_amd as fp8

pytestmark = pytest.mark.gpu

FORMATS = ["e4m3", "e5m2"]


def _amax_bits(a) -> int:
    return int(np.array([a], dtype=np.float32).view(np.uint32)[0])


def _run_cast(x_np, dtype, fmt, scale, with_q=True, with_qt=False, amax0=0.0):
    """Contiguous source and codes (the flat kernels); with the transposed copy, a BF16 source and code
    buffers with 16-byte row pitches (the tile kernel)."""
    rows, cols = x_np.shape
    if with_qt:
        xd, _ = pitched(rows, cols, torch.int16)
        xd.copy_(dev(x_np))
        q = pitched(rows, cols, torch.uint8)[0] if with_q else None
        qt = pitched(cols, rows, torch.uint8)[0]
    else:
        xd = dev(x_np)
        q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda") if with_q else None
        qt = None
    am = f32(amax0)
    fp8.fp8_amax_cast(xd, fmt, f32(scale), q, qt, am)
    return (host(q) if with_q else None), (host(qt) if with_qt else None), f32_bits(am)[0]


SCALES = [1.0, 2.0 ** -20, 2.0 ** 20, 448.0 / 3.0, 0.7, 1.0e-30, 3.0e30, 2.0 ** -126, 57344.0 / 11.0,
          float(np.float32(448.0) / np.float32(6.5e4))]


@pytest.mark.parametrize("fmt", FORMATS)
def test_all_bf16_patterns_at_many_scales(fmt):
    require_gpu()
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    for s in SCALES:
        banner("all-bf16", fmt, s)
        q, _, am = _run_cast(x, "bf16", fmt, s)
        want = oracle.cast(x, np.float32(s), fmt, "bf16")
        assert np.array_equal(q, want), f"scale {s}: {first_diff(q, want)}"
        assert am == 0x7FC00000   # the patterns include NaNs


@pytest.mark.parametrize("fmt", FORMATS)
def test_zero_infinite_and_nan_scales_without_nan_sources(fmt):
    """Every BF16 pattern except the NaNs (so no source forces the NaN checks), at scales for which
    0 * Inf or a NaN scale makes some products NaN: 0 * Inf and Inf * 0 give the NaN code with the
    product's sign, and a NaN scale gives it for every element. The cast may skip its NaN checks only
    when the scale is finite and nonzero; here every product has to take them."""
    require_gpu()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[(pats & 0x7FFF) <= 0x7F80]                       # no NaN sources
    x = np.zeros(256 * 256, dtype=np.uint16)
    x[: pats.size] = pats
    x = x.reshape(256, 256)
    for s in (0.0, -0.0, float("inf"), float("-inf"), float("nan"), 1.5):
        banner("no-NaN sources", fmt, s)
        q, _, am = _run_cast(x, "bf16", fmt, s)
        want = oracle.cast(x, np.float32(s), fmt, "bf16")
        assert np.array_equal(q, want), f"scale {s}: {first_diff(q, want)}"
        assert am == 0x7F800000   # the sources' magnitude max is Inf


def _boundary_f32(fmt):
    """fp32 values at, just above and just below every rounding boundary of the format."""
    t = decode_table(fmt)
    top = FMT[fmt].max_code
    vals = t[: top + 1]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    sat = np.float32(vals[-1] + (vals[-1] - vals[-2]) / 2)      # tie between the top and the next binade
    pts = np.concatenate([vals.astype(np.float32), mids, [sat]])
    out = [pts]
    up, dn = pts.copy(), pts.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up, dn]
    v = np.concatenate(out).astype(np.float32)
    return np.concatenate([v, -v])


def _specials():
    b = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF, 0x7F800000, 0xFF800000, 0x00000000,
                  0x80000000, 0x00000001, 0x807FFFFF, 0x00800000, 0x7F7FFFFF, 0xFF7FFFFF], dtype=np.uint32)
    return b.view(np.float32)


@pytest.mark.parametrize("fmt", FORMATS)
def test_fp32_rounding_boundaries_and_specials(fmt):
    require_gpu()
    rng = np.random.default_rng(11)
    rand_bits = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([_boundary_f32(fmt), _specials(), rand_bits])
    pad = (-v.size) % 1024
    v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, 1024)
    for s in (1.0, 0.5, 3.0):
        banner("fp32-boundaries", fmt, s)
        q, _, am = _run_cast(v, "f32", fmt, s)
        want = oracle.cast(v, np.float32(s), fmt, "f32")
        assert np.array_equal(q, want), f"scale {s}: {first_diff(q, want)}"
        assert am == 0x7FC00000


@pytest.mark.parametrize("fmt", FORMATS)
def test_scaled_boundaries_hit_exact_ties(fmt):
    """x * s lands exactly on FP8 midpoints for power-of-two scales."""
    require_gpu()
    v = _boundary_f32(fmt)
    v = np.concatenate([v, np.zeros((-v.size) % 256, np.float32)]).reshape(-1, 256)
    for k in (-8, -3, 5, 9):
        s = 2.0 ** k
        x = (v * np.float32(2.0 ** -k)).astype(np.float32)
        banner("pow2-ties", fmt, k)
        q, _, _ = _run_cast(x, "f32", fmt, s)
        want = oracle.cast(x, np.float32(s), fmt, "f32")
        assert np.array_equal(q, want), first_diff(q, want)


def _bf16_matrix(rows, cols, seed, std=1.0):
    return wl.small_normal(seed, (rows, cols), std=std, outlier_factor=20.0)


LAYOUT_SHAPES = [(1, 1), (1, 17), (3, 5), (16, 16), (33, 100), (256, 64), (300, 200), (257, 129),
                 (512, 1024), (1000, 77), (64, 4097)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", LAYOUT_SHAPES)
def test_layouts_with_transpose(fmt, shape):
    require_gpu()
    rows, cols = shape
    x = _bf16_matrix(rows, cols, rows * 7919 + cols)
    s = float(oracle.primed_scale(x, fmt, "bf16").scale)
    banner("layout", fmt, shape)
    q, qt, am = _run_cast(x, "bf16", fmt, s, with_q=True, with_qt=True)
    want = oracle.cast(x, np.float32(s), fmt, "bf16")
    assert np.array_equal(q, want), first_diff(q, want)
    assert np.array_equal(qt, want.T), first_diff(qt, want.T)
    assert am == _amax_bits(oracle.amax(x, "bf16"))
    # transposed copy only, and q only through the tile path
    banner("layout-qt-only", fmt, shape)
    _, qt2, am2 = _run_cast(x, "bf16", fmt, s, with_q=False, with_qt=True)
    assert np.array_equal(qt2, want.T) and am2 == am


@pytest.mark.parametrize("fmt", FORMATS)
def test_strided_views(fmt):
    require_gpu()
    base = _bf16_matrix(130, 320, 5)
    xd_full = dev(base)
    s = 3.5
    # (rows, cols of the source view): every view starts on a 16-byte boundary, rows 640 bytes apart
    cases = {
        "row-slice": (slice(1, 129), slice(0, 320)),                 # contiguous rows, offset start
        "strided-vector": (slice(0, 128), slice(0, 256)),            # ld 320, full tiles
        "strided-ragged": (slice(2, 130), slice(64, 300)),           # ld 320, ragged right and bottom edges
    }
    for name, (rs, cs) in cases.items():
        banner("strided", fmt, name)
        xv = xd_full[rs, cs]
        rows, cols = xv.shape
        q, q_store = pitched(rows, cols, torch.uint8, fill=0x5A, pad_bytes=16)
        qt, _ = pitched(cols, rows, torch.uint8)
        am = f32(0.0)
        fp8.fp8_amax_cast(xv, fmt, f32(s), q, qt, am)
        xh = base[rs, cs]
        want = oracle.cast(xh, np.float32(s), fmt, "bf16")
        assert np.array_equal(host(q), want), first_diff(host(q), want)
        assert np.array_equal(host(qt), want.T)
        assert f32_bits(am)[0] == _amax_bits(oracle.amax(xh, "bf16"))
        assert (host(q_store)[:, cols:] == 0x5A).all(), "wrote past cols"
        # the same view cast without the transposed copy (tile path, q only)
        q2, _ = pitched(rows, cols, torch.uint8)
        fp8.fp8_amax_cast(xv, fmt, f32(s), q2, None, None)
        assert np.array_equal(host(q2), want)


def test_layouts_the_kernels_do_not_take_are_refused():
    """Starts or row pitches that are not multiples of 16 bytes are invalid arguments; fp32 sources
    that are strided or need the transposed copy are unsupported. Nothing is written."""
    require_gpu()
    base = dev(_bf16_matrix(130, 320, 5))
    q, _ = pitched(130, 200, torch.uint8, fill=0x5A)
    qt, _ = pitched(200, 130, torch.uint8, fill=0x5A)
    f32src = torch.zeros(64, 64, dtype=torch.float32, device="cuda")
    cases = {
        "source start not 16-byte aligned": (base[:, 3:203], q, qt, 1),
        "source rows 2 elements apart from 16-byte": (torch.zeros(130, 204, dtype=torch.int16, device="cuda")[:, :200],
                                                      q, qt, 1),
        "codes start not 16-byte aligned": (base[:, :200], torch.zeros(130, 216, dtype=torch.uint8,
                                                                       device="cuda")[:, 8:208], None, 1),
        "codes pitch not a multiple of 16": (base[:, :200], torch.zeros(130, 200, dtype=torch.uint8, device="cuda"),
                                             None, 1),
        "transposed codes pitch not a multiple of 16": (base[:, :200], None,
                                                        torch.zeros(200, 130, dtype=torch.uint8, device="cuda"), 1),
        "fp32 with a transposed copy": (f32src, None, torch.zeros(64, 64, dtype=torch.uint8, device="cuda"), 2),
        "strided fp32": (torch.zeros(64, 128, dtype=torch.float32, device="cuda")[:, :64],
                         torch.zeros(64, 64, dtype=torch.uint8, device="cuda"), None, 2),
    }
    for name, (x, qq, qqt, status) in cases.items():
        banner("refused", name)
        am = f32(0.0)
        with pytest.raises(fp8.Fp8mpError) as ei:
            fp8.fp8_amax_cast(x, "e4m3", f32(1.0), qq, qqt, am)
        assert ei.value.status == status, name
        assert f32_bits(am)[0] == 0, name
    assert (host(q) == 0x5A).all() and (host(qt) == 0x5A).all()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_flat_ragged_tail_amax_only_and_accumulate(fmt, dtype):
    require_gpu()
    rng = np.random.default_rng(21)
    for numel in (1, 15, 16, 17, 4096 + 13, 100003):
        x32 = (rng.standard_normal(numel) * 5).astype(np.float32)
        x = wl.f32_to_bf16_bits(x32) if dtype == "bf16" else x32
        x = x.reshape(1, numel)
        s = 13.0
        banner("flat", fmt, dtype, numel)
        q, _, am = _run_cast(x, dtype, fmt, s)
        want = oracle.cast(x, np.float32(s), fmt, dtype)
        assert np.array_equal(q, want), first_diff(q, want)
        a = oracle.amax(x, dtype)
        assert am == _amax_bits(a)
        # amax only, folded into a larger previous value and into a smaller one
        xd = dev(x)
        for prev in (0.0, float(a) * 2, float(a) / 2):
            amd = f32(prev)
            fp8.fp8_amax_cast(xd, fmt, None, None, None, amd)
            assert f32_bits(amd)[0] == _amax_bits(max(np.float32(prev), a))


def test_empty_and_nan_amax():
    require_gpu()
    banner("empty")
    x = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda")
    am = f32(1.5)
    fp8.fp8_amax_cast(x, "e4m3", f32(1.0), torch.empty(0, 16, dtype=torch.uint8, device="cuda"), None, am)
    assert f32_bits(am)[0] == _amax_bits(np.float32(1.5))
    banner("nan-amax")
    v = np.ones((64, 64), np.float32)
    v[17, 3] = np.array([0xFF812345], np.uint32).view(np.float32)[0]   # negative NaN with payload
    q, _, am = _run_cast(v, "f32", "e4m3", 1.0, amax0=2.0)
    assert am == 0x7FC00000
    assert q[17, 3] == 0xFF
    # a NaN already in the slot stays the canonical NaN
    am2 = torch.tensor([np.array([0x7FC00000], np.uint32).view(np.float32)[0]], device="cuda")
    fp8.fp8_amax_cast(dev(np.ones((4, 4), np.float32)), "e4m3", None, None, None, am2)
    assert f32_bits(am2)[0] == 0x7FC00000


def test_invalid_arguments_raise():
    require_gpu()
    x = torch.zeros(4, 4, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp8.Fp8mpError):
        fp8.fp8_amax_cast(x, "e4m3", None, torch.empty(4, 4, dtype=torch.uint8, device="cuda"))


def test_batched_cast_equals_separate_calls():
    """fp8_amax_cast_batched over 11 items (two batched launches plus the fp32 source's own kernel): BF16
    with ragged tails, amax-only and codes-only items, an empty one; codes and amax bit-identical to the
    oracle. An item whose source or codes do not start on a 16-byte boundary makes the whole call an
    invalid argument, refused before anything runs."""
    require_gpu()
    import workloads as wl
    rng = np.random.default_rng(77)
    sizes = [16, 17, 1000, 4099, 65536, 300001, 5, 12345, 7, 0, 2048]
    items, refs = [], []
    for k, n in enumerate(sizes):
        fmt = "e4m3" if k % 2 == 0 else "e5m2"
        x = wl.small_normal(500 + k, (1, max(n, 1)), std=float(np.exp2(rng.uniform(-4, 4))), outlier_factor=20.0)
        x = x[:, :n]
        if k == 8:
            xt = dev(oracle.bf16_to_f32(x[0]))            # fp32 source: its own flat kernel
        else:
            xt = dev(x[0]) if n else torch.zeros(0, dtype=torch.int16, device="cuda")
        s = np.float32(np.exp2(rng.uniform(-6, 6)))
        q = torch.full((n,), 0x33, dtype=torch.uint8, device="cuda") if k != 3 else None       # k = 3: amax only
        am = f32(0.0) if k != 5 else None                                                       # k = 5: codes only
        items.append((xt, fmt, f32(s), q, am))
        refs.append((x[0], fmt, s, k))
    banner("batched-cast", len(items))
    fp8.fp8_amax_cast_batched(items)
    for (xt, fmt, ds, q, am), (x, _, s, k) in zip(items, refs):
        dtype = "f32" if k == 8 else "bf16"
        src = oracle.bf16_to_f32(x) if k == 8 else x
        if q is not None:
            want = oracle.cast(src, s, fmt, dtype)
            assert np.array_equal(host(q), want), (k, first_diff(host(q), want))
        if am is not None:
            assert f32_bits(am)[0] == np.float32(oracle.amax(src, dtype)).view(np.uint32), k
    banner("batched-cast misaligned item")
    src = torch.zeros(4097, dtype=torch.int16, device="cuda")
    q = torch.full((4096,), 0x5A, dtype=torch.uint8, device="cuda")
    am = f32(0.0)
    with pytest.raises(fp8.Fp8mpError) as ei:
        fp8.fp8_amax_cast_batched([(dev(np.ones(64, np.uint16)), "e4m3", f32(1.0), None, am),
                                   (src[1:], "e4m3", f32(1.0), q, None)])
    assert ei.value.status == 1 and f32_bits(am)[0] == 0 and (host(q) == 0x5A).all()


def test_beyond_two_to_the_31_elements():
    """A 32769 x 65537 BF16 tensor (2^31 + 98305 elements): 64-bit indexing in the flat, batched and
    cast-transpose paths. A repeating pattern of small values with one larger value planted past
    element 2^31 gives the amax exactly; codes are compared with the oracle around the 2^31 boundary,
    at both ends and at random positions, and q^T with q at sampled positions."""
    require_gpu()
    rows, cols = 32769, 65537
    n = rows * cols
    assert n > 2 ** 31
    rng = np.random.default_rng(31)
    pattern = wl.f32_to_bf16_bits((rng.standard_normal(4099) * 20).astype(np.float32))
    reps = -(-n // pattern.size)
    x = dev(pattern).view(torch.int16).repeat(reps)[:n].contiguous()
    peak = n - 5
    x[peak] = int(wl.f32_to_bf16_bits(np.array([1000.0], np.float32))[0].astype(np.int16))
    x2 = x.view(rows, cols)
    idx = np.unique(np.concatenate([np.arange(2 ** 31 - 40, 2 ** 31 + 40), np.arange(0, 40), np.arange(n - 40, n),
                                    rng.integers(0, n, 4000)]))
    ti = torch.from_numpy(idx).cuda()
    xs = host(x[ti]).view(np.uint16)
    s = 4.25
    want_amax = np.float32(1000.0)
    for fmt in FORMATS:
        want = oracle.cast(xs, np.float32(s), fmt, "bf16")
        banner("cast >2^31 flat", fmt)
        q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
        am = f32(0.0)
        fp8.fp8_amax_cast(x2, fmt, f32(s), q, None, am)
        got = host(q.view(-1)[ti])
        assert np.array_equal(got, want), first_diff(got, want)
        assert f32_bits(am)[0] == _amax_bits(want_amax)
        banner("cast >2^31 batched", fmt)
        q.fill_(0x5A)
        am = f32(0.0)
        fp8.fp8_amax_cast_batched([(x, fmt, f32(s), q.view(-1), am)])
        got = host(q.view(-1)[ti])
        assert np.array_equal(got, want), first_diff(got, want)
        assert f32_bits(am)[0] == _amax_bits(want_amax)
        del q
        torch.cuda.empty_cache()
    banner("cast-transpose >2^31")
    xp, xp_store = pitched(rows, cols, torch.int16)   # 16-byte row pitch for the tile kernel
    xp.copy_(x2)
    del x, x2
    torch.cuda.empty_cache()
    q, _ = pitched(rows, cols, torch.uint8)
    qt, _ = pitched(cols, rows, torch.uint8)
    am = f32(0.0)
    fp8.fp8_amax_cast(xp, "e4m3", f32(s), q, qt, am)
    r, c = idx // cols, idx % cols
    got_q = host(q[torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda()])
    got_qt = host(qt[torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda()])
    want = oracle.cast(xs, np.float32(s), "e4m3", "bf16")
    assert np.array_equal(got_q, want), first_diff(got_q, want)
    assert np.array_equal(got_qt, want), first_diff(got_qt, want)
    assert f32_bits(am)[0] == _amax_bits(want_amax)
