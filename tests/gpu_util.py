"""Helpers shared by the GPU parity tests: host <-> device copies and case banners."""
import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def banner(*parts):
    """Name the case on stdout before a GPU step, so a crash still says what ran."""
    print("CASE", *parts, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """Copy a host array to cuda:0 keeping its bits (uint16 BF16 patterns become int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        return a.view(np.uint16)
    return a


def f32(v) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def f32_bits(t: torch.Tensor) -> np.ndarray:
    return host(t).astype(np.float32).view(np.uint32)


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    idx = np.argwhere(np.asarray(a) != np.asarray(b))
    if idx.size == 0:
        return "equal"
    i = tuple(idx[0])
    return f"{idx.shape[0]} mismatches, first at {i}: got {a[i]!r} want {b[i]!r}"


def pitched(rows: int, cols: int, dtype, fill=None, pad_bytes: int = 0):
    """A rows x cols device view whose rows start 16 bytes apart multiples (row pitch rounded up to 16
    bytes, plus pad_bytes, a multiple of 16) in a 16-byte aligned allocation, as the C-ABI requires of
    every strided buffer. Returns (view, storage); the storage shows writes past the view's columns."""
    assert pad_bytes % 16 == 0
    esz = torch.empty(0, dtype=dtype).element_size()
    ld = (-(-cols * esz // 16) * 16 + pad_bytes) // esz
    store = torch.empty(rows, max(ld, 1), dtype=dtype, device="cuda")
    if fill is not None:
        store.fill_(fill)
    return store[:, :cols], store
