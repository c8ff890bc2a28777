"""Seeded synthetic operands for the per-tensor-scaled FP8 linear layer.

This module only draws inputs. It holds none of the method's arithmetic (no
FP8 codec, no amax, no scaling, no GEMM), so both the CPU oracle and the HIP
path consume exactly the arrays produced here.

The pages measure LLM training at GPT-3 and 7B..70B scale on unnamed data
(「NVIDIA Transformer EngineとFP8混合精度の実装ガイド」, sections
「ベンチマーク環境の構築とテスト方法」 and 「結果の解釈とFP8が有効なケース・不要なケース」).
No dataset is named, so seeded Llama-shaped operands stand in for them:
activations are standard normal with a sparse set of large outliers (the
outlier-heavy activations that 「NVIDIA TensorRTによるFP8量子化」 §FP8量子化の技術的優位性と背景
says FP8 handles better than INT8), weights are narrow normals, and gradients
are heavy tailed (Student-t, nu = 3).

Recipe, shared by every tensor:
  * generator: numpy PCG64 seeded with SeedSequence([20261202, config_id, tensor_id]);
  * normals: standard_normal(float32) times the stated standard deviation (in fp32);
  * Student-t: standard_t(3) cast to float32, times the stated scale;
  * outliers: exactly round(1e-3 * numel) distinct flat positions drawn with
    choice(numel, k, replace=False) from the same generator after the values,
    multiplied (in fp32) by the stated factor;
  * BF16 operands: the fp32 array rounded to the nearest BF16, ties to even,
    returned as uint16 bit patterns (no NaN or Inf can occur here).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

ROOT_SEED = 20261202

# tensor ids inside one config's seed sequence
TID_X, TID_W, TID_W2, TID_DY, TID_STEP_FACTORS = 0, 1, 2, 3, 9


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, int]
    dist: str                 # "normal" or "student_t3"
    scale: float              # standard deviation (normal) or scale (Student-t)
    outlier_factor: Optional[float] = None
    dtype: str = "bf16"       # "bf16" (uint16 bits) or "f32"
    tensor_id: int = 0


@dataclass(frozen=True)
class GemmSpec:
    """One FP8 GEMM of the workload: C[m x n] = A[m x k] . B[n x k]^T."""
    name: str
    a: str                    # tensor name whose (possibly transposed) codes form A
    a_transposed: bool
    a_fmt: str                # "e4m3" or "e5m2"
    b: str
    b_transposed: bool
    b_fmt: str
    m: int
    n: int
    k: int


@dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    description: str
    tensors: Tuple[TensorSpec, ...]
    gemms: Tuple[GemmSpec, ...]
    formats: Dict[str, str] = field(default_factory=dict)   # tensor -> FP8 format
    transposed: Tuple[str, ...] = ()                       # tensors cast with a transposed copy
    history_len: int = 1024
    margin: int = 0
    steps: int = 1                                         # recipe steps (after priming)

    def tensor(self, name: str) -> TensorSpec:
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)


def _x(shape, cid_outlier=20.0):
    return TensorSpec("X", shape, "normal", 1.0, cid_outlier, "bf16", TID_X)


WORKLOADS: List[Workload] = [
    Workload(
        0, "tiny_fwd_256",
        "Tiny FP8 linear forward, fp32 X[256x256] and W[256x256], 16 delayed-scaling steps",
        (TensorSpec("X", (256, 256), "normal", 1.0, 50.0, "f32", TID_X),
         TensorSpec("W", (256, 256), "normal", 1.0, 50.0, "f32", TID_W)),
        (GemmSpec("fwd", "X", False, "e4m3", "W", False, "e4m3", 256, 256, 256),),
        {"X": "e4m3", "W": "e4m3"}, (), history_len=16, margin=0, steps=16),
    Workload(
        1, "mlp7b_up_fwd",
        "7B-class MLP up-projection forward, M=4096 N=11008 K=4096",
        (_x((4096, 4096)),
         TensorSpec("W", (11008, 4096), "normal", 0.02, None, "bf16", TID_W)),
        (GemmSpec("fwd", "X", False, "e4m3", "W", False, "e4m3", 4096, 11008, 4096),),
        {"X": "e4m3", "W": "e4m3"}),
    Workload(
        2, "mlp7b_bwd_hybrid",
        "7B-class MLP up-projection backward, HYBRID: dY in E5M2, X and W in E4M3",
        (_x((4096, 4096)),
         TensorSpec("W", (11008, 4096), "normal", 0.02, None, "bf16", TID_W),
         TensorSpec("dY", (4096, 11008), "student_t3", 1e-3, None, "bf16", TID_DY)),
        # dX[4096x4096] = dY[4096x11008] . W[11008x4096]   -> A = dYq, B = (Wq)^T
        # dW[11008x4096] = dY^T[11008x4096] . X[4096x4096] -> A = (dYq)^T, B = (Xq)^T
        (GemmSpec("dgrad", "dY", False, "e5m2", "W", True, "e4m3", 4096, 4096, 11008),
         GemmSpec("wgrad", "dY", True, "e5m2", "X", True, "e4m3", 11008, 4096, 4096)),
        {"X": "e4m3", "W": "e4m3", "dY": "e5m2"}, ("X", "W", "dY")),
    Workload(
        3, "proj13b_fwd",
        "13B-class QKV and MLP projections forward, X[8192x5120]",
        (_x((8192, 5120)),
         TensorSpec("Wqkv", (15360, 5120), "normal", 0.02, None, "bf16", TID_W),
         TensorSpec("Wmlp", (13824, 5120), "normal", 0.02, None, "bf16", TID_W2)),
        (GemmSpec("qkv", "X", False, "e4m3", "Wqkv", False, "e4m3", 8192, 15360, 5120),
         GemmSpec("mlp", "X", False, "e4m3", "Wmlp", False, "e4m3", 8192, 13824, 5120)),
        {"X": "e4m3", "Wqkv": "e4m3", "Wmlp": "e4m3"}),
    Workload(
        4, "slice70b_fwd",
        "70B-class single-GPU layer slice, X[16384x8192], W[28672x8192], cast+transpose",
        (_x((16384, 8192)),
         TensorSpec("W", (28672, 8192), "normal", 0.015, None, "bf16", TID_W)),
        (GemmSpec("fwd", "X", False, "e4m3", "W", False, "e4m3", 16384, 28672, 8192),),
        {"X": "e4m3", "W": "e4m3"}, ("X", "W")),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def rng_for(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, config_id, tensor_id]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest BF16 (ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_f32(config_id: int, spec: TensorSpec, shape: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """The fp32 values of a tensor before any BF16 rounding."""
    shape = spec.shape if shape is None else shape
    rng = rng_for(config_id, spec.tensor_id)
    numel = int(np.prod(shape))
    if spec.dist == "normal":
        x = rng.standard_normal(numel, dtype=np.float32)
    elif spec.dist == "student_t3":
        x = rng.standard_t(3, size=numel).astype(np.float32)
    else:
        raise ValueError(spec.dist)
    if spec.scale != 1.0:
        x *= np.float32(spec.scale)
    if spec.outlier_factor is not None:
        k = int(round(1e-3 * numel))
        pos = rng.choice(numel, k, replace=False)
        x[pos] *= np.float32(spec.outlier_factor)
    return x.reshape(shape)


def draw(config_id: int, spec: TensorSpec, shape: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """A tensor in its storage dtype: float32, or BF16 as uint16 bits."""
    x = draw_f32(config_id, spec, shape)
    if spec.dtype == "f32":
        return x
    return f32_to_bf16_bits(x)


def step_factors(config_id: int, steps: int) -> np.ndarray:
    """Per-step activation rescale factors u_t ~ U[0.5, 2), float32."""
    rng = rng_for(config_id, TID_STEP_FACTORS)
    return rng.uniform(0.5, 2.0, size=steps).astype(np.float32)


def tiny_step_inputs(x: np.ndarray, u: np.ndarray) -> List[np.ndarray]:
    """X_t = fp32(X * u_t) for each step of the tiny workload."""
    return [(x * np.float32(ut)).astype(np.float32) for ut in u]


def load(name: str, shape_override: Optional[Dict[str, Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """Every input tensor of one workload, keyed by tensor name."""
    w = BY_NAME[name]
    shape_override = shape_override or {}
    return {t.name: draw(w.config_id, t, shape_override.get(t.name)) for t in w.tensors}


def small_normal(seed: int, shape, std: float = 1.0, outlier_factor: Optional[float] = None,
                 dtype: str = "bf16", dist: str = "normal") -> np.ndarray:
    """A reduced-size operand with the same recipe, for fast parity cases."""
    spec = TensorSpec("s", tuple(shape), dist, std, outlier_factor, dtype, 0)
    return draw(1000 + seed, spec)
