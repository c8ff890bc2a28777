"""One step of a per-tensor-scaled FP8 linear layer, as a sequence of C-ABI calls.

[TE] §基本的なFP8トレーニングコードの構成: the FP8 linear layer replaces nn.Linear and
runs inside an FP8 recipe context; [TE] §動的スケーリングとFP8レシピの設定: HYBRID uses
E4M3 in the forward pass and E5M2 in the backward pass. A step is:

  1. for every operand tensor: one fused pass that casts it with the scale of
     the previous step and records its amax into history[0] (and, when an
     operand is needed K-contiguous the other way round, writes the transposed
     codes in the same pass);
  2. every GEMM, dequantised by the inverse scales those codes were made with;
  3. the delayed-scaling update of every tensor's scale.

An operand marked ``layernorm`` is the LayerNorm of its source, normalised and
cast in one pass (fp8_layernorm_amax_cast; [TE] §基本的なFP8トレーニングコードの構成
swaps nn.LayerNorm along with nn.Linear); ``ln_params`` supplies its gamma,
beta (device fp32) and eps.

With ``output_cast`` the GEMM outputs are also cast to E4M3 for a following
layer ([TE] §基本的なFP8トレーニングコードの構成 chains te.Linear layers), under the
same delayed recipe with a state of their own: "fused" does it in the GEMM's
epilogue (fp8_scaled_gemm_amax_cast), "separate" with a second pass over the
BF16 output (fp8_amax_cast), the unfused reference. "fused_codes" is "fused"
without storing the BF16 output, for a following layer that reads the codes
only.

``gemm_accum`` "exact" (the default) multiplies with FP32 accumulation;
"fast" uses the FP8 matrix instruction's reduced-precision accumulation
(fp8_scaled_gemm_fast_accum, within 2**-9 of sum|a*b|) for every GEMM.

The plan owns its device buffers (allocated once, through torch, with rows
starting 16 bytes apart multiples as the C-ABI requires of strided buffers); a
step allocates nothing and never synchronises.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import (CastBatch, CurrentScalingState, DelayedScalingState, ScaleUpdateBatch, fp8_amax_cast,
               fp8_amax_cast_batched, fp8_layernorm_amax_cast, fp8_scale_update_batched, fp8_scaled_gemm,
               fp8_scaled_gemm_amax_cast, fp8_scaled_gemm_amax_cast_fast_accum, fp8_scaled_gemm_fast_accum)


def _pitched(rows: int, cols: int, dtype, device) -> torch.Tensor:
    """A rows x cols buffer whose rows start 16 bytes apart multiples (the C-ABI's rule for strided
    buffers); contiguous when a row is already a multiple of 16 bytes."""
    esz = torch.empty(0, dtype=dtype).element_size()
    ld = -(-cols * esz // 16) * 16 // esz
    return torch.empty(rows, max(ld, 1), dtype=dtype, device=device)[:, :cols]


@dataclass(frozen=True)
class OperandSpec:
    name: str
    shape: Tuple[int, int]
    fmt: str                  # "e4m3" or "e5m2"
    transposed: bool = False  # also produce the transposed codes
    plain: bool = True        # produce the row-major codes
    layernorm: bool = False   # the operand is LayerNorm(source) (row-major codes only)


@dataclass(frozen=True)
class GemmOp:
    name: str
    a: str
    a_transposed: bool
    b: str
    b_transposed: bool


class LayerPlan:
    """recipe "delayed" (the default) or "current" (just-in-time scaling: amax pass, update, cast);
    output_cast None, "fused", "fused_codes" (no BF16 output stored) or "separate" (delayed recipe only);
    gemm_accum "exact" (FP32 accumulation) or "fast" (the FP8 matrix instruction's own accumulation)."""

    def __init__(self, operands: Sequence[OperandSpec], gemms: Sequence[GemmOp], history_len: int = 1024,
                 margin: int = 0, device: str = "cuda", recipe: str = "delayed", output_cast: Optional[str] = None,
                 ln_params: Optional[Dict[str, tuple]] = None, gemm_accum: str = "exact"):
        if recipe not in ("delayed", "current"):
            raise ValueError(recipe)
        if gemm_accum not in ("exact", "fast"):
            raise ValueError(gemm_accum)
        self.gemm_accum = gemm_accum
        fast = gemm_accum == "fast"
        self._gemm = fp8_scaled_gemm_fast_accum if fast else fp8_scaled_gemm
        self._gemm_cast = fp8_scaled_gemm_amax_cast_fast_accum if fast else fp8_scaled_gemm_amax_cast
        if output_cast not in (None, "fused", "fused_codes", "separate"):
            raise ValueError(output_cast)
        if output_cast and recipe != "delayed":
            raise ValueError("the output cast follows the delayed recipe (its amax is taken while casting)")
        self.recipe = recipe
        self.output_cast = output_cast
        self.ln = {}
        for o in operands:
            if o.layernorm:
                if o.transposed or not o.plain:
                    raise ValueError(f"{o.name}: the LayerNorm path writes row-major codes only")
                if recipe != "delayed":
                    raise ValueError("the LayerNorm path follows the delayed recipe")
                if not ln_params or o.name not in ln_params:
                    raise ValueError(f"{o.name}: gamma, beta, eps missing")
                self.ln[o.name] = ln_params[o.name]
        self.ystate: Dict[str, DelayedScalingState] = {}
        self.yq: Dict[str, torch.Tensor] = {}
        self.operands = {o.name: o for o in operands}
        self.gemms = list(gemms)
        self.state: Dict[str, DelayedScalingState] = {}
        self.q: Dict[str, Optional[torch.Tensor]] = {}
        self.qt: Dict[str, Optional[torch.Tensor]] = {}
        self.out: Dict[str, torch.Tensor] = {}
        for o in operands:
            r, c = o.shape
            self.state[o.name] = (DelayedScalingState(o.fmt, history_len, margin, device) if recipe == "delayed"
                                  else CurrentScalingState(o.fmt, margin, device))
            self.q[o.name] = _pitched(r, c, torch.uint8, device) if o.plain else None
            self.qt[o.name] = _pitched(c, r, torch.uint8, device) if o.transposed else None
        self._batch = None
        self._cast_batch = None
        self._gemm_args = []
        for g in self.gemms:
            a = self.qt[g.a] if g.a_transposed else self.q[g.a]
            b = self.qt[g.b] if g.b_transposed else self.q[g.b]
            if a is None or b is None:
                raise ValueError(f"gemm {g.name}: operand layout not produced")
            if a.shape[1] != b.shape[1]:
                raise ValueError(f"gemm {g.name}: K mismatch {tuple(a.shape)} vs {tuple(b.shape)}")
            c = _pitched(a.shape[0], b.shape[0], torch.bfloat16, device)
            self.out[g.name] = c
            if output_cast:
                self.ystate[g.name] = DelayedScalingState("e4m3", history_len, margin, device)
                self.yq[g.name] = _pitched(a.shape[0], b.shape[0], torch.uint8, device)
            sa, sb = self.state[g.a], self.state[g.b]
            self._gemm_args.append((a, sa.fmt, b, sb.fmt, sa.scale_inv, sb.scale_inv, c))

    def prime(self, inputs: Dict[str, torch.Tensor], stream=None) -> None:
        """An amax-only pass over every operand, then one update (single-shot workloads)."""
        if self.recipe == "current":
            return
        for name, st in self.state.items():
            if name in self.ln:
                g, b, eps = self.ln[name]
                fp8_layernorm_amax_cast(inputs[name], g, b, eps, st.fmt, None, None, None, st.amax_slot,
                                        stream=stream)
            else:
                fp8_amax_cast(inputs[name], st.fmt, None, None, None, st.amax_slot, stream)
        for st in self.state.values():
            st.update(stream)
        if self.output_cast:
            # the outputs' scales need the outputs: cast (without recording), multiply, record their amax
            for name, st in self.state.items():
                if name in self.ln:
                    g, b, eps = self.ln[name]
                    fp8_layernorm_amax_cast(inputs[name], g, b, eps, st.fmt, None, st.scale, self.q[name], None,
                                            stream=stream)
                else:
                    st.cast(inputs[name], self.q[name], self.qt[name], False, stream)
            for g, (a, af, b, bf, sa, sb, c) in zip(self.gemms, self._gemm_args):
                ys = self.ystate[g.name]
                self._gemm_cast(a, af, b, bf, sa, sb, c if self.output_cast != "fused_codes" else None,
                                ys.fmt, None, None, ys.amax_slot, stream)
            for ys in self.ystate.values():
                ys.update(stream)

    def cast_all(self, inputs: Dict[str, torch.Tensor], stream=None) -> None:
        """Every operand's cast. Under the delayed recipe the plain row-major casts of contiguous sources go
        out as one batched launch (built on first use for these input tensors)."""
        batched = set()
        if self.recipe == "delayed":
            names = [n for n, o in self.operands.items()
                     if n not in self.ln and not o.transposed and inputs[n].is_contiguous()
                     and self.q[n] is not None and self.q[n].is_contiguous()]
            key = tuple((n, inputs[n].data_ptr(), inputs[n].dtype, inputs[n].numel()) for n in names)
            if names and (self._cast_batch is None or self._cast_batch[0] != key):
                items = [(inputs[n], self.state[n].fmt, self.state[n].scale, self.q[n], self.state[n].amax_slot)
                         for n in names]
                self._cast_batch = (key, CastBatch(items))
            if names:
                fp8_amax_cast_batched(self._cast_batch[1], stream)
                batched = set(names)
        for name, st in self.state.items():
            if name in batched:
                continue
            if name in self.ln:
                g, b, eps = self.ln[name]
                fp8_layernorm_amax_cast(inputs[name], g, b, eps, st.fmt, None, st.scale, self.q[name], st.amax_slot,
                                        stream=stream)
            elif self.recipe == "delayed":
                st.cast(inputs[name], self.q[name], self.qt[name], True, stream)
            else:
                st.cast(inputs[name], self.q[name], self.qt[name], stream)

    def gemm_all(self, stream=None) -> None:
        for g, (a, af, b, bf, sa, sb, c) in zip(self.gemms, self._gemm_args):
            if self.output_cast in ("fused", "fused_codes"):
                ys = self.ystate[g.name]
                self._gemm_cast(a, af, b, bf, sa, sb, c if self.output_cast == "fused" else None, ys.fmt,
                                ys.scale, self.yq[g.name], ys.amax_slot, stream)
            else:
                self._gemm(a, af, b, bf, sa, sb, c, stream)

    def output_cast_all(self, stream=None) -> None:
        """The unfused output cast (a no-op unless output_cast == "separate")."""
        if self.output_cast != "separate":
            return
        for g in self.gemms:
            ys = self.ystate[g.name]
            ys.cast(self.out[g.name], self.yq[g.name], None, True, stream)

    def update_all(self, stream=None) -> None:
        """Every tensor's delayed-scaling update, in one launch."""
        if self.recipe == "current":
            return
        if self._batch is None:
            self._batch = ScaleUpdateBatch(list(self.state.values()) + list(self.ystate.values()))
        fp8_scale_update_batched(self._batch, stream)

    def step(self, inputs: Dict[str, torch.Tensor], stream=None) -> None:
        self.cast_all(inputs, stream)
        self.gemm_all(stream)
        self.output_cast_all(stream)
        self.update_all(stream)

    def capture(self, inputs: Dict[str, torch.Tensor], steps: int = 1) -> "torch.cuda.CUDAGraph":
        """`steps` consecutive steps captured as one HIP graph (through torch's graph API): replaying it
        runs their launches without host launch overhead or gaps between kernels. The graph reads
        `inputs` and writes the plan's buffers at the addresses they have now; every replay advances the
        recipe by `steps` steps, like that many calls of step(). A training loop captures a whole
        iteration (many layers) the same way, so the cost of launching a graph is spread over them.
        The step issues only kernel launches (no memset or copy nodes). Call prime() (and, for the
        batched cast, one eager step) first, so nothing is allocated during capture."""
        if steps < 1:
            raise ValueError("steps must be at least 1")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.step(inputs)
        return g

    def gemm_operands(self) -> List[tuple]:
        """Per GEMM: (a codes, a format, b codes, b format, a scale_inv, b scale_inv, BF16 output), the
        arguments the step passes to the GEMM call."""
        return list(self._gemm_args)

    def gemm_flops(self) -> int:
        return sum(2 * a.shape[0] * b.shape[0] * a.shape[1] for a, _, b, _, _, _, _ in self._gemm_args)

    def cast_bytes(self, inputs: Dict[str, torch.Tensor]) -> int:
        """Algorithmic bytes of the casts: source read once (twice for just-in-time scaling),
        each code layout written once."""
        reads = 1 if self.recipe == "delayed" else 2
        total = 0
        for name, o in self.operands.items():
            n = o.shape[0] * o.shape[1]
            total += reads * n * inputs[name].element_size() + n * (int(o.plain) + int(o.transposed))
        return total

    def output_cast_bytes(self) -> int:
        """Algorithmic bytes of the output casts beyond the BF16 outputs themselves: the codes
        written, plus (separate only) a second read of each output. With "fused_codes" the GEMM
        writes the codes instead of the BF16 output."""
        total = 0
        for c in self.out.values() if self.output_cast else ():
            total += c.numel() * (1 + (2 if self.output_cast == "separate" else 0))
        return total


def plan_from_workload(w, device: str = "cuda", recipe: str = "delayed", output_cast: Optional[str] = None,
                       layernorm: Sequence[str] = (), ln_params: Optional[Dict[str, tuple]] = None,
                       gemm_accum: str = "exact") -> LayerPlan:
    """A LayerPlan from a workload description with the attributes
    ``tensors`` (``name``, ``shape``), ``formats``, ``transposed``, ``gemms``
    (``name``, ``a``, ``a_transposed``, ``b``, ``b_transposed``), ``history_len``
    and ``margin``."""
    ops = [OperandSpec(t.name, tuple(t.shape), w.formats[t.name], t.name in w.transposed, True, t.name in layernorm)
           for t in w.tensors]
    gemms = [GemmOp(g.name, g.a, g.a_transposed, g.b, g.b_transposed) for g in w.gemms]
    return LayerPlan(ops, gemms, w.history_len, w.margin, device, recipe, output_cast, ln_params, gemm_accum)
