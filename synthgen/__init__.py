"""Seeded synthetic weight generators and workload descriptions.

This module only draws inputs: dense weight matrices with the shapes and value
distributions of the linear layers the EntroPack paper compresses, and the
lists of shapes/targets that make up each workload.  It holds none of the
compression arithmetic (no normalisation, quantisation, coding or rounding to
a weight container); both the CPU oracle and the GPU path consume what it
returns.

Distribution: heavy-tailed Student-t entries (nu = 5) times a per-row
lognormal(0, 0.5) scale, times 0.02.  The paper measures on trained
Z-Image-Turbo / Qwen weights that are not available here; these seeded tensors
stand in for them at the same shapes.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

__all__ = [
    "student_t_weights",
    "TensorSpec",
    "workload",
    "WORKLOADS",
]


def student_t_weights(rows: int, cols: int, seed: int, *, df: int = 5,
                      row_sigma: float = 0.5, base: float = 0.02,
                      outlier_frac: float = 0.0, outlier_mult: float = 20.0,
                      bf16: bool = False, device: str = "cpu") -> torch.Tensor:
    """Return a float32 [rows, cols] tensor of seeded Student-t weights.

    t = N(0,1) / sqrt(chi2_df / df) with chi2_df a sum of df squared normals;
    each row is multiplied by exp(row_sigma * N(0,1)).  ``outlier_frac`` of the
    positions (distinct, seeded) are multiplied by ``outlier_mult``.  With
    ``bf16`` the values are rounded to bfloat16 (torch's cast) and returned as
    float32, i.e. a BF16 checkpoint seen in fp32.
    """
    if rows <= 0 or cols <= 0:
        return torch.zeros(max(rows, 0), max(cols, 0), dtype=torch.float32, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    z = torch.randn(rows, cols, generator=g, device=device)
    chi = torch.zeros(rows, cols, device=device)
    for _ in range(df):
        chi.add_(torch.randn(rows, cols, generator=g, device=device).square_())
    w = z.div_(chi.div_(float(df)).sqrt_())
    del chi
    rs = torch.exp(row_sigma * torch.randn(rows, 1, generator=g, device=device))
    w.mul_(rs).mul_(base)
    if outlier_frac > 0.0:
        k = int(outlier_frac * rows * cols)
        if k > 0:
            idx = torch.randperm(rows * cols, generator=g, device=device)[:k]
            w.view(-1)[idx] *= outlier_mult
    if bf16:
        w = w.to(torch.bfloat16).to(torch.float32)
    return w.contiguous()


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    """One weight tensor of a workload: shape [rows, cols] = [out, in]."""
    name: str
    rows: int
    cols: int
    seed: int
    target_bpp: float
    route: str = "direct"        # "direct", "fp8" (row-scaled e4m3) or "int8" (row-scaled)
    bf16: bool = True            # input checkpoint dtype
    outlier_frac: float = 0.0
    prob_bits: Optional[int] = None   # None: the encoder's default for the target
    vectors_per_tile: Optional[int] = None  # None: the encoder's default for the target
    out_dtype: str = "bf16"      # "bf16", "fp8", "int8"

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    def weights(self, device: str = "cpu") -> torch.Tensor:
        return student_t_weights(self.rows, self.cols, self.seed, bf16=self.bf16,
                                 outlier_frac=self.outlier_frac, device=device)


def _cfg1(vpt: int = 512) -> List[TensorSpec]:
    # 256x512 fp32 matrix, 4 bpp, 12-bit probabilities, tiles of 4096 coordinates.
    return [TensorSpec("w256x512", 256, 512, 1, 4.0, bf16=False, prob_bits=12,
                       vectors_per_tile=vpt)]


def _cfg2(target: float) -> List[TensorSpec]:
    # one 3840x3840 BF16 weight with 0.1% outliers x20, one W for all targets.
    return [TensorSpec(f"w3840_{int(target)}bpp", 3840, 3840, 2, float(target),
                       outlier_frac=0.001)]


_DIT_BLOCK = (("qkv", 11520, 3840), ("out", 3840, 3840), ("up", 10240, 3840),
              ("gate", 10240, 3840), ("down", 3840, 10240))


def _cfg3(blocks: int = 30, prob_bits: Optional[int] = None) -> List[TensorSpec]:
    # DiT linear set: blocks x {QKV 3840->11520, out, FFN up/gate 3840->10240, down}.
    # prob_bits overrides the encoder's default precision (same weights).
    out = []
    i = 0
    for blk in range(blocks):
        for name, r, c in _DIT_BLOCK:
            out.append(TensorSpec(f"b{blk}.{name}", r, c, 3000 + i, 4.0, prob_bits=prob_bits))
            i += 1
    return out


_LLM_LAYER = (("qkv", 7168, 5120), ("o", 5120, 5120), ("gate", 17408, 5120),
              ("up", 17408, 5120), ("down", 5120, 17408))


def _cfg4(layers: int = 16) -> List[TensorSpec]:
    # LLM prefill set, row-scaled FP8-e4m3 route, 5 bpp, decoded to FP8 codes.
    out = []
    i = 0
    for lay in range(layers):
        for name, r, c in _LLM_LAYER:
            out.append(TensorSpec(f"l{lay}.{name}", r, c, 4000 + i, 5.0, route="fp8",
                                  out_dtype="fp8"))
            i += 1
    return out


def _cfg5(n: int = 300) -> List[TensorSpec]:
    # Mixed-bit set: shapes uniform over {1536,2048,3840,5120,10240}^2 (seed 5),
    # sensitivity scores U(0,1) (seed 55); the top 10% by score at 8 bpp, the
    # rest at 2 bpp; row-scaled INT8 route decoded to INT8 codes.
    dims = np.array([1536, 2048, 3840, 5120, 10240])
    rs = np.random.default_rng(5)
    shapes = dims[rs.integers(0, len(dims), size=(n, 2))]
    score = np.random.default_rng(55).random(n)
    top = set(np.argsort(-score, kind="stable")[: max(1, n // 10)].tolist())
    out = []
    for i in range(n):
        tgt = 8.0 if i in top else 2.0
        out.append(TensorSpec(f"t{i}", int(shapes[i, 0]), int(shapes[i, 1]), 5000 + i, tgt,
                              route="int8", out_dtype="int8"))
    return out


def _ref_layer(target: float) -> List[TensorSpec]:
    # the paper's reference layer shape (an FFN projection, 3840 -> 10240), one tensor
    return [TensorSpec(f"ref_layer_{int(target)}bpp", 10240, 3840, 6, float(target))]


WORKLOADS = {
    "w256x512_4bpp_fp32": lambda: _cfg1(512),
    "w256x512_4bpp_fp32_s4096": lambda: _cfg1(455),
    "w3840_4bpp": lambda: _cfg2(4),
    "w3840_5bpp": lambda: _cfg2(5),
    "w3840_6bpp": lambda: _cfg2(6),
    "w3840_7bpp": lambda: _cfg2(7),
    "w3840_8bpp": lambda: _cfg2(8),
    "ref_layer_10240x3840_4bpp_bf16": lambda: _ref_layer(4),
    "ref_layer_10240x3840_8bpp_bf16": lambda: _ref_layer(8),
    "dit_linear_set_30x5_4bpp_bf16": lambda: _cfg3(30),
    "dit_linear_set_30x5_4bpp_b9_bf16": lambda: _cfg3(30, 9),
    "llm_prefill_16x5_fp8route_5bpp": lambda: _cfg4(16),
    "mixed_300_int8route_2or8bpp": lambda: _cfg5(300),
}


def workload(name: str) -> List[TensorSpec]:
    """Tensor list of a named workload."""
    return WORKLOADS[name]()
