"""The five video-shaped workloads of the Pyramid Sparse Attention forward path.

Shapes, grids, block sizes and level counts follow the method's problem
statement (query blocks, 64-token KV blocks pooled to 64/32/16/8 rows at levels
0..3; "PSA: Pyramid Sparse Attention for Efficient Video Understanding and
Generation", abstract; the skillmd.com summary's pyramid and scoring sections).
The host models they imitate are the ones the top168.com article names in its
results paragraphs (Wan2.1-1.3B / 14B, CogVideoX-5B, Qwen2.5-VL-7B).

This module holds data only: no step of the method's arithmetic lives here.
Thresholds for the four sparsity-targeted workloads (and the ranked rule's
matched block fractions) are read from ``thresholds.json``, which the oracle's
calibration script writes.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
THRESHOLDS_FILE = os.path.join(_HERE, "thresholds.json")

# Reference thresholds for the tiny workload, and the base of the one-parameter
# family tau_l(x) = TAU0_l ** x used to hit the other workloads' FLOP fractions.
TAU0 = (0.6, 0.8, 0.9, 0.95)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    H_kv: int
    d: int
    grid: Tuple[int, int, int]          # (T, H_grid, W) video latent grid, raster order
    n_text: int                          # i.i.d. N(0,1) tokens placed before the grid
    dtype: str                           # "f32" or "bf16": I/O dtype of q, k, v, pyramid, o
    q_block: int
    kv_block: int = 64
    num_levels: int = 4
    ft_max: float = 2.0                  # temporal frequency range U[0, ft_max] cycles per extent
    target_rho: Optional[float] = None   # FLOP fraction the thresholds are calibrated to
    n_dense_prefix: int = 0              # tokens whose KV blocks are always kept at level 0
    fixed_thresholds: Optional[Tuple[float, ...]] = None
    causal: bool = False                 # query row r sees tokens 0..r only
    description: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        T, Hg, W = self.grid
        return self.n_text + T * Hg * W

    @property
    def nqb(self) -> int:
        return -(-self.N // self.q_block)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.kv_block)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def thresholds(self) -> Tuple[float, ...]:
        """Cumulative-mass thresholds, one per level (as float32-representable values)."""
        if self.fixed_thresholds is not None:
            return tuple(self.fixed_thresholds[: self.num_levels])
        with open(THRESHOLDS_FILE) as f:
            table = json.load(f)
        entry = table.get(self.name)
        if entry is None:
            raise KeyError(f"no calibrated thresholds for workload {self.name!r} in {THRESHOLDS_FILE}")
        return tuple(float(t) for t in entry["thresholds"][: self.num_levels])

    def ranked_fractions(self) -> Tuple[float, ...]:
        """Cumulative block fractions per level for the ranked rule, matched to the
        threshold mask's mean level counts (written by the same calibration script)."""
        with open(THRESHOLDS_FILE) as f:
            entry = json.load(f).get(self.name, {})
        if "ranked_fractions" not in entry:
            raise KeyError(f"no ranked fractions for workload {self.name!r} in {THRESHOLDS_FILE}")
        return tuple(float(x) for x in entry["ranked_fractions"][: self.num_levels])

    def dense_flops(self) -> float:
        """4*B*H*N^2*d: QK^T plus PV of dense attention (causal: the N(N+1)/2 visible pairs)."""
        pairs = self.N * (self.N + 1) / 2 if self.causal else float(self.N) * self.N
        return 4.0 * self.B * self.H * pairs * self.d


WORKLOADS = {
    "tiny": Workload(
        name="tiny", index=0, B=1, H=2, H_kv=2, d=64, grid=(8, 16, 16), n_text=0,
        dtype="f32", q_block=64, fixed_thresholds=TAU0,
        description="tiny reference case, 2048 tokens on an 8x16x16 grid, fp32"),
    "wan13b": Workload(
        name="wan13b", index=1, B=1, H=12, H_kv=12, d=128, grid=(21, 30, 52), n_text=0,
        dtype="bf16", q_block=128, ft_max=0.5, target_rho=0.09,
        description="Wan2.1-1.3B-style self-attention layer, 32760 tokens, ~91% sparsity"),
    "cogvx5b": Workload(
        name="cogvx5b", index=2, B=1, H=48, H_kv=48, d=64, grid=(13, 30, 45), n_text=226,
        dtype="bf16", q_block=128, target_rho=0.15, n_dense_prefix=226,
        description="CogVideoX-5B-style full attention, 226 text + 17550 video tokens, ~85% sparsity"),
    "qwen7b": Workload(
        name="qwen7b", index=3, B=1, H=28, H_kv=4, d=128, grid=(16, 32, 32), n_text=0,
        dtype="bf16", q_block=64, target_rho=0.35,
        description="Qwen2.5-VL-7B-style GQA bidirectional attention, 16384 tokens, ~35% of dense FLOPs"),
    "wan13b_causal": Workload(
        name="wan13b_causal", index=5, B=1, H=12, H_kv=12, d=128, grid=(21, 30, 52), n_text=0,
        dtype="bf16", q_block=128, ft_max=0.5, target_rho=0.09, causal=True,
        description="Wan2.1-1.3B-style layer in causal use, 32760 tokens, ~91% sparsity of causal attention"),
    "wan14b": Workload(
        name="wan14b", index=4, B=1, H=40, H_kv=40, d=128, grid=(21, 45, 80), n_text=0,
        dtype="bf16", q_block=128, target_rho=0.09,
        description="Wan2.1-14B-style 720p/81-frame self-attention layer, 75600 tokens, ~91% sparsity"),
}

BY_INDEX = {w.index: w for w in WORKLOADS.values()}


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return BY_INDEX[name_or_index]
    return WORKLOADS[name_or_index]
