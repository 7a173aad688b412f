"""The layer workloads (c1..c7) as plain parameters.

c1  tiny CPU-checkable layer, fp32, 2 heads, d=64, grid 4x8x8, 64-token blocks,
    window of +-1 frame keeping every candidate block pair.
c2  small video layer, bf16, 12 heads, d=64, grid 8x16x16, 10% window.
c3  headline layer, bf16, 12 heads, d=128, grid 21x30x52 (32760 tokens padded
    to 32768), 10% window (+-1 frame).
c4  large-DiT dynamic layer, bf16, 40 heads, d=128, same grid, pooled-score
    top-k at 10% per query block, gate = sigmoid(mean(Q) . w_g).
c5  long-video layer, bf16, 12 heads, d=128, grid 41x45x80 (147600 tokens
    padded to 147712), 128-token blocks, per-head density U(3%, 10%); heads 0-5
    use a +-2-frame window, heads 6-11 a pooled-score top-k.

c6  small bf16 layer with SICS heads (top key blocks by the sum of intra-block
    cosine similarities, 10%, plus the diagonal), c2's shape.
c7  c3's shape (21x30x52, 12 heads, d=128) with SICS heads at 10%.
c8  c3's layer with flat 1x8x8 cuboid blocks (tokens stored cuboid by cuboid),
    10% window (+-1 frame).
c9  small ragged cuboid layer, bf16, 4 heads, d=64, grid 5x10x14, 2x4x8 cuboids
    (partial cuboids on every axis): two window heads, one top-k, one SICS,
    gate from Q.

The per-head densities of c5 are drawn here (stream 8 of the config's seed) so
that every consumer sees the same mask specification.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

WINDOW = 0
TOPK = 1
SICS = 2


@dataclass(frozen=True)
class HeadSpec:
    """Mask request for one head.

    kind      WINDOW (static spatio-temporal window), TOPK (pooled-score top-k) or SICS
              (top key blocks by the sum of intra-block cosine similarities)
    t_window  window heads: keep token pairs at most this many frames apart
    r_max     window heads: cap on the spatial (Chebyshev) block distance, -1 = none
    density   fraction of block pairs to keep; <= 0 keeps every window candidate
    """

    kind: int
    t_window: int = 1
    r_max: int = -1
    density: float = 0.0


@dataclass(frozen=True)
class LayerConfig:
    name: str
    seed: int
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    block: int
    dtype: str  # "f32" or "bf16"
    specs: Tuple[HeadSpec, ...]
    gate_kind: str  # "const", "uniform" (U(0, 0.3) per head) or "from_q"
    gate_const: float = 0.0
    eps: float = 1e-6
    description: str = ""
    extra: dict = field(default_factory=dict, compare=False)
    # cuboid block shape (ct, ch, cw), product = block; (0, 0, 0) = frame-major runs
    cuboid: Tuple[int, int, int] = (0, 0, 0)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    @property
    def n_pad(self) -> int:
        return self.nb * self.block

    def dense_equiv_flop(self) -> float:
        """4 * B * H * N^2 * d: the dense-attention count (QK^T plus PV)."""
        return 4.0 * self.batch * self.heads * float(self.N) ** 2 * self.head_dim


def _c5_densities(seed: int, heads: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 8])
    return rng.uniform(0.03, 0.10, size=heads)


def _build() -> dict:
    cfgs = {}
    cfgs["c1"] = LayerConfig(
        name="c1", seed=1, batch=1, heads=2, head_dim=64, T=4, H=8, W=8, block=64,
        dtype="f32", specs=tuple(HeadSpec(WINDOW, 1, -1, 0.0) for _ in range(2)),
        gate_kind="const", gate_const=0.1,
        description="tiny fp32 layer, 2 heads, d=64, 4x8x8 grid, +-1 frame window (all candidates)")
    cfgs["c2"] = LayerConfig(
        name="c2", seed=2, batch=1, heads=12, head_dim=64, T=8, H=16, W=16, block=64,
        dtype="bf16", specs=tuple(HeadSpec(WINDOW, 1, -1, 0.10) for _ in range(12)),
        gate_kind="uniform",
        description="small bf16 layer, 12 heads, d=64, 8x16x16 grid, 10% window")
    cfgs["c3"] = LayerConfig(
        name="c3", seed=3, batch=1, heads=12, head_dim=128, T=21, H=30, W=52, block=64,
        dtype="bf16", specs=tuple(HeadSpec(WINDOW, 1, -1, 0.10) for _ in range(12)),
        gate_kind="uniform",
        description="headline bf16 layer, 12 heads, d=128, 21x30x52 grid (32760 tokens), 10% window")
    cfgs["c4"] = LayerConfig(
        name="c4", seed=4, batch=1, heads=40, head_dim=128, T=21, H=30, W=52, block=64,
        dtype="bf16", specs=tuple(HeadSpec(TOPK, 0, -1, 0.10) for _ in range(40)),
        gate_kind="from_q",
        description="large-DiT bf16 layer, 40 heads, d=128, pooled-score top-k at 10%, gate from Q")
    rho = _c5_densities(5, 12)
    specs5 = tuple(
        HeadSpec(WINDOW, 2, -1, float(rho[h])) if h < 6 else HeadSpec(TOPK, 0, -1, float(rho[h]))
        for h in range(12))
    cfgs["c5"] = LayerConfig(
        name="c5", seed=5, batch=1, heads=12, head_dim=128, T=41, H=45, W=80, block=128,
        dtype="bf16", specs=specs5, gate_kind="uniform",
        description="long-video bf16 layer, 12 heads, d=128, 41x45x80 grid (147600 tokens), "
                    "128-token blocks, per-head density U(3%,10%), heads 0-5 window, 6-11 top-k")
    cfgs["c6"] = LayerConfig(
        name="c6", seed=6, batch=1, heads=12, head_dim=64, T=8, H=16, W=16, block=64,
        dtype="bf16", specs=tuple(HeadSpec(SICS, 0, -1, 0.10) for _ in range(12)),
        gate_kind="uniform",
        description="small bf16 layer, 12 heads, d=64, 8x16x16 grid, SICS key blocks at 10% + diagonal")
    cfgs["c7"] = LayerConfig(
        name="c7", seed=7, batch=1, heads=12, head_dim=128, T=21, H=30, W=52, block=64,
        dtype="bf16", specs=tuple(HeadSpec(SICS, 0, -1, 0.10) for _ in range(12)),
        gate_kind="uniform",
        description="bf16 layer, 12 heads, d=128, 21x30x52 grid (32760 tokens), SICS key blocks at 10% + diagonal")
    cfgs["c8"] = LayerConfig(
        name="c8", seed=8, batch=1, heads=12, head_dim=128, T=21, H=30, W=52, block=64,
        dtype="bf16", specs=tuple(HeadSpec(WINDOW, 1, -1, 0.10) for _ in range(12)),
        gate_kind="uniform", cuboid=(1, 8, 8),
        description="bf16 layer, 12 heads, d=128, 21x30x52 grid (32760 tokens), 1x8x8 cuboid blocks, "
                    "10% window")
    cfgs["c9"] = LayerConfig(
        name="c9", seed=9, batch=1, heads=4, head_dim=64, T=5, H=10, W=14, block=64,
        dtype="bf16", specs=(HeadSpec(WINDOW, 1, -1, 0.30), HeadSpec(WINDOW, 0, 2, 0.0),
                             HeadSpec(TOPK, 0, -1, 0.25), HeadSpec(SICS, 0, -1, 0.2)),
        gate_kind="from_q", cuboid=(2, 4, 8),
        description="small ragged cuboid layer, bf16, 4 heads, d=64, 5x10x14 grid, 2x4x8 cuboids, "
                    "window/top-k/SICS heads, gate from Q")
    return cfgs


CONFIGS = _build()


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
