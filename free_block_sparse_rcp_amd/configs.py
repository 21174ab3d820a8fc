"""The SparsePR workloads used by the tests and the bench.

Shapes, head counts, head dims, densities and probe budgets are those of the
four model families the pages evaluate on (skillfed article, results
paragraph; arxivdaily 2608.18484, English abstract) restated as synthetic
calls; grid shapes and the parameters the pages leave open are this build's
choices. Inputs come from ``inputs.py``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

from . import inputs as _inputs


@dataclass
class Params:
    """Mirror of the C ``sparsepr_params`` struct."""

    heads: int
    n_tokens: int
    head_dim: int
    dtype: str               # "f32" | "bf16"
    q_block: int             # B_q
    n_groups: int            # G
    n_samples: int           # S
    kmeans_iters: int        # T
    density: float           # rho, executed-pair density including probes
    n_probes: int            # m
    rank: int                # k
    ridge_lambda: float      # lambda
    partition_mode: int = 0  # 0 response-coupled, 1 random-block, 2 semantic comparator

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // self.q_block)

    @property
    def key_budget(self) -> int:
        """Per-row key budget kappa = floor(rho * N - m)."""
        return int(math.floor(self.density * self.n_tokens - self.n_probes))


@dataclass
class Workload:
    name: str
    grid: Tuple[int, int, int]
    params: Params
    scales: Sequence[float]
    generator: str            # "g1" | "g2"
    seed: int
    blur: Tuple[float, float, float] = (1.5, 3.0, 3.0)
    key_smoothing: bool = False
    description: str = ""

    def make_inputs(self, heads: Optional[Sequence[int]] = None) -> _inputs.Inputs:
        p = self.params
        if self.generator == "g1":
            assert p.heads == 1
            return _inputs.gen_g1(self.grid, p.head_dim, p.n_samples, p.n_groups, self.seed,
                                  self.scales[0], p.dtype)
        return _inputs.gen_g2(self.grid, p.head_dim, p.heads, p.n_samples, p.n_groups,
                              self.seed, self.scales, self.blur, self.key_smoothing,
                              p.dtype, heads)

    def with_params(self, **kw) -> "Workload":
        return replace(self, params=replace(self.params, **kw))


def _n(grid):
    return grid[0] * grid[1] * grid[2]


_R128 = 1.0 / math.sqrt(128.0)

TINY = Workload(
    name="tiny_f32_n2048_d64", grid=(8, 16, 16),
    params=Params(heads=1, n_tokens=2048, head_dim=64, dtype="f32", q_block=64, n_groups=32,
                  n_samples=128, kmeans_iters=8, density=0.25, n_probes=64, rank=16,
                  ridge_lambda=1e-3),
    scales=[1.0 / 8.0], generator="g1", seed=1,
    description="single head, fp32, N=2048 on 8x16x16, d=64")

WAN = Workload(
    name="wan22_bf16_h40_n32760", grid=(21, 30, 52),
    params=Params(heads=40, n_tokens=_n((21, 30, 52)), head_dim=128, dtype="bf16", q_block=128,
                  n_groups=256, n_samples=512, kmeans_iters=8, density=0.22, n_probes=128,
                  rank=32, ridge_lambda=1e-3),
    scales=[_R128] * 40, generator="g2", seed=2, blur=(1.5, 3.0, 3.0),
    description="Wan2.2-I2V-shaped: 40 heads, N=32760 on 21x30x52, d=128, 22% density")

HUNYUAN = Workload(
    name="hunyuan_bf16_h24_n118800", grid=(33, 45, 80),
    params=Params(heads=24, n_tokens=_n((33, 45, 80)), head_dim=128, dtype="bf16", q_block=128,
                  n_groups=512, n_samples=512, kmeans_iters=8, density=0.22, n_probes=128,
                  rank=32, ridge_lambda=1e-3),
    scales=[_R128] * 24, generator="g2", seed=3, blur=(3.0, 6.0, 6.0), key_smoothing=True,
    description="HunyuanVideo-13B-shaped: 24 heads, N=118800 on 33x45x80, d=128, 22% density")

COSMOS = Workload(
    name="cosmos_bf16_h40_n45056", grid=(22, 32, 64),
    params=Params(heads=40, n_tokens=_n((22, 32, 64)), head_dim=128, dtype="bf16", q_block=128,
                  n_groups=256, n_samples=512, kmeans_iters=8, density=0.26, n_probes=192,
                  rank=48, ridge_lambda=1e-3),
    scales=[0.3 * _R128] * 40, generator="g2", seed=4, blur=(1.5, 3.0, 3.0),
    description="broad-row Cosmos-like: 40 heads, N=45056 on 22x32x64, d=128, tau=0.3/sqrt(d)")

SWEEP = Workload(
    name="sweep_bf16_h32_n65536", grid=(16, 64, 64),
    params=Params(heads=32, n_tokens=_n((16, 64, 64)), head_dim=128, dtype="bf16", q_block=128,
                  n_groups=512, n_samples=512, kmeans_iters=8, density=0.22, n_probes=128,
                  rank=32, ridge_lambda=1e-3),
    scales=[2.0 * _R128] * 16 + [0.3 * _R128] * 16, generator="g2", seed=5,
    blur=(1.5, 3.0, 3.0),
    description="sensitivity sweep: 32 heads (16 concentrated, 16 broad), N=65536 on 16x64x64")

SWEEP_PROBES = (32, 64, 128, 256)
SWEEP_DENSITIES = (0.15, 0.22, 0.30)

WORKLOADS = {w.name: w for w in (TINY, WAN, HUNYUAN, COSMOS, SWEEP)}
ALIASES = {"tiny": TINY.name, "wan": WAN.name, "hunyuan": HUNYUAN.name,
           "cosmos": COSMOS.name, "sweep": SWEEP.name}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]
