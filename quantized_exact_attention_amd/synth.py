"""Seeded synthetic inputs for the attention workloads (no method arithmetic).

The pages' workload is the attention of a video diffusion transformer whose
canonical tensors are not available ("Experiment Log", Phase 0 Import And
Verification records them as missing), so seeded Gaussian stand-ins are drawn
with the shapes below.  K carries a per-channel bias so that K smoothing has
something to remove; some workloads scale a small fraction of Q/K entries by
20 to create outliers for the per-block INT8 scales.

Draw order for workload k, from ``torch.Generator().manual_seed(1000 + k)`` on
the CPU: Q, K, V ~ N(0, 1) float32; outlier masks for Q then K (uniform < p),
masked entries x20; bias = 2 * N(0, 1) of shape [B, H, 1, D] added to K; cast
to bfloat16 (round to nearest even).

This module is shared by the tests (which also feed the oracle) and by the
benchmark.  It only draws random numbers.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    Nq: int
    Nkv: int
    D: int
    outlier_p: float
    description: str

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def flops(self) -> float:
        """Effective attention FLOP count 4*B*H*Nq*Nkv*D (QK and PV, dense)."""
        return 4.0 * self.B * self.H * self.Nq * self.Nkv * self.D


WORKLOADS = {
    w.name: w for w in [
        Workload("single_tile", 0, 1, 1, 128, 192, 128, 0.0,
                 "single Q128 x KV192 x D128 tile, non-causal"),
        Workload("ragged_tails", 1, 1, 8, 1000, 1000, 128, 0.03,
                 "ragged tails, 3% Q/K outliers x20"),
        Workload("dit_block", 2, 2, 24, 4096, 4096, 128, 0.0,
                 "DiT-style block attention"),
        Workload("long_video", 3, 1, 24, 32760, 32760, 128, 0.0,
                 "long video-token sequence, N not a multiple of the tile"),
        Workload("headdim64", 4, 4, 16, 16383, 16383, 64, 0.01,
                 "head-dim 64, 1% Q/K outliers x20"),
    ]
}


def make_inputs(w: Workload, seed: int | None = None, B=None, H=None, Nq=None, Nkv=None, D=None):
    """Draw (q, k, v) bfloat16 CPU tensors [B, H, N, D] for workload ``w``.

    Shape overrides allow small cases with the same distribution.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    Nq = w.Nq if Nq is None else Nq
    Nkv = w.Nkv if Nkv is None else Nkv
    D = w.D if D is None else D
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    q = torch.randn(B, H, Nq, D, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, Nkv, D, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, Nkv, D, generator=g, dtype=torch.float32)
    if w.outlier_p > 0:
        mq = torch.rand(B, H, Nq, D, generator=g) < w.outlier_p
        mk = torch.rand(B, H, Nkv, D, generator=g) < w.outlier_p
        q = torch.where(mq, q * 20.0, q)
        k = torch.where(mk, k * 20.0, k)
    bias = 2.0 * torch.randn(B, H, 1, D, generator=g, dtype=torch.float32)
    k = k + bias
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
