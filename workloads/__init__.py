"""Seeded synthetic inputs for the SLiM compressed linear layer.

This module only draws random tensors with the shapes and distributions of the
workloads; it holds none of the layer's arithmetic (no quantisation, pruning,
packing or products).  Both the CPU oracle tests and the GPU path (tests and
benchmark) take their inputs from here, so the two sides see identical bytes.

Workload shapes follow the LLaMA-2-7B linear layers that the SLiM layer-wise
speed-ups are quoted on (Compression Trinity, Table 7.7 and Fig. E.1 captions;
page 4 "developinglight" summary: 4-bit weight-only quantisation with group 128,
adapters at 10% of the hidden size).  The pages' own evaluation used trained
LLaMA-2 weights and C4 calibration data; synthetic Gaussian tensors of the same
shapes stand in for them.

Recipe (one ``numpy.random.default_rng(seed)`` per case, fixed draw order):
  1. X  ~ N(0, 1)    float32 [M, K]   -> float16 (round to nearest even)
  2. W  ~ N(0, 0.02) float32 [N, K]   (kept in float32: it is the pack input)
  3. outlier input columns (gate/up case only): round(0.01*K) distinct column
     indices drawn without replacement; those columns of W are multiplied by 20
  4. L  ~ N(0, 0.02) float32 [K, r]   -> float16
  5. R  ~ N(0, 0.02) float32 [r, N]   -> float16
"""
from __future__ import annotations

import dataclasses
from typing import Iterator

import numpy as np

GROUP = 128
HIDDEN = 4096          # LLaMA-2-7B hidden size
MLP = 11008            # LLaMA-2-7B SwiGLU intermediate size
RANK = 416             # 10% of 4096 = 409.6, rounded up to a multiple of 32


@dataclasses.dataclass(frozen=True)
class Case:
    """One linear-layer problem: Y[M,N] = X[M,K] . W[N,K]^T (+ adapter)."""
    name: str
    M: int
    N: int
    K: int
    r: int
    seed: int = 0
    outlier_frac: float = 0.0     # fraction of input columns scaled by 20
    w_std: float = 0.02
    lr_std: float = 0.02

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.K))

    def with_M(self, M: int) -> "Case":
        return dataclasses.replace(self, M=M, name=f"{self.name.split('@')[0]}@M{M}")


# The five configurations of the workload (seed 0 throughout).
TINY = Case("tiny", M=16, N=512, K=512, r=32)
QPROJ = Case("q_proj", M=1, N=HIDDEN, K=HIDDEN, r=RANK)
GATEUP = Case("gate_up", M=16, N=MLP, K=HIDDEN, r=RANK, outlier_frac=0.01)
DOWN = Case("down", M=2048, N=HIDDEN, K=MLP, r=RANK)

BLOCK_LAYERS = {
    # LLaMA-2-7B decoder block: (N = d_out, K = d_in)
    "q_proj": (HIDDEN, HIDDEN),
    "k_proj": (HIDDEN, HIDDEN),
    "v_proj": (HIDDEN, HIDDEN),
    "o_proj": (HIDDEN, HIDDEN),
    "gate_proj": (MLP, HIDDEN),
    "up_proj": (MLP, HIDDEN),
    "down_proj": (HIDDEN, MLP),
}
SWEEP_M = (1, 16, 256, 2048)


def block_sweep() -> Iterator[Case]:
    """The decoder-block sweep: every layer shape at every token count."""
    for M in SWEEP_M:
        for name, (N, K) in BLOCK_LAYERS.items():
            yield Case(f"{name}@M{M}", M=M, N=N, K=K, r=RANK)


def all_configs() -> list[Case]:
    return [TINY, QPROJ, QPROJ.with_M(16), GATEUP, DOWN]


@dataclasses.dataclass
class Inputs:
    X: np.ndarray          # float16 [M, K]
    W: np.ndarray          # float32 [N, K]
    L: np.ndarray          # float16 [K, r]
    R: np.ndarray          # float16 [r, N]
    outlier_cols: np.ndarray  # int64 [n_outliers]


def make_inputs(case: Case) -> Inputs:
    """Draw X, W, L, R for ``case`` in the fixed order documented above."""
    rng = np.random.default_rng(case.seed)
    X = rng.standard_normal((case.M, case.K), dtype=np.float32).astype(np.float16)
    W = rng.standard_normal((case.N, case.K), dtype=np.float32)
    W *= np.float32(case.w_std)
    cols = np.zeros(0, dtype=np.int64)
    if case.n_outliers > 0:
        cols = np.sort(rng.choice(case.K, size=case.n_outliers, replace=False))
        W[:, cols] *= np.float32(20.0)
    L = (rng.standard_normal((case.K, case.r), dtype=np.float32)
         * np.float32(case.lr_std)).astype(np.float16)
    R = (rng.standard_normal((case.r, case.N), dtype=np.float32)
         * np.float32(case.lr_std)).astype(np.float16)
    return Inputs(X=X, W=W, L=L, R=R, outlier_cols=cols)


def random_weights(rng: np.random.Generator, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """Gaussian float32 weights [N, K] from an existing generator."""
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(std)
    return W


def random_fp16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float16)
