"""Seeded synthetic inputs shaped like the workloads the BitNet b1.58 pages
discuss (a 3B-shaped block with hidden 3200 / FFN 8640, a 70B-shaped block with
hidden 8192 / FFN 28672 and grouped-query k/v of width 1024, and a hidden 4096 /
FFN 11008 block).

This module holds random number generation only -- none of the method's
arithmetic -- and is the one place both the product path (benchmark, GPU
tests) and the CPU oracle side take their inputs from.

Conventions
-----------
* Every latent weight matrix is stored ``[N][K]`` (out x in, as nn.Linear
  stores it); a shape written "K->N" maps K input features to N outputs.
* Host tensors come from ``numpy.random.default_rng`` (PCG64).  The single
  2048x2048 layer uses ``default_rng(0)`` and draws W first, then x.  Every
  other tensor uses ``default_rng([config, layer, proj, role, M])`` with
  ``role`` 0 = W, 1 = x, 2 = outlier channel set, 3 = gamma (M = 0 for the
  weight roles).
* The 70B-shaped sweep holds 68.45 G latent weights (274 GB as float32), far
  beyond what a host generator can produce in a benchmark's setup time.  Its
  latent matrices are drawn on the GPU by ``torch.randn`` under a seeded
  ``torch.Generator``, one matrix at a time; a test that needs one on the host
  copies that generator's output back (the generator, not the method, made
  it).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

W_STD = np.float32(0.02)

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
ROLE_W, ROLE_X, ROLE_OUTLIER, ROLE_GAMMA = 0, 1, 2, 3


@dataclass(frozen=True)
class Proj:
    name: str
    index: int
    K: int  # input features
    N: int  # output features


def block_projections(hidden: int, ffn: int, kv: Optional[int] = None) -> List[Proj]:
    """The seven linear projections of a transformer block."""
    kv = hidden if kv is None else kv
    shapes = [(hidden, hidden), (hidden, kv), (hidden, kv), (hidden, hidden),
              (hidden, ffn), (hidden, ffn), (ffn, hidden)]
    return [Proj(n, i, K, N) for i, (n, (K, N)) in enumerate(zip(PROJ_NAMES, shapes))]


# Config 2: 3B-shaped block, hidden 3200, FFN 8640.
C2_PROJS = block_projections(3200, 8640)
# Config 4: 70B-shaped block, hidden 8192, FFN 28672, GQA k/v 1024; 80 layers.
C4_PROJS = block_projections(8192, 28672, kv=1024)
C4_LAYERS = 80
# Config 5: hidden 4096, FFN 11008.
C5_PROJS = block_projections(4096, 11008)
# Config 3: prefill GEMMs, M = 2048 tokens.
C3_SHAPES = [(3200, 8640), (8640, 3200)]  # (K, N)
C3_M = 2048


def _rng(config: int, layer: int, proj: int, role: int, M: int) -> np.random.Generator:
    return np.random.default_rng([config, layer, proj, role, M])


def normal_f32(rng: np.random.Generator, shape, scale=None) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale is not None:
        a *= np.float32(scale)
    return a


# ---------------------------------------------------------------- config 1
def c1_inputs() -> Tuple[np.ndarray, np.ndarray]:
    """Single BitLinear layer, M=1: W [2048][2048] ~ N(0, 0.02), x [1][2048] ~ N(0,1), seed 0."""
    rng = np.random.default_rng(0)
    W = normal_f32(rng, (2048, 2048), W_STD)
    x = normal_f32(rng, (1, 2048))
    return W, x


# ---------------------------------------------------------------- generic
def latent_weight(config: int, layer: int, proj: Proj) -> np.ndarray:
    return normal_f32(_rng(config, layer, proj.index, ROLE_W, 0), (proj.N, proj.K), W_STD)


def activations_normal(config: int, layer: int, proj_index: int, M: int, K: int) -> np.ndarray:
    return normal_f32(_rng(config, layer, proj_index, ROLE_X, M), (M, K))


# ---------------------------------------------------------------- config 2
def c2_weight(proj: Proj) -> np.ndarray:
    return latent_weight(2, 0, proj)


def c2_x(proj: Proj, M: int) -> np.ndarray:
    return activations_normal(2, 0, proj.index, M, proj.K)


# ---------------------------------------------------------------- config 3
def c3_inputs(p: int) -> Tuple[np.ndarray, np.ndarray]:
    """Prefill GEMM p (0: 3200->8640, 1: 8640->3200): x Student-t(3) [2048][K], W ~ N(0,0.02)."""
    K, N = C3_SHAPES[p]
    W = normal_f32(_rng(3, 0, p, ROLE_W, 0), (N, K), W_STD)
    x = _rng(3, 0, p, ROLE_X, C3_M).standard_t(3, size=(C3_M, K)).astype(np.float32)
    return W, x


# ---------------------------------------------------------------- config 4
def c4_x(layer: int, proj: Proj, M: int) -> np.ndarray:
    return activations_normal(4, layer, proj.index, M, proj.K)


def c4_seed(layer: int, proj: Proj) -> int:
    return 4_000_000 + 16 * layer + proj.index


def c4_weight_device(layer: int, proj: Proj, device="cuda"):
    """Latent W [N][K] ~ N(0, 0.02) drawn on the GPU by torch.randn (seeded)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(c4_seed(layer, proj))
    W = torch.randn((proj.N, proj.K), generator=g, device=device, dtype=torch.float32)
    W.mul_(float(W_STD))
    return W


# ---------------------------------------------------------------- config 5
def c5_ternary(proj: Proj) -> Tuple[np.ndarray, np.float32]:
    """Ternary weights drawn directly: P(0)=0.6, P(+1)=P(-1)=0.2; gamma ~ U(0.01, 0.05)."""
    u = _rng(5, 0, proj.index, ROLE_W, 0).random((proj.N, proj.K))
    Wt = np.where(u < 0.6, 0, np.where(u < 0.8, 1, -1)).astype(np.int8)
    gamma = np.float32(_rng(5, 0, proj.index, ROLE_GAMMA, 0).uniform(0.01, 0.05))
    return Wt, gamma


def c5_outlier_channels(proj: Proj) -> np.ndarray:
    n = int(round(0.01 * proj.K))
    return np.sort(_rng(5, 0, proj.index, ROLE_OUTLIER, 0).choice(proj.K, size=n, replace=False))


def c5_x(proj: Proj, M: int) -> np.ndarray:
    """x ~ N(0,1) with 1% of the input channels (fixed per projection) scaled by 20."""
    x = activations_normal(5, 0, proj.index, M, proj.K)
    x[:, c5_outlier_channels(proj)] *= np.float32(20.0)
    return x


# ---------------------------------------------------------------- misc
def random_latent(seed: int, N: int, K: int, std=W_STD) -> np.ndarray:
    return normal_f32(np.random.default_rng(seed), (N, K), std)


def random_x(seed: int, M: int, K: int, dist: str = "normal") -> np.ndarray:
    rng = np.random.default_rng(seed)
    if dist == "normal":
        return normal_f32(rng, (M, K))
    if dist == "t3":
        return rng.standard_t(3, size=(M, K)).astype(np.float32)
    raise ValueError(dist)


def random_ternary(seed: int, N: int, K: int, p_zero: float = 1.0 / 3.0) -> np.ndarray:
    u = np.random.default_rng(seed).random((N, K))
    p1 = p_zero + (1.0 - p_zero) / 2
    return np.where(u < p_zero, 0, np.where(u < p1, 1, -1)).astype(np.int8)
