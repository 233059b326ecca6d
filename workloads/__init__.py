"""Seeded synthetic inputs for the 2:4 sparse GEMM workloads.

This module is shared by the tests, the benchmark and the smoke check.  It holds
only random-number recipes and bit-pattern views: no pruning, no compression, no
quantisation and no matrix product.  Every tensor is drawn in float32 on the CPU
from a ``torch.Generator`` with a fixed seed and then rounded to bfloat16
(round-to-nearest-even, PyTorch's CPU cast).

Workloads (weights are ``[N, K]`` in the ``nn.Linear.weight`` layout, activations
``[M, K]``, and the product is ``Y = X @ W.T``):

* ``tiny``     -- X[8,256] ~ N(0,1), W[256,256] ~ N(0, 0.02^2), one generator, seed 0.
* ``up``       -- FFN up-projection, K=4096, N=14336, W ~ N(0, 0.02^2) (seed 1);
                  X[M,4096] ~ N(0,1) (seed 1000+M) with 41 outlier K-channels
                  (1% of K, chosen by ``randperm`` with seed 11) scaled by 20.
* ``down``     -- FFN down-projection, K=14336, N=4096, W ~ N(0, 0.015^2) (seed 2);
                  X[M,14336] = SiLU(N(0,1)) (seed 2000+M).
* ``prefill``  -- M=8192, K=8192, N=28672, W ~ N(0, 0.01^2) (seed 3); X ~ N(0,1) (seed 3000).
* ``layers``   -- 32 decoder layers of an 8B-class model at M=256: QKV (K=4096, N=6144),
                  O (4096 -> 4096), gate+up fused (K=4096, N=28672), down (K=14336, N=4096);
                  W ~ N(0, 0.02^2) with seed 5000 + 4*layer + proj; X seeds 4000 (N(0,1),
                  K=4096) and 4001 (SiLU(N(0,1)), K=14336).

The pages behind this library run their evaluation on trained models and
public task suites; none of that is available here, so these seeded draws stand
in for the projection weights and activations of such a model.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "randn_bf16", "bf16_bits", "bits_to_bf16",
    "tiny", "up_weight", "up_x", "down_weight", "down_x",
    "prefill_weight", "prefill_x", "LAYER_PROJS", "layer_weight", "layer_x",
    "UP", "DOWN", "PREFILL", "TINY",
]

# (M, K, N) of each workload; decode workloads list their token counts.
TINY = dict(M=8, K=256, N=256)
UP = dict(Ms=(1, 16, 64), K=4096, N=14336)
DOWN = dict(Ms=(1, 16, 64), K=14336, N=4096)
PREFILL = dict(M=8192, K=8192, N=28672)
LAYER_PROJS = (("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672),
               ("down", 14336, 4096))
LAYER_M = 256
N_LAYERS = 32


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def randn_bf16(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    """float32 N(0, std^2) samples from a fresh generator, rounded to bfloat16."""
    x = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a CPU bfloat16 tensor, as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(bits: np.ndarray) -> torch.Tensor:
    """Inverse of :func:`bf16_bits`."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)


def tiny():
    """X[8,256] ~ N(0,1) then W[256,256] ~ N(0,0.02^2) from one generator (seed 0)."""
    g = _gen(0)
    x = torch.randn(8, 256, generator=g, dtype=torch.float32)
    w = torch.randn(256, 256, generator=g, dtype=torch.float32) * 0.02
    return x.to(torch.bfloat16), w.to(torch.bfloat16)


def up_weight() -> torch.Tensor:
    return randn_bf16((UP["N"], UP["K"]), seed=1, std=0.02)


def up_outlier_channels(k: int = 4096) -> torch.Tensor:
    n_out = int(round(0.01 * k))
    return torch.randperm(k, generator=_gen(11))[:n_out]


def up_x(m: int) -> torch.Tensor:
    k = UP["K"]
    x = torch.randn(m, k, generator=_gen(1000 + m), dtype=torch.float32)
    x[:, up_outlier_channels(k)] *= 20.0
    return x.to(torch.bfloat16)


def down_weight() -> torch.Tensor:
    return randn_bf16((DOWN["N"], DOWN["K"]), seed=2, std=0.015)


def down_x(m: int) -> torch.Tensor:
    x = torch.randn(m, DOWN["K"], generator=_gen(2000 + m), dtype=torch.float32)
    return torch.nn.functional.silu(x).to(torch.bfloat16)


def prefill_weight() -> torch.Tensor:
    return randn_bf16((PREFILL["N"], PREFILL["K"]), seed=3, std=0.01)


def prefill_x() -> torch.Tensor:
    return randn_bf16((PREFILL["M"], PREFILL["K"]), seed=3000)


def layer_weight(layer: int, proj: int) -> torch.Tensor:
    _, k, n = LAYER_PROJS[proj]
    return randn_bf16((n, k), seed=5000 + 4 * layer + proj, std=0.02)


def layer_x(k: int) -> torch.Tensor:
    if k == 4096:
        return randn_bf16((LAYER_M, 4096), seed=4000)
    x = torch.randn(LAYER_M, k, generator=_gen(4001), dtype=torch.float32)
    return torch.nn.functional.silu(x).to(torch.bfloat16)
