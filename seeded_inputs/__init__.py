"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds no arithmetic of the method: it only draws random matrices,
rounds them to the storage type, and lists the workload shapes.  Both the HIP
path and the oracle consume exactly the half-precision values produced here
(the oracle widens them to fp64 exactly).

Recipe (the same for every caller):

* ``numpy.random.default_rng(seed)`` (PCG64); fp64 samples, A first, then B,
  from the same stream; scale first, then round once to the storage type.
  binary16: numpy's float64 -> float16 conversion (round to nearest even).
  bfloat16: float64 -> float32 (numpy) -> bfloat16 (torch, round to nearest even).
* distributions:
    ``uniform``      U(-1, 1)                      (square FP16 workloads)
    ``int2``         integers in {-2..2}            (exact-equality variant)
    ``int1``         integers in {-1, 0, 1}         (exact bfloat16 variant)
    ``normal_sqrtk`` N(0, 1) / sqrt(K)              (large square BF16 workloads)
    ``decode``       A ~ N(0, 1), B ~ N(0, 0.02^2)  (skinny decode GEMMs)

The 24-shape sweep draws (M, N, K) without replacement from the 1000 triples
over {64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384}^3 (the grid of
the CUDA-L2 explanation, section "方法论"), ordered lexicographically, with
``default_rng(0).choice(1000, 24, replace=False)``; the data seed of sweep
shape i is 1000 + i.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
SWEEP_SIZES = (64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384)


def _round_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.float16)))
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.float32))).to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw(rng, shape, dist: str, K: int, which: str) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "int2":
        return rng.integers(-2, 3, size=shape).astype(np.float64)
    if dist == "int1":
        return rng.integers(-1, 2, size=shape).astype(np.float64)
    if dist == "normal_sqrtk":
        return rng.standard_normal(size=shape) / np.sqrt(max(K, 1))
    if dist == "decode":
        x = rng.standard_normal(size=shape)
        return x if which == "A" else 0.02 * x
    raise ValueError(f"unknown distribution {dist!r}")


def gen(M: int, N: int, K: int, dtype: str = "f16", dist: str = "uniform", seed: int = 0):
    """Return (A, B) as CPU torch tensors of the storage type, A: M x K, B: K x N."""
    rng = np.random.default_rng(seed)
    A = _draw(rng, (M, K), dist, K, "A")
    B = _draw(rng, (K, N), dist, K, "B")
    return _round_storage(A, dtype), _round_storage(B, dtype)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a half-precision tensor (widening is exact)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """The 16-bit patterns of a half-precision tensor."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def sweep_shapes(n: int = 24, seed: int = 0):
    grid = list(itertools.product(SWEEP_SIZES, repeat=3))
    idx = np.random.default_rng(seed).choice(len(grid), n, replace=False)
    return [tuple(int(v) for v in grid[i]) for i in idx]


# The workloads, by what they are.
SQUARE_512_F16 = dict(M=512, N=512, K=512, dtype="f16", dist="uniform", seed=0)
SQUARE_512_F16_INT = dict(M=512, N=512, K=512, dtype="f16", dist="int2", seed=0)
SQUARE_4096_BF16 = dict(M=4096, N=4096, K=4096, dtype="bf16", dist="normal_sqrtk", seed=0)
SQUARE_16384_BF16 = dict(M=16384, N=16384, K=16384, dtype="bf16", dist="normal_sqrtk", seed=0)
SQUARE_32768_BF16 = dict(M=32768, N=32768, K=32768, dtype="bf16", dist="normal_sqrtk", seed=0)
DECODE_MS = (1, 4, 16, 64)


def decode_shape(m: int):
    return dict(M=m, N=14336, K=4096, dtype="bf16", dist="decode", seed=0)


def decode_long_k_shape(m: int):
    """The same layer's product with N and K exchanged: few column strips over a long K."""
    return dict(M=m, N=4096, K=14336, dtype="bf16", dist="decode", seed=0)


def sweep_workloads():
    return [dict(M=M, N=N, K=K, dtype="f16", dist="uniform", seed=1000 + i)
            for i, (M, N, K) in enumerate(sweep_shapes())]
