"""Seeded synthetic inputs shared by the GPU path and the oracle.

This module only draws random numbers and packs them into the storage formats
the GEMM and the add consume (bf16 bit patterns, OCP e4m3 bytes, e8m0 scale
bytes, fp32 arrays).  It holds none of the method's arithmetic: no product,
no sum, no scheduling.  Every array is a NumPy array on the host; callers move
it to the device (GPU side) or decode it (oracle side) themselves.

Generator: ``numpy.random.Generator(PCG64(seed))``.  Rounding of fp32 draws to
bf16 and to e4m3 is done by torch's dtype casts (round to nearest even), so
both sides see exactly the same stored bits.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "rng",
    "bf16_bits_uniform",
    "bf16_bits_normal",
    "bf16_bits_from_f32",
    "f32_normal",
    "fp8_blockscaled",
    "SCALE_BLOCK_K",
]

#: K elements that share one e8m0 scale (block-scale shape (1, 1, 128)).
SCALE_BLOCK_K = 128


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE, via torch) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_uniform(shape, seed: int) -> np.ndarray:
    """iid uniform[-1, 1) drawn in fp32, rounded to bf16; uint16 bit patterns."""
    x = rng(seed).uniform(-1.0, 1.0, size=shape).astype(np.float32)
    return bf16_bits_from_f32(x)


def bf16_bits_normal(shape, seed: int) -> np.ndarray:
    """iid normal(0, 1) drawn in fp32, rounded to bf16; uint16 bit patterns."""
    x = rng(seed).standard_normal(size=shape, dtype=np.float32)
    return bf16_bits_from_f32(x)


def f32_normal(shape, seed: int) -> np.ndarray:
    """iid normal(0, 1) in fp32."""
    return rng(seed).standard_normal(size=shape, dtype=np.float32)


def fp8_blockscaled(rows: int, k: int, seed_vals: int, seed_exps: int,
                    k_major: bool):
    """Block-scaled e4m3 operand with one power-of-two scale per 128 K.

    Draws x ~ normal(0, 1) in fp32 and, per (row, 128-K block), an integer
    exponent e uniform in [-4, 4].  Stores q = e4m3(clamp(x / 2**e, +-448))
    (torch cast, RNE) and the e8m0 scale byte e + 127, so q * 2**(byte-127)
    approximates x.

    ``k_major=True``  returns q laid out [rows][k]   (operand A, row-major).
    ``k_major=False`` returns q laid out [k][rows]   (operand B, row-major
    [K][N] with ``rows`` = N).
    The scale array is always [k / 128][rows] (K-group-major), uint8.
    """
    if k % SCALE_BLOCK_K:
        raise ValueError("K must be a multiple of 128 for block scales")
    g = rng(seed_vals)
    x = g.standard_normal(size=(rows, k), dtype=np.float32)
    e = rng(seed_exps).integers(-4, 5, size=(rows, k // SCALE_BLOCK_K))
    denom = np.repeat(np.exp2(e).astype(np.float32), SCALE_BLOCK_K, axis=1)
    y = np.clip(x / denom, -448.0, 448.0)
    if not k_major:
        y = np.ascontiguousarray(y.T)
    q = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    scale = np.ascontiguousarray((e + 127).astype(np.uint8).T)
    return q, scale
