"""The five measured workloads: shapes, tile sizes, seeds and value recipes.

Seeds follow one rule: operand A of workload c uses 1000 + 10*c, operand B
that seed + 1, block-scale exponents of A and B that seed + 2 and + 3; the
add uses 2001 (X) and 2002 (Y).  Nothing here computes anything.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class GemmShape:
    M: int
    N: int
    K: int


@dataclass(frozen=True)
class GemmWorkload:
    name: str
    cfg: int                 # workload number (seed base 1000 + 10*cfg)
    dtype: str               # "bf16_out_f32" | "bf16_out_bf16" | "fp8_b128_out_bf16"
    shapes: tuple
    tile: tuple              # (BM, BN, BK)
    dist: str                # "uniform" | "normal" | "fp8_normal_scaled"
    scheds: tuple = field(default_factory=tuple)

    def seeds(self, which: int = 0):
        a = 1000 + 10 * self.cfg + 100 * which
        return {"A": a, "B": a + 1, "SA": a + 2, "SB": a + 3}


ALL_SCHEDS = ("blocked", "interleaved", "grouped", "work_stealing")

GEMM_512 = GemmWorkload(
    "bf16 GEMM 512^3, fp32 C, 128x128x64 tiles", 1, "bf16_out_f32",
    (GemmShape(512, 512, 512),), (128, 128, 64), "uniform", ("blocked",))

GEMM_8192 = GemmWorkload(
    "bf16 GEMM 8192^3, bf16 C, 256x256x64 tiles", 3, "bf16_out_bf16",
    (GemmShape(8192, 8192, 8192),), (256, 256, 64), "normal", ALL_SCHEDS)

GEMM_RAGGED = GemmWorkload(
    "bf16 GEMM ragged shapes, bf16 C, 256x256x64 tiles", 4, "bf16_out_bf16",
    (GemmShape(5120, 5120, 4096), GemmShape(4864, 8000, 8192),
     GemmShape(3000, 7000, 2048)), (256, 256, 64), "uniform", ALL_SCHEDS)

GEMM_FP8_SKINNY = GemmWorkload(
    "block-scaled fp8 e4m3 GEMM 256x28672x8192, bf16 C, 128x128x128 tiles", 5,
    "fp8_b128_out_bf16", (GemmShape(256, 28672, 8192),), (128, 128, 128),
    "fp8_normal_scaled", ("grouped", "work_stealing"))

GEMM_FP8_SQUARE = GemmWorkload(
    "block-scaled fp8 e4m3 GEMM 8192^3, bf16 C, 256x256x128 tiles", 5,
    "fp8_b128_out_bf16", (GemmShape(8192, 8192, 8192),), (256, 256, 128),
    "fp8_normal_scaled", ("grouped", "work_stealing"))

ADD_ROWS, ADD_COLS = 8192, 8192
ADD_TILES = ((32, 16), (128, 128))
ADD_SEEDS = {"X": 2001, "Y": 2002}
