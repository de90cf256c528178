"""Decoders for the stored operand formats, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

* bf16: the upper 16 bits of an IEEE binary32; value = float32(bits << 16).
* e4m3 (OCP FP8 E4M3, "fn" variant: bias 7, no infinities, S.1111.111 is NaN):
  exponent field 0 -> subnormal 2**-6 * m/8; 1..15 -> 2**(e-7) * (1 + m/8).
  This is the element format of the MXFP8 operands in "[Feature] Introduce
  tile scheduler" (TileLang PR #2441), example header.
* e8m0 (scale byte of the (1, 1, 128) block scale in the same example):
  value 2**(b - 127); b = 255 is NaN.
"""
from __future__ import annotations

import numpy as np

SCALE_BLOCK_K = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact values as fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # signalling-NaN codes stay NaN
        return b.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (2.0 ** -6) * (m / 8.0)
        else:
            t[code] = s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return t


E4M3_TABLE = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    out = np.exp2(c - 127.0)
    out[c == 255.0] = np.nan
    return out


def dequant_fp8_a(q: np.ndarray, sa: np.ndarray) -> np.ndarray:
    """A[i][k] = e4m3(q[i][k]) * 2**(SA[k // 128][i] - 127); q is [M][K], SA [K/128][M]."""
    vals = e4m3_to_f64(q)
    scale = e8m0_to_f64(sa).T                        # [M][K/128]
    return vals * np.repeat(scale, SCALE_BLOCK_K, axis=1)


def dequant_fp8_b(q: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """B[k][j] = e4m3(q[k][j]) * 2**(SB[k // 128][j] - 127); q is [K][N], SB [K/128][N]."""
    vals = e4m3_to_f64(q)
    return vals * np.repeat(e8m0_to_f64(sb), SCALE_BLOCK_K, axis=0)
