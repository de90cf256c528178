"""Pins for the oracle's format decoders: hand-worked values, field-by-field
derivations and torch's own dtype casts (a library routine) on every code."""
import math

import numpy as np
import pytest
import torch

from oracle import codecs


def _parse(rows, base):
    out = []
    for r in rows:
        c, v = r.split()
        out.append((int(c, base), float(v)))
    return out


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_bf16_golden(golden):
    for code, val in _parse(golden("bf16_values.txt"), 16):
        got = float(codecs.bf16_to_f64(np.array([code], np.uint16))[0])
        assert _same(got, val), (hex(code), got, val)


def test_bf16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_all_finite_codes_match_field_formula():
    # sign / exponent / fraction fields of a binary32 with the low 16 bits zero
    for code in range(0, 65536, 7):
        s = -1.0 if code >> 15 else 1.0
        e = (code >> 7) & 0xFF
        f = code & 0x7F
        if e == 0xFF:
            continue
        if e == 0:
            want = s * f * 2.0 ** (-126 - 7)
        else:
            want = s * (1.0 + f / 128.0) * 2.0 ** (e - 127)
        got = float(codecs.bf16_to_f64(np.array([code], np.uint16))[0])
        assert _same(got, want), hex(code)


def test_e4m3_golden(golden):
    for code, val in _parse(golden("e4m3_values.txt"), 16):
        got = float(codecs.e4m3_to_f64(np.array([code], np.uint8))[0])
        assert _same(got, val), (hex(code), got, val)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_round_trip_through_torch_cast():
    # every finite code decodes to a value that torch's RNE cast maps back to it
    codes = np.arange(256, dtype=np.uint8)
    vals = codecs.e4m3_to_f64(codes)
    fin = ~np.isnan(vals)
    back = torch.from_numpy(vals[fin].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(back, codes[fin])


def test_e8m0_golden(golden):
    for code, val in _parse(golden("e8m0_values.txt"), 10):
        got = float(codecs.e8m0_to_f64(np.array([code], np.uint8))[0])
        assert _same(got, val), (code, got, val)


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e8m0_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_dequant_scale_indexing_closed_form():
    # q = 1.0 everywhere; SA[g][i] = 127 + g + i, SB[g][j] = 127 - j, so
    # A[i][k] = 2**(k//128 + i) and B[k][j] = 2**(-j): indexing is pinned exactly.
    M, N, K = 3, 2, 256
    qa = np.full((M, K), 0x38, np.uint8)
    qb = np.full((K, N), 0x38, np.uint8)
    sa = np.array([[127 + g + i for i in range(M)] for g in range(K // 128)], np.uint8)
    sb = np.array([[127 - j for j in range(N)] for g in range(K // 128)], np.uint8)
    A = codecs.dequant_fp8_a(qa, sa)
    B = codecs.dequant_fp8_b(qb, sb)
    for i in range(M):
        for k in range(K):
            assert A[i, k] == 2.0 ** (k // 128 + i)
    for k in range(K):
        for j in range(N):
            assert B[k, j] == 2.0 ** (-j)


@pytest.mark.parametrize("k_major", [True, False])
def test_generator_fp8_represents_the_draw(k_major):
    # the synthetic generator's bytes decode (by the oracle) to within e4m3
    # rounding of the normal draw it started from
    from synthetic import fp8_blockscaled, rng
    rows, K = 5, 384
    q, s = fp8_blockscaled(rows, K, 11, 12, k_major)
    x = rng(11).standard_normal(size=(rows, K), dtype=np.float32).astype(np.float64)
    if k_major:
        deq = codecs.dequant_fp8_a(q, s)
    else:
        deq = codecs.dequant_fp8_b(q, s).T
    big = np.abs(x) > 2.0 ** -2
    rel = np.abs(deq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12   # e4m3 keeps 3 fraction bits
    assert s.shape == (K // 128, rows) and s.min() >= 123 and s.max() <= 131
