"""Pins for the oracle GEMM: closed forms (identity, rank-1, all ones, a
block-scaled fp8 case), a pure-Python triple loop (bit-exact: same order, no
fused multiply-add) and numpy's float64 matmul (a library routine)."""
import numpy as np
import pytest

from oracle import gemm as og
from oracle.codecs import bf16_to_f64

ONE_BF16 = 0x3F80


def _bf16_bits(vals):
    import torch
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_identity_bf16():
    from synthetic import bf16_bits_normal
    K, N = 96, 40
    a = np.zeros((K, K), np.uint16)
    np.fill_diagonal(a, ONE_BF16)
    b = bf16_bits_normal((K, N), 5)
    C, S = og.gemm_bf16(a, b)
    assert np.array_equal(C, bf16_to_f64(b))
    assert np.array_equal(S, np.abs(bf16_to_f64(b)))


@pytest.mark.parametrize("K", [1, 64, 1024, 8192])
def test_rank1_closed_form(K):
    r = np.random.default_rng(K)
    M, N = 7, 9
    s = r.integers(-8, 9, size=M)
    t = r.integers(-8, 9, size=N)
    a = _bf16_bits(np.repeat(s[:, None], K, axis=1))
    b = _bf16_bits(np.repeat(t[None, :], K, axis=0))
    C, S = og.gemm_bf16(a, b)
    assert np.array_equal(C, K * np.outer(s, t).astype(np.float64))
    assert np.array_equal(S, K * np.outer(np.abs(s), np.abs(t)).astype(np.float64))


def test_all_ones():
    M, N, K = 5, 6, 777
    a = np.full((M, K), ONE_BF16, np.uint16)
    b = np.full((K, N), ONE_BF16, np.uint16)
    C, S = og.gemm_bf16(a, b)
    assert np.all(C == K) and np.all(S == K)


def test_fp8_closed_form():
    # A[i][k] = 2**(k//128 + i), B[k][j] = 2**(-j), K = 256:
    # C[i][j] = 128 * (2**i + 2**(i+1)) * 2**(-j) = 384 * 2**(i-j)
    M, N, K = 3, 2, 256
    qa = np.full((M, K), 0x38, np.uint8)
    qb = np.full((K, N), 0x38, np.uint8)
    sa = np.array([[127 + g + i for i in range(M)] for g in range(2)], np.uint8)
    sb = np.array([[127 - j for j in range(N)] for g in range(2)], np.uint8)
    C, S = og.gemm_fp8_b128(qa, sa, qb, sb)
    want = np.array([[384.0 * 2.0 ** (i - j) for j in range(N)] for i in range(M)])
    assert np.array_equal(C, want) and np.array_equal(S, want)


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (15, 17, 33), (4, 1, 65), (1, 9, 2)])
def test_brute_force_bit_exact(shape):
    M, N, K = shape
    r = np.random.default_rng(sum(shape))
    A = r.standard_normal((M, K))
    B = r.standard_normal((K, N))
    C, S = og.gemm_f64(A, B)
    Cn, Sn = og.gemm_naive(A.tolist(), B.tolist())
    assert np.array_equal(C, np.array(Cn).reshape(M, N))
    assert np.array_equal(S, np.array(Sn).reshape(M, N))


@pytest.mark.parametrize("shape", [(64, 80, 300), (129, 65, 1000)])
def test_matches_numpy_matmul(shape):
    M, N, K = shape
    r = np.random.default_rng(M)
    A = r.standard_normal((M, K))
    B = r.standard_normal((K, N))
    C, S = og.gemm_f64(A, B)
    assert np.all(np.abs(C - A @ B) <= 1e-12 * S)
    assert np.allclose(S, np.abs(A) @ np.abs(B), rtol=1e-13, atol=0)


def test_sampled_equals_full():
    r = np.random.default_rng(3)
    A = r.standard_normal((40, 70))
    B = r.standard_normal((70, 50))
    C, S = og.gemm_f64(A, B)
    rows, cols = [0, 7, 39], [1, 2, 49]
    Cs, Ss = og.gemm_f64_sampled(A, B, rows, cols)
    assert np.array_equal(Cs, C[np.ix_(rows, cols)])
    assert np.array_equal(Ss, S[np.ix_(rows, cols)])


def test_planted_mistake_is_caught():
    # a dropped term (last k) must fail the brute-force comparison
    r = np.random.default_rng(9)
    A = r.standard_normal((3, 5))
    B = r.standard_normal((5, 4))
    Cn, _ = og.gemm_naive(A.tolist(), B.tolist())
    C_bad, _ = og.gemm_f64(A[:, :4], B[:4, :])
    assert not np.array_equal(C_bad, np.array(Cn))
