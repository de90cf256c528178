"""GPU parity of the persistent bf16 GEMM against the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import gemm as og
from synthetic import bf16_bits_normal, bf16_bits_uniform
from tests.gpu_util import (BF16_TOL, Guarded, assert_abs_bound, assert_within, config,
                            dev_bf16, note, sync)

pytestmark = pytest.mark.gpu

SCHEDS = ["blocked", "interleaved", "grouped", "work_stealing", "blocked_grouped", "work_stealing_xcc"]
EDGE = [1, 2, 15, 63, 64, 65, 127, 128, 129, 255, 257]


def _shapes():
    # every edge value in every position, plus a few mixed triples
    out = set()
    for i, v in enumerate(EDGE):
        out.add((v, EDGE[(i + 3) % len(EDGE)], EDGE[(i + 7) % len(EDGE)]))
        out.add((EDGE[(i + 5) % len(EDGE)], v, EDGE[(i + 2) % len(EDGE)]))
        out.add((EDGE[(i + 1) % len(EDGE)], EDGE[(i + 9) % len(EDGE)], v))
    out |= {(257, 257, 257), (1, 1, 1), (64, 64, 64), (129, 255, 65)}
    return sorted(out)


def run_gemm(a_bits, b_bits, M, N, K, out, sched, tile, **kw):
    cfg = config()
    A = dev_bf16(a_bits)
    B = dev_bf16(b_bits)
    C = Guarded(M * N, "bf16" if out == "bf16_out_bf16" else "f32")
    args = pg.make_args(tile=tile, **kw)
    note(f"pgemm_run M={M} N={N} K={K} {out} sched={sched} tile={tile} {kw}")
    pg.pgemm_run(cfg, A, B, C.view, M, N, K, out, sched, args)
    sync()
    return C


@pytest.mark.parametrize("staged", [False, True], ids=["lds_dma", "register_staged"])
@pytest.mark.parametrize("tile", [(128, 128, 64), (256, 256, 64)])
@pytest.mark.parametrize("out", ["bf16_out_f32", "bf16_out_bf16"])
def test_brute_force_shapes(tile, out, staged):
    flags = pg._abi.DEBUG_REGISTER_STAGED if staged else 0
    for si, (M, N, K) in enumerate(_shapes()):
        a = bf16_bits_uniform((M, K), 7 + si)
        b = bf16_bits_uniform((K, N), 8 + si)
        Cref, Abs = og.gemm_bf16(a, b)
        for sched in SCHEDS:
            C = run_gemm(a, b, M, N, K, out, sched, tile, debug_flags=flags)
            assert C.guards_intact(), (M, N, K, sched)
            assert_within(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL,
                          out == "bf16_out_bf16", f"{(M, N, K)} {sched} {tile} {out}")


@pytest.mark.parametrize("out", ["bf16_out_f32", "bf16_out_bf16"])
def test_unaligned_scalar_path(out):
    # K and N not multiples of 8 take the element-wise load path
    for M, N, K in [(300, 301, 77), (5, 259, 130), (257, 7, 513)]:
        a = bf16_bits_normal((M, K), M)
        b = bf16_bits_normal((K, N), N)
        Cref, Abs = og.gemm_bf16(a, b)
        for sched in ["blocked", "work_stealing"]:
            C = run_gemm(a, b, M, N, K, out, sched, (256, 256, 64))
            assert C.guards_intact()
            assert_within(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL,
                          out == "bf16_out_bf16", f"{(M, N, K)} {sched}")


def test_identity_bit_exact():
    K, N = 512, 384
    a = np.zeros((K, K), np.uint16)
    np.fill_diagonal(a, 0x3F80)
    b = bf16_bits_normal((K, N), 3)
    for sched in SCHEDS:
        C = run_gemm(a, b, K, N, K, "bf16_out_bf16", sched, (256, 256, 64))
        assert np.array_equal(C.body_bits().view(np.uint16), b.reshape(-1)), sched


@pytest.mark.parametrize("K", [64, 1024, 8192])
def test_rank1_exact(K):
    r = np.random.default_rng(K)
    M, N = 300, 200
    s = r.integers(-8, 9, size=M).astype(np.float32)
    t = r.integers(-8, 9, size=N).astype(np.float32)
    from synthetic import bf16_bits_from_f32
    a = bf16_bits_from_f32(np.repeat(s[:, None], K, 1))
    b = bf16_bits_from_f32(np.repeat(t[None, :], K, 0))
    want = K * np.outer(s, t).astype(np.float64)
    for out in ["bf16_out_f32", "bf16_out_bf16"]:
        C = run_gemm(a, b, M, N, K, out, "work_stealing", (256, 256, 64))
        assert np.array_equal(C.as_f64().reshape(M, N), want), out


def test_cfg1_512_fp32_out_full():
    """Workload 1: 512^3, uniform[-1,1) bf16, fp32 C, 128x128x64 tiles, blocked."""
    M = N = K = 512
    a = bf16_bits_uniform((M, K), 1010)
    b = bf16_bits_uniform((K, N), 1011)
    Cref, Abs = og.gemm_bf16(a, b)
    C = run_gemm(a, b, M, N, K, "bf16_out_f32", "blocked", (128, 128, 64))
    assert C.guards_intact()
    assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, "512^3")
    for sched in SCHEDS[1:]:
        C2 = run_gemm(a, b, M, N, K, "bf16_out_f32", sched, (128, 128, 64))
        assert np.array_equal(C2.body_bits(), C.body_bits()), sched


def _full_check(a, b, C, M, N, tol, what):
    """Every element of C against the oracle (fp64 over the decoded operands)."""
    note(f"oracle on all of C ({M}x{N}): {what}")
    Cref, Abs = og.gemm_bf16(a, b)
    assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, tol, what)


@pytest.mark.parametrize("shape", [(5120, 5120, 4096), (4864, 8000, 8192), (3000, 7000, 2048)])
def test_ragged_all_schedulers(shape):
    """Workload 4: ragged shapes, uniform[-1,1) bf16, bf16 C, 256x256x64, every scheduler:
    the first scheduler's C against the oracle on every element (masked edge
    tiles included), every other scheduler bit-identical to it."""
    M, N, K = shape
    a = bf16_bits_uniform((M, K), 1040 + M)
    b = bf16_bits_uniform((K, N), 1041 + N)
    ref_bits = None
    for sched in SCHEDS:
        C = run_gemm(a, b, M, N, K, "bf16_out_bf16", sched, (256, 256, 64))
        assert C.guards_intact(), sched
        bits = C.body_bits()
        if ref_bits is None:
            _full_check(a, b, C, M, N, BF16_TOL, f"{shape} {sched}")
            ref_bits = bits
        else:
            assert np.array_equal(bits, ref_bits), f"{shape}: {sched} differs from blocked"


def test_8192_all_schedulers():
    """Workload 3: 8192^3, normal(0,1) bf16, bf16 C, 256x256x64, every scheduler and
    group sizes 8 / 16 on the direct-to-LDS kernel: the first scheduler's C against the
    oracle on every element, bitwise equality across schedulers.  The register-staged
    kernel (32x32 MFMA blocks, so its own rounding order) is checked against the
    oracle on every element as well."""
    M = N = K = 8192
    a = bf16_bits_normal((M, K), 1030)
    b = bf16_bits_normal((K, N), 1031)
    note("oracle on all of C (8192x8192)")
    Cref, Abs = og.gemm_bf16(a, b)
    ref_bits = None
    for sched, gs in [("blocked", 0), ("interleaved", 0), ("grouped", 8), ("grouped", 16),
                      ("work_stealing", 8), ("work_stealing", 16), ("blocked_grouped", 8),
                      ("work_stealing_xcc", 8)]:
        C = run_gemm(a, b, M, N, K, "bf16_out_bf16", sched, (256, 256, 64), group_size=gs)
        assert C.guards_intact()
        bits = C.body_bits()
        if ref_bits is None:
            assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, f"8192^3 {sched}")
            ref_bits = bits
        else:
            assert np.array_equal(bits, ref_bits), f"8192^3: {sched}/{gs} differs"
    C = run_gemm(a, b, M, N, K, "bf16_out_bf16", "work_stealing", (256, 256, 64), group_size=8,
                 debug_flags=pg._abi.DEBUG_REGISTER_STAGED)
    assert C.guards_intact()
    assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, "8192^3 register-staged")


@pytest.mark.parametrize("tile", [(128, 128, 64), (256, 256, 64)])
def test_balanced_grid_same_bits_as_full_grid(tile):
    """The default (balanced) grid changes which program computes a tile,
    never the tile's K order: C is bit-identical to a launch on every
    resident slot, for every data-parallel scheduler, on a ragged shape
    whose tiles fill less than one round (the default grid is then the tile
    count rounded up to the XCDs), and within the bound of the oracle."""
    cfg = config()
    M, N, K = 1300, 900, 256
    a, b = bf16_bits_uniform((M, K), 4400), bf16_bits_uniform((K, N), 4401)
    Cref, Abs = og.gemm_bf16(a, b)
    for sched in SCHEDS:
        plan = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", sched, pg.make_args(tile=tile))
        full = cfg.info["num_cus"] * plan["occupancy"]
        assert plan["grid"] <= full and plan["grid"] % cfg.info["num_xcds"] == 0
        Cb = run_gemm(a, b, M, N, K, "bf16_out_bf16", sched, tile)
        Cf = run_gemm(a, b, M, N, K, "bf16_out_bf16", sched, tile, grid=full)
        assert Cb.guards_intact() and Cf.guards_intact(), sched
        assert np.array_equal(Cb.body_bits(), Cf.body_bits()), f"{sched} {tile}: grid {plan['grid']} vs {full}"
        assert_within(Cb.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, True, f"{sched} {tile} balanced grid")
