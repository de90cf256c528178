"""GPU parity of the persistent block-scaled fp8 (e4m3, e8m0 per 128 K) GEMM
against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import gemm as og
from synthetic import fp8_blockscaled
from tests.gpu_util import FP8_TOL, Guarded, assert_abs_bound, config, dev_u8, note, sync

pytestmark = pytest.mark.gpu

SCHEDS = ["blocked", "interleaved", "grouped", "work_stealing", "blocked_grouped", "work_stealing_xcc"]


def make_inputs(M, N, K, seed):
    qa, sa = fp8_blockscaled(M, K, seed, seed + 2, k_major=True)
    qb, sb = fp8_blockscaled(N, K, seed + 1, seed + 3, k_major=False)
    return qa, sa, qb, sb


def run_fp8(qa, sa, qb, sb, M, N, K, sched, tile, **kw):
    cfg = config()
    A, B, SA, SB = dev_u8(qa), dev_u8(qb), dev_u8(sa), dev_u8(sb)
    C = Guarded(M * N, "bf16")
    note(f"pgemm_run fp8 M={M} N={N} K={K} sched={sched} tile={tile} {kw}")
    pg.pgemm_run(cfg, A, B, C.view, M, N, K, "fp8_b128_out_bf16", sched,
                 pg.make_args(tile=tile, a_scale=SA, b_scale=SB, **kw))
    sync()
    return C


def test_closed_form_scales():
    # q = 1.0 everywhere; SA[g][i] = 127 + (g + i) % 5 - 2, SB[g][j] = 127 - (j % 3):
    # C[i][j] = 128 * sum_g 2**(SA - 127) * 2**(SB - 127), exact in bf16 here.
    M, N, K = 300, 272, 512
    qa = np.full((M, K), 0x38, np.uint8)
    qb = np.full((K, N), 0x38, np.uint8)
    G = K // 128
    sa = np.array([[127 + (g + i) % 5 - 2 for i in range(M)] for g in range(G)], np.uint8)
    sb = np.array([[127 - (j % 3) for j in range(N)] for g in range(G)], np.uint8)
    want = np.zeros((M, N))
    for g in range(G):
        want += 128.0 * np.outer(2.0 ** (sa[g].astype(float) - 127), 2.0 ** (sb[g].astype(float) - 127))
    for tile in [(128, 128, 128), (256, 256, 128), (128, 256, 128)]:
        for sched in SCHEDS:
            C = run_fp8(qa, sa, qb, sb, M, N, K, sched, tile)
            assert C.guards_intact()
            assert np.array_equal(C.as_f64().reshape(M, N), want), (tile, sched)


@pytest.mark.parametrize("tile", [(128, 128, 128), (256, 256, 128), (128, 256, 128)])
def test_small_shapes(tile):
    shapes = [(1, 16, 128), (100, 112, 256), (129, 128, 384), (256, 272, 128), (300, 400, 256),
              (257, 16, 640), (64, 1024, 128)]
    for i, (M, N, K) in enumerate(shapes):
        qa, sa, qb, sb = make_inputs(M, N, K, 50 + i)
        Cref, Abs = og.gemm_fp8_b128(qa, sa, qb, sb)
        for sched in SCHEDS:
            C = run_fp8(qa, sa, qb, sb, M, N, K, sched, tile)
            assert C.guards_intact(), (M, N, K, sched)
            assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, FP8_TOL, f"{(M, N, K)} {sched} {tile}")


@pytest.mark.parametrize("tile", [(128, 128, 128), (256, 256, 128), (128, 256, 128)])
def test_program_order_keeps_c(tile):
    """Static walks with their programs numbered XCD-major and in workgroup
    order: the same tiles per program, so the same bits of C, and both within
    the oracle's bound."""
    M, N, K = 1100, 4352, 512
    qa, sa, qb, sb = make_inputs(M, N, K, 77)
    Cref, Abs = og.gemm_fp8_b128(qa, sa, qb, sb)
    for sched in ["blocked", "interleaved", "grouped", "blocked_grouped"]:
        Cx = run_fp8(qa, sa, qb, sb, M, N, K, sched, tile, program_order="xcd_major")
        Cd = run_fp8(qa, sa, qb, sb, M, N, K, sched, tile, program_order="dispatch")
        assert Cx.guards_intact() and Cd.guards_intact()
        assert np.array_equal(Cx.body_bits(), Cd.body_bits()), (sched, tile)
        assert_abs_bound(Cx.as_f64().reshape(M, N), Cref, Abs, FP8_TOL, f"{sched} {tile} XCD-major")


def test_unsupported_shapes_are_rejected():
    cfg = config()
    qa, sa, qb, sb = make_inputs(64, 24, 128, 3)
    A, B, SA, SB = dev_u8(qa), dev_u8(qb), dev_u8(sa), dev_u8(sb)
    C = torch.empty(64 * 24, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run(cfg, A, B, C, 64, 24, 128, "fp8_b128_out_bf16", "blocked",
                     pg.make_args(tile=(128, 128, 128), a_scale=SA, b_scale=SB))
    assert e.value.code == pg._abi.ERR_UNSUPPORTED


def _full(qa, sa, qb, sb, C, M, N, what):
    """Every element of C against the oracle (fp64 over the dequantised operands)."""
    note(f"oracle on all of C ({M}x{N}): {what}")
    Cref, Abs = og.gemm_fp8_b128(qa, sa, qb, sb)
    assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, FP8_TOL, what)


def test_skinny_256x28672x8192():
    """Workload 5a: M=256, N=28672, K=8192, 128x128x128 tiles (and 128x256x128 on
    the three-stage ring), work stealing vs grouped; the first run's C against
    the oracle on every element, every other run bit-identical (the tile shape
    never changes an element's K order)."""
    M, N, K = 256, 28672, 8192
    qa, sa, qb, sb = make_inputs(M, N, K, 1050)
    ref = None
    for sched, tile in [("work_stealing", (128, 128, 128)), ("grouped", (128, 128, 128)),
                        ("blocked", (128, 128, 128)), ("interleaved", (128, 128, 128)),
                        ("work_stealing", (128, 256, 128)), ("grouped", (128, 256, 128))]:
        C = run_fp8(qa, sa, qb, sb, M, N, K, sched, tile)
        assert C.guards_intact()
        if ref is None:
            _full(qa, sa, qb, sb, C, M, N, f"5a {sched}")
            ref = C.body_bits()
        else:
            assert np.array_equal(C.body_bits(), ref), (sched, tile)


def test_square_8192():
    """Workload 5b: 8192^3, 256x256x128 tiles, work stealing vs grouped: the
    first run's C against the oracle on every element, the other bit-identical."""
    M = N = K = 8192
    qa, sa, qb, sb = make_inputs(M, N, K, 1050)
    ref = None
    for sched in ["work_stealing", "grouped"]:
        C = run_fp8(qa, sa, qb, sb, M, N, K, sched, (256, 256, 128))
        assert C.guards_intact()
        if ref is None:
            _full(qa, sa, qb, sb, C, M, N, f"5b {sched}")
            ref = C.body_bits()
        else:
            assert np.array_equal(C.body_bits(), ref), sched
