"""GPU parity of the stream-K scheduler (data-parallel full waves, slab runs
for the rest, split tiles summed by the fix-up kernel) against the oracle,
through the C ABI, on the bf16 and the block-scaled fp8 kernels.  Tiles that
no run splits are computed exactly as under the grouped scheduler (same
tile, same slab order), so they must match it bit for bit; split tiles only
within the tolerance."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import gemm as og
from oracle import sched_model as sm
from oracle.codecs import bf16_to_f64
from synthetic import bf16_bits_normal, bf16_bits_uniform
from tests.gpu_util import (BF16_TOL, Guarded, assert_abs_bound, assert_within, config,
                            dev_bf16, note, sync)

pytestmark = pytest.mark.gpu


def _run(A, B, M, N, K, out, sched, tile, **kw):
    cfg = config()
    C = Guarded(M * N, "bf16" if out == "bf16_out_bf16" else "f32")
    args = pg.make_args(tile=tile, **kw)
    note(f"pgemm_run M={M} N={N} K={K} {out} sched={sched} tile={tile} {kw}")
    pg.pgemm_run(cfg, A, B, C.view, M, N, K, out, sched, args)
    sync()
    assert C.guards_intact(), (M, N, K, sched)
    return C


def _split_mask(M, N, K, tile, G, gs=8):
    """Elements of C in tiles the stream-K runs split (from the oracle's model)."""
    pm, pn = -(-M // tile[0]), -(-N // tile[1])
    nk = -(-K // tile[2])
    mask = np.zeros((M, N), bool)
    for v in sm.streamk_partials(pm * pn, nk, G):
        r, c = sm.grouped_decode(v, pm, pn, gs)
        mask[r * tile[0]:(r + 1) * tile[0], c * tile[1]:(c + 1) * tile[1]] = True
    return mask


# (M, N, K): T < G, T a multiple of G (nothing split), T just above G, K tail,
# one slab per tile, ragged edges in both dimensions
SHAPES = [(512, 512, 512), (1024, 1024, 64), (2048, 2048, 200), (4096, 1024, 256),
          (1100, 904, 776), (2304, 4352, 128), (264, 8000, 136)]


@pytest.mark.parametrize("tile", [(128, 128, 64), (256, 256, 64)])
@pytest.mark.parametrize("out", ["bf16_out_f32", "bf16_out_bf16"])
def test_streamk_parity(tile, out):
    cfg = config()
    for si, (M, N, K) in enumerate(SHAPES):
        a = bf16_bits_uniform((M, K), 300 + si)
        b = bf16_bits_uniform((K, N), 400 + si)
        A, B = dev_bf16(a), dev_bf16(b)
        Cref, Abs = og.gemm_bf16(a, b)
        C = _run(A, B, M, N, K, out, "stream_k", tile)
        got = C.as_f64().reshape(M, N)
        assert_within(got, Cref, Abs, BF16_TOL, out == "bf16_out_bf16", f"{(M, N, K)} {tile} {out}")
        # unsplit tiles equal the grouped scheduler's bit for bit; split ones may differ
        Cg = _run(A, B, M, N, K, out, "grouped", tile)
        G = pg.plan_gemm(cfg, M, N, K, out, "stream_k", pg.make_args(tile=tile))["grid"]
        split = _split_mask(M, N, K, tile, G)
        same = C.body_bits().reshape(M, N) == Cg.body_bits().reshape(M, N)
        assert np.all(same | split), f"{(M, N, K)} {tile}: unsplit tiles differ from grouped"
        note(f"  split tiles cover {split.mean():.3f} of C")


def test_streamk_deterministic_and_grid_override():
    M, N, K = 1500, 1704, 520
    a, b = bf16_bits_normal((M, K), 501), bf16_bits_normal((K, N), 502)
    A, B = dev_bf16(a), dev_bf16(b)
    Cref, Abs = og.gemm_bf16(a, b)
    first = None
    for grid in [0, 0, 7, 13, 300]:
        C = _run(A, B, M, N, K, "bf16_out_bf16", "stream_k", (128, 128, 64), grid=grid)
        assert_within(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, True, f"grid {grid}")
        if grid == 0:
            if first is None:
                first = C.body_bits().copy()
            else:
                assert np.array_equal(C.body_bits(), first), "two stream-K runs differ"


@pytest.mark.parametrize("shape", [(5120, 5120, 4096), (4864, 8000, 8192), (3000, 7000, 2048)])
def test_streamk_ragged_configs(shape):
    """Workload 4 shapes under stream-K: sampled rows (every tile edge) against the oracle."""
    M, N, K = shape
    a = bf16_bits_uniform((M, K), 1040 + M)
    b = bf16_bits_uniform((K, N), 1041 + N)
    A, B = dev_bf16(a), dev_bf16(b)
    C = _run(A, B, M, N, K, "bf16_out_bf16", "stream_k", (256, 256, 64))
    rng = np.random.default_rng(M)
    rows = {0, M - 1}
    for t in range(0, M, 256):
        rows |= {t, min(t + 255, M - 1)}
    rows |= set(rng.integers(0, M, size=16).tolist())
    rows = np.array(sorted(rows))
    Cref, Abs = og.gemm_f64_sampled(bf16_to_f64(a), bf16_to_f64(b), rows, np.arange(N))
    assert_abs_bound(C.as_f64().reshape(M, N)[rows, :], Cref, Abs, BF16_TOL, f"{shape} stream_k")


def test_streamk_unsupported_combinations():
    cfg = config()
    M, N, K = 256, 256, 128
    A = dev_bf16(bf16_bits_uniform((M, K), 1))
    B = dev_bf16(bf16_bits_uniform((K, N), 2))
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    for kw in [dict(debug_flags=pg._abi.DEBUG_WITNESS), dict(debug_flags=pg._abi.DEBUG_REGISTER_STAGED)]:
        if "debug_flags" in kw and kw["debug_flags"] == pg._abi.DEBUG_WITNESS:
            cfg.witness_enable(16, 1024)
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", "stream_k", pg.make_args(**kw))
        assert e.value.code == pg._abi.ERR_UNSUPPORTED
    # K not a multiple of 8 takes the register-staged kernel: not for stream-K
    A2 = dev_bf16(bf16_bits_uniform((M, 100), 3))
    B2 = dev_bf16(bf16_bits_uniform((100, N), 4))
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run(cfg, A2, B2, C, M, N, 100, "bf16_out_bf16", "stream_k")
    assert e.value.code == pg._abi.ERR_UNSUPPORTED


# block-scaled fp8 under stream-K: N a multiple of 16, K of 128
FP8_SHAPES = [(512, 512, 512), (1024, 1024, 128), (2048, 2048, 384), (1100, 912, 768),
              (264, 8000, 256), (2304, 4352, 128)]
FP8_TILES = [(128, 128, 128), (256, 256, 128), (128, 256, 128)]


def _run_fp8(qa, sa, qb, sb, M, N, K, sched, tile):
    from tests.gpu_util import dev_u8
    cfg = config()
    A, B, SA, SB = dev_u8(qa), dev_u8(qb), dev_u8(sa), dev_u8(sb)
    C = Guarded(M * N, "bf16")
    note(f"pgemm_run fp8 M={M} N={N} K={K} sched={sched} tile={tile}")
    pg.pgemm_run(cfg, A, B, C.view, M, N, K, "fp8_b128_out_bf16", sched,
                 pg.make_args(tile=tile, a_scale=SA, b_scale=SB))
    sync()
    assert C.guards_intact(), (M, N, K, sched, tile)
    return C


@pytest.mark.parametrize("shape", FP8_SHAPES)
def test_streamk_fp8_parity(shape):
    from synthetic import fp8_blockscaled
    from tests.gpu_util import FP8_TOL
    M, N, K = shape
    qa, sa = fp8_blockscaled(M, K, 3000 + M, 3002 + M, k_major=True)
    qb, sb = fp8_blockscaled(N, K, 3001 + N, 3003 + N, k_major=False)
    Cref, Abs = og.gemm_fp8_b128(qa, sa, qb, sb)
    cfg = config()
    for tile in FP8_TILES:
        C = _run_fp8(qa, sa, qb, sb, M, N, K, "stream_k", tile)
        assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, FP8_TOL, f"fp8 {shape} {tile}")
        Cg = _run_fp8(qa, sa, qb, sb, M, N, K, "grouped", tile)
        G = pg.plan_gemm(cfg, M, N, K, "fp8_b128_out_bf16", "stream_k", pg.make_args(tile=tile))["grid"]
        split = _split_mask(M, N, K, tile, G)
        same = C.body_bits().reshape(M, N) == Cg.body_bits().reshape(M, N)
        assert np.all(same | split), f"fp8 {shape} {tile}: unsplit tiles differ from grouped"


def test_streamk_fp8_skinny_256x28672x8192():
    """Workload 5a under stream-K: 112 tiles at 256x256 (all split over the
    grid) and 224 at 128x256; sampled rows against the oracle, and two runs
    bit-identical."""
    from oracle.codecs import dequant_fp8_a, dequant_fp8_b
    from synthetic import fp8_blockscaled
    from tests.gpu_util import FP8_TOL
    M, N, K = 256, 28672, 8192
    qa, sa = fp8_blockscaled(M, K, 1050, 1052, k_major=True)
    qb, sb = fp8_blockscaled(N, K, 1051, 1053, k_major=False)
    rows = np.array([0, 1, 31, 64, 127, 128, 200, 255])
    Cref, Abs = og.gemm_f64(dequant_fp8_a(qa[rows], sa[:, rows]), dequant_fp8_b(qb, sb))
    for tile in [(256, 256, 128), (128, 256, 128)]:
        C = _run_fp8(qa, sa, qb, sb, M, N, K, "stream_k", tile)
        assert_abs_bound(C.as_f64().reshape(M, N)[rows], Cref, Abs, FP8_TOL, f"5a stream_k {tile}")
        C2 = _run_fp8(qa, sa, qb, sb, M, N, K, "stream_k", tile)
        assert np.array_equal(C.body_bits(), C2.body_bits()), f"5a stream_k {tile}: runs differ"
