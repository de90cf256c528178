"""pgemm_run_noalloc, the entry point for callers that cannot allocate device
memory, against pgemm_run on the same inputs: bit-identical results, two
calls in a row with the second on a smaller problem (the static scratch
keeps the first call's counters and partial sums, so anything not cleared
or not rewritten would show), and the scratch-size limit refused with
nothing written."""
import numpy as np
import pytest

import tile_scheduling_persistent_amd as pg
from synthetic import bf16_bits_uniform, fp8_blockscaled
from tests.gpu_util import Guarded, config, dev_bf16, dev_u8, note, sync

pytestmark = pytest.mark.gpu

# (scheduler, tile, grid): work stealing takes its counters from the scratch,
# stream-K its partial sums (256x256 tiles only on a grid of at most 128)
BF16_CASES = [("work_stealing", (256, 256, 64), 0), ("work_stealing_xcc", (256, 256, 64), 0),
              ("work_stealing", (128, 128, 64), 0), ("grouped", (256, 256, 64), 0),
              ("stream_k", (128, 128, 64), 0), ("stream_k", (256, 256, 64), 128)]
SHAPES = [(1536, 1280, 1024), (700, 520, 320)]   # second call smaller, ragged


def _run(fn, A, B, M, N, K, out, sched, args):
    C = Guarded(M * N, "bf16" if out != "bf16_out_f32" else "f32")
    note(f"{fn.__name__} M={M} N={N} K={K} {out} {sched}")
    fn(config(), A, B, C.view, M, N, K, out, sched, args)
    sync()
    assert C.guards_intact(), (fn.__name__, sched)
    return C.body_bits()


@pytest.mark.parametrize("sched,tile,grid", BF16_CASES)
def test_noalloc_bf16_matches_pgemm_run(sched, tile, grid):
    for i, (M, N, K) in enumerate(SHAPES):
        a = bf16_bits_uniform((M, K), 5100 + i)
        b = bf16_bits_uniform((K, N), 5200 + i)
        A, B = dev_bf16(a), dev_bf16(b)
        for out in ("bf16_out_bf16", "bf16_out_f32"):
            args = pg.make_args(tile=tile, grid=grid)
            want = _run(pg.pgemm_run, A, B, M, N, K, out, sched, args)
            got = _run(pg.pgemm_run_noalloc, A, B, M, N, K, out, sched, args)
            assert np.array_equal(got, want), (sched, tile, (M, N, K), out)


@pytest.mark.parametrize("sched", ["work_stealing", "stream_k"])
def test_noalloc_fp8_matches_pgemm_run(sched):
    for i, (M, N, K) in enumerate([(1024, 1536, 1024), (384, 640, 512)]):
        qa, sa = fp8_blockscaled(M, K, 5300 + i, 5310 + i, k_major=True)
        qb, sb = fp8_blockscaled(N, K, 5320 + i, 5330 + i, k_major=False)
        A, B, SA, SB = dev_u8(qa), dev_u8(qb), dev_u8(sa), dev_u8(sb)
        args = pg.make_args(tile=(128, 256, 128), a_scale=SA, b_scale=SB)
        want = _run(pg.pgemm_run, A, B, M, N, K, "fp8_b128_out_bf16", sched, args)
        got = _run(pg.pgemm_run_noalloc, A, B, M, N, K, "fp8_b128_out_bf16", sched, args)
        assert np.array_equal(got, want), (sched, (M, N, K))


def test_noalloc_refuses_partial_sums_beyond_the_scratch():
    """Stream-K at 256x256 tiles on every CU needs 512 KiB of partial sums per
    program, more than the scratch holds: refused, nothing written."""
    cfg = config()
    M, N, K = 1536, 1280, 1024
    A = dev_bf16(bf16_bits_uniform((M, K), 5400))
    B = dev_bf16(bf16_bits_uniform((K, N), 5401))
    args = pg.make_args(tile=(256, 256, 64))
    plan = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", "stream_k", args)
    assert plan["grid"] * 2 * 256 * 256 * 4 > pg._abi.NOALLOC_SCRATCH_BYTES - 4096
    C = Guarded(M * N, "bf16")
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run_noalloc(cfg, A, B, C.view, M, N, K, "bf16_out_bf16", "stream_k", args)
    assert e.value.code == pg._abi.ERR_INVALID
    sync("refused no-alloc call")
    assert np.all(C.body_bits().view(np.uint16) == 0x7FC1)
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run_noalloc(cfg, A, B, C.view, M, N, K, "bf16_out_bf16", "work_stealing",
                             pg.make_args(debug_flags=pg._abi.DEBUG_WITNESS))
    assert e.value.code == pg._abi.ERR_UNSUPPORTED
