"""GPU parity of the persistent 2-D add: bit-exact against the oracle add."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle.add import add_f32
from synthetic import f32_normal
from tests.gpu_util import GUARD, SENTINEL_F32, config, dev_f32, note, sync

pytestmark = pytest.mark.gpu

SCHEDS = ["blocked", "interleaved", "grouped", "work_stealing", "blocked_grouped", "work_stealing_xcc"]
TILES = [(32, 16), (64, 64), (128, 128)]


def run_add(x, y, tile, sched, **kw):
    rows, cols = x.shape
    cfg = config()
    X, Y = dev_f32(x), dev_f32(y)
    full = torch.full((rows * cols + 2 * GUARD,), SENTINEL_F32, dtype=torch.int32, device="cuda:0")
    C = full[GUARD:GUARD + rows * cols].view(torch.float32)
    note(f"padd_run {rows}x{cols} tile={tile} sched={sched} {kw}")
    pg.padd_run(cfg, X, Y, C, rows, cols, tile[0], tile[1], sched, pg.make_args(**kw))
    sync()
    h = full.cpu().numpy()
    assert np.all(h[:GUARD] == SENTINEL_F32) and np.all(h[GUARD + rows * cols:] == SENTINEL_F32)
    return h[GUARD:GUARD + rows * cols].view(np.float32).reshape(rows, cols)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("shape", [(1, 1), (1, 4), (33, 20), (1000, 1000), (999, 1001),
                                   (257, 4100), (4096, 36)])
def test_add_bit_exact(tile, shape):
    x = f32_normal(shape, 2001)
    y = f32_normal(shape, 2002)
    want = add_f32(x, y).view(np.uint32)
    for sched in SCHEDS:
        got = run_add(x, y, tile, sched)
        assert np.array_equal(got.view(np.uint32), want), (shape, tile, sched)


@pytest.mark.parametrize("tile", [(32, 16), (128, 128)])
def test_add_8192_all_schedulers(tile):
    """Workload 2: fp32 8192x8192, normal(0,1), tiles 32x16 and 128x128."""
    x = f32_normal((8192, 8192), 2001)
    y = f32_normal((8192, 8192), 2002)
    want = add_f32(x, y).view(np.uint32)
    for sched in SCHEDS:
        got = run_add(x, y, tile, sched)
        assert np.array_equal(got.view(np.uint32), want), (tile, sched)


def test_add_special_values():
    v = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 1e-45, 3.4e38, -3.4e38,
                  2.0 ** -24, 1.0 + 2.0 ** -23], np.float32)
    x = np.tile(v, (len(v), 1))
    y = x.T.copy()
    with np.errstate(over="ignore", invalid="ignore"):
        want = add_f32(x, y)
    got = run_add(x, y, (32, 16), "interleaved")
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m].view(np.uint32), want[m].view(np.uint32))


def test_add_in_place():
    x = f32_normal((300, 400), 5)
    y = f32_normal((300, 400), 6)
    want = add_f32(x, y).view(np.uint32)
    cfg = config()
    X, Y = dev_f32(x), dev_f32(y)
    pg.padd_run(cfg, X, Y, X, 300, 400, 32, 16, "work_stealing")
    sync()
    assert np.array_equal(X.cpu().numpy().view(np.uint32), want)
