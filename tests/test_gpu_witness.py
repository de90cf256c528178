"""GPU schedule witness: every tile computed exactly once under every scheduler;
static schedules equal the oracle's model tile for tile; work-stealing runs
satisfy the model's invariants (owner on the right XCD, increasing claims,
final counters); work stealing across XCDs satisfies its own (each program
starts on the counter of the hardware XCC it ran on, recorded by the
witness)."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import sched_model as sm
from synthetic import bf16_bits_uniform, f32_normal
from tests.gpu_util import config, dev_bf16, dev_f32, note, sync

pytestmark = pytest.mark.gpu

STATIC = ["blocked", "interleaved", "grouped", "blocked_grouped"]
WS = ["work_stealing", "work_stealing_xcc"]


def _check(w, kind, pm, pn, G, X, gs, chunk=1):
    T = pm * pn
    visits, owner, order = w["visits"][:T], w["owner"][:T], w["order"][:T]
    assert np.all(visits == 1), f"{kind}: tiles visited {np.unique(visits)} times"
    assert int(w["n_tiles"][:G].sum()) == T
    if kind in STATIC:
        model = sm.static_schedule(kind, pm, pn, G, gs)
        for p, seq in enumerate(model):
            for i, (v, _, _) in enumerate(seq):
                assert owner[v] == p and order[v] == i, (kind, v, owner[v], p, order[v], i)
            assert w["n_tiles"][p] == len(seq)
    elif kind == "work_stealing":
        sm.check_ws_execution(visits.tolist(), owner.tolist(), order.tolist(),
                              w["counters"].tolist(), T, G, X, chunk)
    else:
        homes = [((int(h) >> 16) & 0xF) % X for h in w["hw_id"][:G]]
        sm.check_wsx_execution(visits.tolist(), owner.tolist(), order.tolist(),
                               w["counters"].tolist(), homes, T, G, X, chunk)


def _gemm_witness(M, N, K, tile, sched, gs=8, grid=0):
    cfg = config()
    G = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", sched,
                     pg.make_args(tile=tile, group_size=gs, grid=grid))["grid"]
    pm, pn = -(-M // tile[0]), -(-N // tile[1])
    cfg.witness_enable(pm * pn, G)
    a = bf16_bits_uniform((M, K), 1)
    b = bf16_bits_uniform((K, N), 2)
    A, B = dev_bf16(a), dev_bf16(b)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    note(f"witness gemm {M}x{N}x{K} tile={tile} {sched} gs={gs} grid={G}")
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched,
                 pg.make_args(tile=tile, group_size=gs, grid=grid, debug_flags=pg._abi.DEBUG_WITNESS))
    w = cfg.witness_read(pm * pn, G)
    # the witness build computes the same bits as the timed build
    C2 = torch.empty_like(C)
    pg.pgemm_run(cfg, A, B, C2, M, N, K, "bf16_out_bf16", sched,
                 pg.make_args(tile=tile, group_size=gs, grid=grid))
    sync()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    return w, pm, pn, G, cfg.info["num_xcds"]


@pytest.mark.parametrize("sched", STATIC + WS)
@pytest.mark.parametrize("shape,tile", [
    ((512, 512, 512), (128, 128, 64)),
    ((5120, 5120, 256), (256, 256, 64)),
    ((3000, 7000, 128), (256, 256, 64)),
    ((8192, 8192, 64), (256, 256, 64)),
])
def test_gemm_schedule_exactly_once(sched, shape, tile):
    M, N, K = shape
    w, pm, pn, G, X = _gemm_witness(M, N, K, tile, sched)
    _check(w, sched, pm, pn, G, X, 8)


@pytest.mark.parametrize("sched", WS)
@pytest.mark.parametrize("chunk", [2, 3, pg._abi.CLAIM_PAIRS])
@pytest.mark.parametrize("shape,tile", [((5120, 5120, 128), (256, 256, 64)),
                                        ((4864, 8000, 64), (256, 256, 64)),
                                        ((1100, 904, 64), (128, 128, 64))])
def test_gemm_chunked_claims(sched, chunk, shape, tile):
    """Claims of several consecutive tiles: every tile once, the claim order
    and the final counters of the model with that chunk; same C as grouped."""
    M, N, K = shape
    cfg = config()
    G = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", sched, pg.make_args(tile=tile))["grid"]
    pm, pn = -(-M // tile[0]), -(-N // tile[1])
    cfg.witness_enable(pm * pn, G)
    A, B = dev_bf16(bf16_bits_uniform((M, K), 1)), dev_bf16(bf16_bits_uniform((K, N), 2))
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    note(f"chunked claims {shape} tile={tile} {sched} chunk={chunk} grid={G}")
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched,
                 pg.make_args(tile=tile, claim_chunk=chunk, debug_flags=pg._abi.DEBUG_WITNESS))
    w = cfg.witness_read(pm * pn, G)
    _check(w, sched, pm, pn, G, cfg.info["num_xcds"], 8, sm.PAIRS if chunk < 0 else chunk)
    Cg = torch.empty_like(C)
    pg.pgemm_run(cfg, A, B, Cg, M, N, K, "bf16_out_bf16", "grouped", pg.make_args(tile=tile))
    sync()
    assert torch.equal(C.view(torch.int16), Cg.view(torch.int16))


def test_gemm_witness_clock():
    """Per-program shader cycles over wall time give a plausible engine clock."""
    w, pm, pn, G, X = _gemm_witness(5120, 5120, 2048, (256, 256, 64), "work_stealing")
    khz = config().info["wall_clock_khz"]
    dt = (w["t_end"][:G] - w["t_start"][:G]) / (khz * 1e3)   # seconds
    busy = dt > 2e-6
    assert busy.sum() >= G // 2
    ghz = w["cycles"][:G][busy] / dt[busy] / 1e9
    note(f"clock GHz min {ghz.min():.3f} median {np.median(ghz):.3f} max {ghz.max():.3f}")
    assert np.all((ghz > 0.3) & (ghz < 3.0)), ghz


@pytest.mark.parametrize("sched", STATIC + WS)
@pytest.mark.parametrize("grid", [1, 7, 8, 13, 300])
def test_gemm_schedule_grid_override(sched, grid):
    if sched == "work_stealing" and grid < config().info["num_xcds"]:
        pytest.skip("work stealing needs at least one program per XCD")
    w, pm, pn, G, X = _gemm_witness(1100, 900, 64, (128, 128, 64), sched, gs=3, grid=grid)
    _check(w, sched, pm, pn, G, X, 3)


@pytest.mark.parametrize("sched", STATIC + WS)
@pytest.mark.parametrize("tile", [(32, 16), (128, 128)])
def test_add_schedule_exactly_once(sched, tile):
    cfg = config()
    rows, cols = 2048, 3000
    pm, pn = -(-rows // tile[0]), -(-cols // tile[1])
    G = pg.plan_add(cfg, rows, cols, tile[0], tile[1], sched)["grid"]
    cfg.witness_enable(pm * pn, G)
    X, Y = dev_f32(f32_normal((rows, cols), 1)), dev_f32(f32_normal((rows, cols), 2))
    C = torch.empty_like(X)
    note(f"witness add {rows}x{cols} tile={tile} {sched}")
    pg.padd_run(cfg, X, Y, C, rows, cols, tile[0], tile[1], sched,
                pg.make_args(debug_flags=pg._abi.DEBUG_WITNESS))
    w = cfg.witness_read(pm * pn, G)
    chunk = {(32, 16): 32, (64, 64): 4, (128, 128): 1}[tile]
    _check(w, sched, pm, pn, G, cfg.info["num_xcds"], 8, chunk)
