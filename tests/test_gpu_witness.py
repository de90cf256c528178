"""GPU schedule witness: every tile computed exactly once under every scheduler;
static schedules equal the oracle's model tile for tile; work-stealing runs
satisfy the model's invariants (owner on the right XCD, increasing claims,
final counters, and each counter equal to the claims the programs recorded
on it with one failing claim per program at home); work stealing across
XCDs satisfies its own (each program starts on the counter of the hardware
XCC it ran on, recorded by the witness)."""
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
        assert not w["claims"][:G].any(), f"{kind}: a static walk recorded claims"
    elif kind == "work_stealing":
        sm.check_ws_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                              T, G, X, chunk, claims=w["claims"][:G, :X].tolist())
    else:
        homes = [((int(h) >> 16) & 0xF) % X for h in w["hw_id"][:G]]
        sm.check_wsx_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                               homes, T, G, X, chunk, claims=w["claims"][:G, :X].tolist())


def _gemm_witness(M, N, K, tile, sched, gs=8, grid=0, order="default"):
    cfg = config()
    G = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", sched,
                     pg.make_args(tile=tile, group_size=gs, grid=grid, program_order=order))["grid"]
    pm, pn = -(-M // tile[0]), -(-N // tile[1])
    cfg.witness_enable(pm * pn, G)
    a = bf16_bits_uniform((M, K), 1)
    b = bf16_bits_uniform((K, N), 2)
    A, B = dev_bf16(a), dev_bf16(b)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    note(f"witness gemm {M}x{N}x{K} tile={tile} {sched} gs={gs} grid={G} order={order}")
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched,
                 pg.make_args(tile=tile, group_size=gs, grid=grid, debug_flags=pg._abi.DEBUG_WITNESS,
                              program_order=order))
    w = cfg.witness_read(pm * pn, G)
    # the witness build computes the same bits as the timed build
    C2 = torch.empty_like(C)
    pg.pgemm_run(cfg, A, B, C2, M, N, K, "bf16_out_bf16", sched,
                 pg.make_args(tile=tile, group_size=gs, grid=grid, program_order=order))
    sync()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    w["C"] = C
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


def _placement(xcc, groups, X):
    """Share of programs on their group's most common XCD, and whether the
    groups' XCDs are all different (the hardware's round robin may start at
    any XCD, so only the grouping is fixed, not which XCD a group gets)."""
    on, homes = 0, []
    for g in np.unique(groups):
        vals, counts = np.unique(xcc[groups == g], return_counts=True)
        on += counts.max()
        homes.append(int(vals[counts.argmax()]))
    return on / len(xcc), len(set(homes)) == len(homes) == X


@pytest.mark.parametrize("sched", STATIC)
def test_gemm_program_order(sched):
    """Static walks under both program numberings: the schedule of the model
    for the programs as numbered, the same C, and (hardware placement being
    round robin, from whichever XCD it starts at) each XCD runs the programs
    [x*G/X, (x+1)*G/X) of one block under XCD-major numbering, and one
    residue class {x, x+X, ...} under dispatch order."""
    M, N, K, tile = 5120, 5120, 256, (256, 256, 64)
    res = {}
    for order in ("xcd_major", "dispatch"):
        plan = pg.plan_gemm(config(), M, N, K, "bf16_out_bf16", sched,
                            pg.make_args(tile=tile, program_order=order))
        w, pm, pn, G, X = _gemm_witness(M, N, K, tile, sched, order=order)
        assert G % X == 0 and plan["xcd_major"] == (order == "xcd_major")
        _check(w, sched, pm, pn, G, X, 8)
        xcc = (w["hw_id"][:G].astype(np.int64) >> 16) & 0xF
        q = np.arange(G)
        frac, distinct = _placement(xcc, q // (G // X) if order == "xcd_major" else q % X, X)
        note(f"{sched} order={order}: share of programs on their group's XCD {frac:.3f}, "
             f"groups on distinct XCDs {distinct}")
        assert frac >= 0.9 and distinct, (sched, order, frac, distinct)
        res[order] = w["C"]
    assert torch.equal(res["xcd_major"].view(torch.int16), res["dispatch"].view(torch.int16))


@pytest.mark.parametrize("shape,dtype,tile,sched,want", [
    ((8192, 8192, 8192), "bf16_out_bf16", (256, 256, 64), "grouped", True),
    ((8192, 8192, 8192), "bf16_out_bf16", (256, 256, 64), "blocked", True),
    ((8192, 8192, 8192), "bf16_out_bf16", (256, 256, 64), "interleaved", False),
    ((8192, 8192, 8192), "bf16_out_bf16", (256, 256, 64), "blocked_grouped", False),
    ((256, 28672, 8192), "fp8_b128_out_bf16", (128, 256, 128), "interleaved", True),
    ((4864, 8000, 8192), "bf16_out_bf16", (256, 256, 64), "grouped", True),
    ((8192, 8192, 8192), "bf16_out_bf16", (256, 256, 64), "work_stealing", False),
    ((8192, 8192, 8192), "bf16_out_bf16", (256, 256, 64), "stream_k", False),
    ((1100, 900, 64), "bf16_out_bf16", (128, 128, 64), "grouped", False),  # grid 7: not a multiple of X
])
def test_default_program_order(shape, dtype, tile, sched, want):
    """The default numbering is the one whose programs' first tiles touch fewer
    operand panels per XCD (rows of tiles x tile_m + columns x tile_n over the
    XCDs; the counts for these launches worked out from the oracle's static
    schedules: grouped 8192^3 96 vs 264 panels of 256, interleaved 264 vs 96,
    blocked-grouped 144 vs 96, fp8 256x28672 interleaved 30720 vs 58368),
    never XCD-major for work stealing or stream-K; the same decision twice in
    a row (the cached one)."""
    M, N, K = shape
    grid = 7 if shape == (1100, 900, 64) else 0
    for _ in range(2):
        plan = pg.plan_gemm(config(), M, N, K, dtype, sched, pg.make_args(tile=tile, grid=grid))
        assert plan["xcd_major"] == want, plan


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
