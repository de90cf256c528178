"""GPU parity of several adds in one persistent launch (padd_run_multi):
every problem bit-exact against the oracle add, guard bands intact, every
tile of the shared virtual id space computed once, static schedules equal
to the oracle's multi-problem model tile for tile."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import sched_model as sm
from oracle.add import add_f32
from synthetic import f32_normal
from tests.gpu_util import Guarded, config, dev_f32, note, sync

pytestmark = pytest.mark.gpu

SCHEDS = ["blocked", "interleaved", "grouped", "work_stealing", "blocked_grouped", "work_stealing_xcc"]
# problem sets: ragged edges, one problem, an empty problem, columns not a
# multiple of 4 (scalar path), many small problems
SETS = [
    [(1000, 1000), (300, 4000), (64, 64)],
    [(999, 1001)],
    [(257, 130), (0, 100), (33, 20), (5, 0)],
    [(129, 35), (64, 64)],
    [(17, 16)] * 8,
]


def _inputs(shapes, seed):
    return [(f32_normal((r, c), seed + 2 * g), f32_normal((r, c), seed + 2 * g + 1))
            for g, (r, c) in enumerate(shapes)]


def _run(shapes, xy, tile, sched, **kw):
    cfg = config()
    devs, outs = [], []
    for (r, c), (x, y) in zip(shapes, xy):
        C = Guarded(r * c, "f32")
        X = dev_f32(x) if r * c else torch.empty(1, dtype=torch.float32, device="cuda:0")
        Y = dev_f32(y) if r * c else torch.empty(1, dtype=torch.float32, device="cuda:0")
        devs.append((X, Y, C.view if r * c else C.full.view(torch.float32), r, c))
        outs.append(C)
    note(f"padd_run_multi {shapes} tile={tile} sched={sched} {kw}")
    pg.padd_run_multi(cfg, devs, tile[0], tile[1], sched, pg.make_args(**kw))
    sync()
    return outs


@pytest.mark.parametrize("tile", [(32, 16), (128, 128)])
@pytest.mark.parametrize("si", range(len(SETS)))
def test_multi_add_bit_exact(tile, si):
    shapes = SETS[si]
    xy = _inputs(shapes, 3000 + 10 * si)
    for sched in SCHEDS:
        outs = _run(shapes, xy, tile, sched)
        for g, ((r, c), (x, y), C) in enumerate(zip(shapes, xy, outs)):
            assert C.guards_intact(), (shapes, tile, sched, g)
            if r * c:
                want = add_f32(x, y).view(np.uint32).ravel()
                assert np.array_equal(C.body_bits().view(np.uint32), want), (shapes, tile, sched, g)


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("tile", [(32, 16), (64, 64)])
def test_multi_add_schedule(sched, tile):
    shapes = [(1000, 1000), (300, 4000), (0, 7), (64, 64)]
    grids = [(-(-r // tile[0]), -(-c // tile[1])) for r, c in shapes]
    T = sm.multi_offsets(grids)[-1]
    cfg = config()
    G = pg.plan_add(cfg, 1000, 1000, tile[0], tile[1], sched)["grid"]
    cfg.witness_enable(T, G)
    xy = _inputs(shapes, 3100)
    _run(shapes, xy, tile, sched, debug_flags=pg._abi.DEBUG_WITNESS)
    w = cfg.witness_read(T, G)
    visits, owner, order = w["visits"][:T], w["owner"][:T], w["order"][:T]
    assert np.all(visits == 1)
    X = cfg.info["num_xcds"]
    chunk = {(32, 16): 32, (64, 64): 4}[tile]
    if sched in sm.STATIC_KINDS:
        for p, seq in enumerate(sm.multi_static_schedule(sched, grids, G)):
            for i, (v, *_rest) in enumerate(seq):
                assert owner[v] == p and order[v] == i, (sched, v)
    elif sched == "work_stealing":
        sm.check_ws_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                              T, G, X, chunk, claims=w["claims"][:G, :X].tolist())
    else:
        homes = [((int(h) >> 16) & 0xF) % X for h in w["hw_id"][:G]]
        sm.check_wsx_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                               homes, T, G, X, chunk, claims=w["claims"][:G, :X].tolist())


def test_multi_add_one_problem_equals_single_call():
    x, y = f32_normal((777, 1234), 41), f32_normal((777, 1234), 42)
    cfg = config()
    X, Y = dev_f32(x), dev_f32(y)
    C1 = torch.empty_like(X)
    C2 = torch.empty_like(X)
    pg.padd_run(cfg, X, Y, C1, 777, 1234, 32, 16, "grouped")
    pg.padd_run_multi(cfg, [(X, Y, C2, 777, 1234)], 32, 16, "grouped")
    sync()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_multi_add_in_place_and_errors():
    cfg = config()
    a, b = f32_normal((300, 400), 7), f32_normal((300, 400), 8)
    c, d = f32_normal((50, 60), 9), f32_normal((50, 60), 10)
    A, B, Cc, D = dev_f32(a), dev_f32(b), dev_f32(c), dev_f32(d)
    # in place within a problem is allowed
    pg.padd_run_multi(cfg, [(A, B, A, 300, 400), (Cc, D, Cc, 50, 60)], 32, 16, "work_stealing")
    sync()
    assert np.array_equal(A.cpu().numpy().view(np.uint32), add_f32(a, b).view(np.uint32))
    assert np.array_equal(Cc.cpu().numpy().view(np.uint32), add_f32(c, d).view(np.uint32))
    E = torch.empty_like(A)
    bad = [
        ([], (32, 16), pg._abi.ERR_INVALID),                                    # no problem
        ([(A, B, E, 300, 400)] * 9, (32, 16), pg._abi.ERR_INVALID),             # too many
        ([(A, B, E, 300, 400), (E, D, Cc, 50, 60)], (32, 16), pg._abi.ERR_INVALID),  # C of 0 read by 1
        ([(A, B, E, 300, 400), (Cc, D, E, 50, 60)], (32, 16), pg._abi.ERR_INVALID),  # two problems write E
        ([(A, B, E, 300, 400)], (16, 16), pg._abi.ERR_UNSUPPORTED),            # tile not built
        ([(A, B, E, -1, 400)], (32, 16), pg._abi.ERR_INVALID),                 # negative size
    ]
    for probs, tile, code in bad:
        with pytest.raises(pg.PgemmError) as e:
            pg.padd_run_multi(cfg, probs, tile[0], tile[1], "blocked")
        assert e.value.code == code, (len(probs), tile)
    with pytest.raises(pg.PgemmError) as e:
        pg.padd_run_multi(cfg, [(A, B, E, 300, 400)], 32, 16, "work_stealing",
                          pg.make_args(claim_chunk=pg._abi.CLAIM_PAIRS))
    assert e.value.code == pg._abi.ERR_UNSUPPORTED
