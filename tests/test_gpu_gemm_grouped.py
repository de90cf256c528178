"""GPU parity of several GEMMs in one persistent launch (pgemm_run_grouped):
every problem within the tolerance of the oracle and bit-identical to a
pgemm_run of that problem alone (same tile, same per-tile K order); every
tile of the shared virtual id space computed once; static schedules equal
to the oracle's multi-problem model tile for tile."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import gemm as og
from oracle import sched_model as sm
from synthetic import bf16_bits_uniform, fp8_blockscaled
from tests.gpu_util import BF16_TOL, FP8_TOL, Guarded, assert_abs_bound, assert_within, config, dev_bf16, note, sync

pytestmark = pytest.mark.gpu

SCHEDS = ["blocked", "interleaved", "grouped", "work_stealing", "blocked_grouped", "work_stealing_xcc"]
# (M, N, K) per problem: different K (slab counts) and N (strides), ragged
# edges, an empty problem, one problem
SETS = [
    [(512, 512, 256), (300, 136, 72), (1024, 256, 64)],
    [(1000, 904, 520)],
    [(256, 128, 8), (0, 64, 64), (130, 200, 328), (64, 64, 64)],
    [(96, 64, 64)] * 8,
]


def _data(shapes, seed):
    return [(bf16_bits_uniform((M, K), seed + 2 * g), bf16_bits_uniform((K, N), seed + 2 * g + 1))
            for g, (M, N, K) in enumerate(shapes)]


def _run(shapes, ab, out, sched, tile, **kw):
    cfg = config()
    probs, outs = [], []
    for (M, N, K), (a, b) in zip(shapes, ab):
        C = Guarded(M * N, "bf16" if out == "bf16_out_bf16" else "f32")
        A = dev_bf16(a) if M * K else torch.empty(8, dtype=torch.bfloat16, device="cuda:0")
        B = dev_bf16(b)
        probs.append((A, B, C.view if M * N else C.full, M, N, K))
        outs.append(C)
    note(f"pgemm_run_grouped {shapes} {out} sched={sched} tile={tile} {kw}")
    pg.pgemm_run_grouped(cfg, probs, out, sched, pg.make_args(tile=tile, **kw))
    sync()
    return outs


@pytest.mark.parametrize("si", [0, 3])
def test_grouped_program_order_keeps_c(si):
    """Several problems in one launch under both program numberings of the
    static walks: every problem's C bit-identical."""
    shapes = SETS[si]
    ab = _data(shapes, 4500 + 10 * si)
    for sched in ["blocked", "interleaved", "grouped", "blocked_grouped"]:
        got = {o: _run(shapes, ab, "bf16_out_bf16", sched, (128, 128, 64), program_order=o)
               for o in ("xcd_major", "dispatch")}
        for g, (Cx, Cd) in enumerate(zip(got["xcd_major"], got["dispatch"])):
            assert Cx.guards_intact() and Cd.guards_intact()
            assert np.array_equal(Cx.body_bits(), Cd.body_bits()), (si, sched, g)


@pytest.mark.parametrize("tile", [(128, 128, 64), (256, 256, 64)])
@pytest.mark.parametrize("out", ["bf16_out_f32", "bf16_out_bf16"])
@pytest.mark.parametrize("si", range(len(SETS)))
def test_grouped_parity(tile, out, si):
    shapes = SETS[si]
    ab = _data(shapes, 4000 + 10 * si)
    cfg = config()
    alone = []
    for (M, N, K), (a, b) in zip(shapes, ab):
        if M * N == 0:
            alone.append(None)
            continue
        C = Guarded(M * N, "bf16" if out == "bf16_out_bf16" else "f32")
        pg.pgemm_run(cfg, dev_bf16(a), dev_bf16(b), C.view, M, N, K, out, "grouped", pg.make_args(tile=tile))
        sync()
        alone.append(C.body_bits())
    for sched in SCHEDS:
        outs = _run(shapes, ab, out, sched, tile)
        for g, ((M, N, K), (a, b), C) in enumerate(zip(shapes, ab, outs)):
            assert C.guards_intact(), (shapes, sched, g)
            if M * N == 0:
                continue
            assert np.array_equal(C.body_bits(), alone[g]), f"{shapes[g]} {sched}: differs from its own pgemm_run"
            if sched == "grouped":
                Cref, Abs = og.gemm_bf16(a, b)
                assert_within(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, out == "bf16_out_bf16",
                              f"{shapes[g]} {tile} {out}")


@pytest.mark.parametrize("sched", SCHEDS)
def test_grouped_schedule(sched):
    shapes = [(512, 512, 256), (300, 136, 72), (0, 64, 64), (1024, 256, 64)]
    tile = (128, 128, 64)
    grids = [(-(-M // 128), -(-N // 128)) for M, N, K in shapes]
    T = sm.multi_offsets(grids)[-1]
    cfg = config()
    # the launch's grid: the balanced grid of all problems' tiles together
    occ = pg.plan_gemm(cfg, 512, 512, 256, "bf16_out_bf16", sched, pg.make_args(tile=tile))["occupancy"]
    G = sm.balanced_grid(T, cfg.info["num_cus"] * occ, cfg.info["num_xcds"])
    cfg.witness_enable(T, G)
    _run(shapes, _data(shapes, 4100), "bf16_out_bf16", sched, tile, debug_flags=pg._abi.DEBUG_WITNESS)
    w = cfg.witness_read(T, G)
    visits, owner, order = w["visits"][:T], w["owner"][:T], w["order"][:T]
    assert np.all(visits == 1)
    X = cfg.info["num_xcds"]
    if sched in sm.STATIC_KINDS:
        for p, seq in enumerate(sm.multi_static_schedule(sched, grids, G)):
            for i, (v, *_rest) in enumerate(seq):
                assert owner[v] == p and order[v] == i, (sched, v)
    elif sched == "work_stealing":
        sm.check_ws_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                              T, G, X, claims=w["claims"][:G, :X].tolist())
    else:
        homes = [((int(h) >> 16) & 0xF) % X for h in w["hw_id"][:G]]
        sm.check_wsx_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                               homes, T, G, X, claims=w["claims"][:G, :X].tolist())


def test_grouped_errors():
    cfg = config()
    a = dev_bf16(bf16_bits_uniform((256, 128), 1))
    b = dev_bf16(bf16_bits_uniform((128, 256), 2))
    c = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda:0")
    d = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda:0")
    b100 = dev_bf16(bf16_bits_uniform((100, 256), 3))
    ok = (a, b, c, 256, 256, 128)
    cases = [
        ([], "bf16_out_bf16", "grouped", pg._abi.ERR_INVALID),
        ([ok] * 9, "bf16_out_bf16", "grouped", pg._abi.ERR_INVALID),
        ([ok, (a, b, c, 256, 256, 128)], "bf16_out_bf16", "grouped", pg._abi.ERR_INVALID),   # two write c
        ([ok, (c, b, d, 256, 256, 128)], "bf16_out_bf16", "grouped", pg._abi.ERR_INVALID),   # reads c
        ([(a, b100, d, 256, 256, 100)], "bf16_out_bf16", "grouped", pg._abi.ERR_UNSUPPORTED),  # K % 8
        ([ok], "bf16_out_bf16", "stream_k", pg._abi.ERR_UNSUPPORTED),
        ([(a.data_ptr(), b.data_ptr(), c.data_ptr(), 256, 256, 128)], "fp8_b128_out_bf16", "grouped",
         pg._abi.ERR_INVALID),                                                              # no scales
        ([(a, b, c, 256, 256, 0)], "bf16_out_bf16", "grouped", pg._abi.ERR_INVALID),          # K = 0
    ]
    for probs, dt, sched, code in cases:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_run_grouped(cfg, probs, dt, sched)
        assert e.value.code == code, (len(probs), dt, sched)
    # bf16 tensors given as fp8 operands: refused by the binding before the call
    with pytest.raises(ValueError, match="dtype"):
        pg.pgemm_run_grouped(cfg, [ok], "fp8_b128_out_bf16", "grouped")


# fp8: (M, N, K) per problem, K a multiple of 128, N of 16
FP8_SETS = [
    [(256, 1024, 512), (100, 272, 256), (0, 64, 128), (384, 128, 1024)],
    [(96, 48, 128)] * 8,
]


@pytest.mark.parametrize("tile", [(128, 128, 128), (256, 256, 128), (128, 256, 128)])
@pytest.mark.parametrize("si", range(len(FP8_SETS)))
def test_grouped_fp8_parity(tile, si):
    shapes = FP8_SETS[si]
    cfg = config()
    data, alone = [], []
    for g, (M, N, K) in enumerate(shapes):
        qa, sa = fp8_blockscaled(M, K, 4200 + 4 * g, 4202 + 4 * g, k_major=True)
        qb, sb = fp8_blockscaled(N, K, 4201 + 4 * g, 4203 + 4 * g, k_major=False)
        dev = [torch.from_numpy(x).to("cuda:0") if x.size else torch.empty(16, dtype=torch.uint8, device="cuda:0")
               for x in (qa, qb, sa, sb)]
        data.append((qa, sa, qb, sb, dev))
        if M * N == 0:
            alone.append(None)
            continue
        C = Guarded(M * N, "bf16")
        pg.pgemm_run(cfg, dev[0], dev[1], C.view, M, N, K, "fp8_b128_out_bf16", "grouped",
                     pg.make_args(tile=tile, a_scale=dev[2], b_scale=dev[3]))
        sync()
        alone.append(C.body_bits())
    for sched in SCHEDS:
        probs, outs = [], []
        for (M, N, K), (qa, sa, qb, sb, dev) in zip(shapes, data):
            C = Guarded(M * N, "bf16")
            probs.append((dev[0], dev[1], C.view if M * N else C.full, M, N, K, dev[2], dev[3]))
            outs.append(C)
        note(f"pgemm_run_grouped fp8 {shapes} sched={sched} tile={tile}")
        pg.pgemm_run_grouped(cfg, probs, "fp8_b128_out_bf16", sched, pg.make_args(tile=tile))
        sync()
        for g, ((M, N, K), (qa, sa, qb, sb, dev), C) in enumerate(zip(shapes, data, outs)):
            assert C.guards_intact(), (shapes, sched, g)
            if M * N == 0:
                continue
            assert np.array_equal(C.body_bits(), alone[g]), f"fp8 {shapes[g]} {sched}: differs from its own pgemm_run"
            if sched == "grouped":
                Cref, Abs = og.gemm_fp8_b128(qa, sa, qb, sb)
                assert_abs_bound(C.as_f64().reshape(M, N), Cref, Abs, FP8_TOL, f"fp8 {shapes[g]} {tile}")

