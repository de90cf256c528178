"""GPU parity of the eight-wave ping-pong bf16 kernel (PGEMM_PIPELINE_PINGPONG)
through the C ABI: against the oracle on ragged and K-tail shapes under every
scheduler and at full size (sampled rows), bit-identical across schedulers (the
per-tile K order does not depend on who computes the tile), every tile
computed exactly once (witness), and graph replays equal to the eager call.
It multiplies 32x32 MFMA blocks while the four-wave kernel uses 16x16 ones, so
the two round differently and are compared through the oracle only."""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import gemm as og
from oracle import sched_model as sm
from synthetic import bf16_bits_normal, bf16_bits_uniform
from oracle.codecs import bf16_to_f64
from tests.gpu_util import BF16_TOL, Guarded, assert_abs_bound, assert_within, config, dev_bf16, note, sync

pytestmark = pytest.mark.gpu

SCHEDS = ["blocked", "interleaved", "grouped", "work_stealing", "blocked_grouped", "work_stealing_xcc"]
TILE = (256, 256, 64)


def _shapes():
    # M any size; N and K multiples of 8 (the direct-to-LDS terms), none a
    # multiple of the tile except where noted: edge tiles in M and N, K tails
    # of every length class, one tile, several rounds of tiles
    Ms = [1, 15, 63, 65, 255, 257, 300, 513, 1000]
    Ns = [8, 56, 136, 264, 520, 776]
    Ks = [8, 56, 64, 72, 136, 200, 520]
    out = []
    for i, M in enumerate(Ms):
        for j in range(2):
            out.append((M, Ns[(i + 2 * j) % len(Ns)], Ks[(i + 3 * j) % len(Ks)]))
    return out + [(256, 256, 64), (512, 512, 512), (1024, 768, 192)]


def _run(a, b, M, N, K, out, sched, pipeline, **kw):
    A, B = dev_bf16(a), dev_bf16(b)
    C = Guarded(M * N, "bf16" if out == "bf16_out_bf16" else "f32")
    note(f"pgemm_run {pipeline} M={M} N={N} K={K} {out} sched={sched} {kw}")
    pg.pgemm_run(config(), A, B, C.view, M, N, K, out, sched, pg.make_args(tile=TILE, pipeline=pipeline, **kw))
    sync()
    assert C.guards_intact(), (M, N, K, sched, pipeline)
    return C


@pytest.mark.parametrize("out", ["bf16_out_f32", "bf16_out_bf16"])
def test_pingpong_against_oracle(out):
    for si, (M, N, K) in enumerate(_shapes()):
        a = bf16_bits_uniform((M, K), 6000 + si)
        b = bf16_bits_uniform((K, N), 6100 + si)
        Cref, Abs = og.gemm_bf16(a, b)
        first = None
        for sched in SCHEDS:
            C = _run(a, b, M, N, K, out, sched, "pingpong")
            assert_within(C.as_f64().reshape(M, N), Cref, Abs, BF16_TOL, out == "bf16_out_bf16",
                          f"pingpong {(M, N, K)} {sched} {out}")
            if first is None:
                first = C.body_bits()
            else:
                assert np.array_equal(C.body_bits(), first), f"pingpong {(M, N, K)} {sched} differs from {SCHEDS[0]}"


@pytest.mark.parametrize("shape", [(8192, 8192, 8192), (5120, 5120, 4096), (4864, 8000, 8192),
                                   (3000, 7000, 2048)])
def test_pingpong_full_size_bit_identical(shape):
    """Full-size workloads: the ping-pong kernel's C under grouped against the
    oracle on sampled rows (both edges of every tile row, random rows), and
    every other scheduler (and paired claims) bit-identical to it."""
    M, N, K = shape
    if shape == (8192, 8192, 8192):
        a, b = bf16_bits_normal((M, K), 1030), bf16_bits_normal((K, N), 1031)
    else:
        a, b = bf16_bits_uniform((M, K), 1040 + M), bf16_bits_uniform((K, N), 1041 + N)
    C = _run(a, b, M, N, K, "bf16_out_bf16", "grouped", "pingpong")
    rows = {0, M - 1}
    for t in range(0, M, 256):
        rows |= {t, min(t + 255, M - 1)}
    rows |= set(np.random.default_rng(M).integers(0, M, size=16).tolist())
    rows = np.array(sorted(rows))
    note(f"oracle on {len(rows)} rows of C ({shape})")
    Cref, Abs = og.gemm_f64_sampled(bf16_to_f64(a), bf16_to_f64(b), rows, np.arange(N))
    assert_abs_bound(C.as_f64().reshape(M, N)[rows, :], Cref, Abs, BF16_TOL, f"pingpong {shape} grouped")
    ref = C.body_bits()
    for sched, chunk in [(s, 0) for s in SCHEDS] + [("work_stealing", pg._abi.CLAIM_PAIRS)]:
        got = _run(a, b, M, N, K, "bf16_out_bf16", sched, "pingpong", claim_chunk=chunk).body_bits()
        assert np.array_equal(got, ref), f"{shape} {sched} chunk={chunk}"


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("shape", [(5120, 5120, 256), (3000, 7000, 128), (8192, 8192, 64), (600, 304, 64)])
def test_pingpong_schedule_exactly_once(sched, shape):
    cfg = config()
    M, N, K = shape
    args = pg.make_args(tile=TILE, pipeline="pingpong")
    plan = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", sched, args)
    assert plan["kernel"] == "bf16_pingpong" and plan["threads"] == 512
    G, T = plan["grid"], plan["tiles"]
    pm, pn = -(-M // 256), -(-N // 256)
    cfg.witness_enable(T, G)
    a, b = bf16_bits_uniform((M, K), 1), bf16_bits_uniform((K, N), 2)
    A, B = dev_bf16(a), dev_bf16(b)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    note(f"witness pingpong {shape} {sched} grid={G}")
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched,
                 pg.make_args(tile=TILE, pipeline="pingpong", debug_flags=pg._abi.DEBUG_WITNESS))
    w = cfg.witness_read(T, G)
    visits, owner, order = w["visits"][:T], w["owner"][:T], w["order"][:T]
    assert np.all(visits == 1), f"{sched}: tiles visited {np.unique(visits)} times"
    X = cfg.info["num_xcds"]
    if sched in ("blocked", "interleaved", "grouped", "blocked_grouped"):
        for p, seq in enumerate(sm.static_schedule(sched, pm, pn, G, 8)):
            for i, (v, _, _) in enumerate(seq):
                assert owner[v] == p and order[v] == i, (sched, v)
    elif sched == "work_stealing":
        sm.check_ws_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                              T, G, X, 1, claims=w["claims"][:G, :X].tolist())
    else:
        homes = [((int(h) >> 16) & 0xF) % X for h in w["hw_id"][:G]]
        sm.check_wsx_execution(visits.tolist(), owner.tolist(), order.tolist(), w["counters"].tolist(),
                               homes, T, G, X, 1, claims=w["claims"][:G, :X].tolist())
    # the witness build computes the same bits as the timed build
    C2 = torch.empty_like(C)
    pg.pgemm_run(cfg, A, B, C2, M, N, K, "bf16_out_bf16", sched, args)
    sync()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))


def test_pingpong_graph_replays():
    cfg = config()
    M, N, K = 1536, 1280, 512
    a, b = bf16_bits_uniform((M, K), 11), bf16_bits_uniform((K, N), 12)
    A, B = dev_bf16(a), dev_bf16(b)
    args = pg.make_args(tile=TILE, pipeline="pingpong")
    ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(ref)
    note("pingpong graph capture (work stealing)")
    pg.pgemm_run(cfg, A, B, ref, M, N, K, "bf16_out_bf16", "work_stealing", args)
    sync()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pg.pgemm_run(cfg, A, B, out, M, N, K, "bf16_out_bf16", "work_stealing", args)
    sync()
    for r in range(3):
        out.zero_()
        g.replay()
        sync()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        pg.pgemm_run(cfg, A, B, ref, M, N, K, "bf16_out_bf16", "work_stealing", args)  # eager in between
        sync()


def test_pingpong_unsupported_requests():
    cfg = config()
    M, N, K = 512, 512, 512
    A = dev_bf16(bf16_bits_uniform((M, K), 3))
    B = dev_bf16(bf16_bits_uniform((K, N), 4))
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    for sched, tile in [("stream_k", TILE), ("work_stealing", (128, 128, 64))]:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched, pg.make_args(tile=tile, pipeline="pingpong"))
        assert e.value.code == pg._abi.ERR_UNSUPPORTED, (sched, tile)
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run_grouped(cfg, [(A, B, C, M, N, K)], "bf16_out_bf16", "grouped",
                             pg.make_args(tile=TILE, pipeline="pingpong"))
    assert e.value.code == pg._abi.ERR_UNSUPPORTED
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", "grouped", pg.make_args(tile=TILE, pipeline=7))
    assert e.value.code == pg._abi.ERR_INVALID
    sync()
