"""A pgemm_run / padd_run call captured in a HIP graph: the work-stealing
counter reset is a fill kernel on the call's stream (no memset node), so
every replay starts from zeroed counters.  Each replay is checked bit for
bit against the eager result, with eager work and synchronisations between
the replays."""
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from synthetic import bf16_bits_uniform, f32_normal
from tests.gpu_util import config, dev_bf16, dev_f32, note, sync

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sched", ["work_stealing", "grouped", "work_stealing_xcc", "stream_k"])
def test_gemm_graph_replays(sched):
    # stream-K: the eager call below sizes the workspace first, so the
    # captured call allocates nothing
    cfg = config()
    M, N, K = 1536, 1280, 512
    A = dev_bf16(bf16_bits_uniform((M, K), 71))
    B = dev_bf16(bf16_bits_uniform((K, N), 72))
    ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(ref)
    args = pg.make_args(tile=(256, 256, 64))
    note(f"graph gemm {M}x{N}x{K} {sched}")
    pg.pgemm_run(cfg, A, B, ref, M, N, K, "bf16_out_bf16", sched, args)  # eager, also warms up
    sync()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pg.pgemm_run(cfg, A, B, out, M, N, K, "bf16_out_bf16", sched, args)
    sync()
    junk = torch.zeros(1 << 20, device="cuda:0")
    for r in range(4):
        out.fill_(float("nan"))
        junk.add_(1.0)                      # unrelated eager work between replays
        pg.pgemm_run(cfg, A, B, ref, M, N, K, "bf16_out_bf16", sched, args)  # eager call in between
        sync()
        g.replay()
        sync()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"


@pytest.mark.parametrize("sched", ["work_stealing", "stream_k"])
def test_fp8_gemm_graph_replays(sched):
    """Block-scaled fp8 under work stealing and stream-K (1536x1280 at
    256x256 tiles: 30 tiles on 256 programs, so stream-K splits every one)."""
    from synthetic import fp8_blockscaled
    from tests.gpu_util import dev_u8
    cfg = config()
    M, N, K = 1536, 1280, 512
    qa, sa = fp8_blockscaled(M, K, 75, 77, k_major=True)
    qb, sb = fp8_blockscaled(N, K, 76, 78, k_major=False)
    A, B, SA, SB = dev_u8(qa), dev_u8(qb), dev_u8(sa), dev_u8(sb)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(ref)
    args = pg.make_args(tile=(256, 256, 128), a_scale=SA, b_scale=SB)
    note(f"graph fp8 gemm {M}x{N}x{K} {sched}")
    pg.pgemm_run(cfg, A, B, ref, M, N, K, "fp8_b128_out_bf16", sched, args)  # eager; sizes the workspace
    sync()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pg.pgemm_run(cfg, A, B, out, M, N, K, "fp8_b128_out_bf16", sched, args)
    sync()
    for r in range(4):
        out.fill_(float("nan"))
        pg.pgemm_run(cfg, A, B, ref, M, N, K, "fp8_b128_out_bf16", sched, args)  # eager call in between
        sync()
        g.replay()
        sync()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"


def test_add_graph_replays():
    cfg = config()
    rows, cols = 1000, 3000
    X, Y = dev_f32(f32_normal((rows, cols), 73)), dev_f32(f32_normal((rows, cols), 74))
    ref = X + Y
    out = torch.empty_like(X)
    note("graph add work stealing")
    pg.padd_run(cfg, X, Y, out, rows, cols, 32, 16, "work_stealing")
    sync()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pg.padd_run(cfg, X, Y, out, rows, cols, 32, 16, "work_stealing")
    sync()
    for r in range(4):
        out.fill_(float("nan"))
        sync()
        g.replay()
        sync()
        assert torch.equal(out, ref), f"replay {r}"


def test_grouped_gemm_and_multi_add_graph_replays():
    """Several GEMMs and several adds per launch, captured together."""
    cfg = config()
    shapes = [(512, 256, 128), (300, 512, 256), (64, 128, 64)]
    probs, refs = [], []
    for g, (M, N, K) in enumerate(shapes):
        A = dev_bf16(bf16_bits_uniform((M, K), 80 + g))
        B = dev_bf16(bf16_bits_uniform((K, N), 90 + g))
        probs.append((A, B, torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0"), M, N, K))
    adds = []
    for g, (r, c) in enumerate([(700, 900), (64, 4096)]):
        X, Y = dev_f32(f32_normal((r, c), 100 + g)), dev_f32(f32_normal((r, c), 110 + g))
        adds.append((X, Y, torch.empty_like(X), r, c))
    note("graph grouped GEMM + several adds")
    pg.pgemm_run_grouped(cfg, probs, "bf16_out_bf16", "work_stealing")
    pg.padd_run_multi(cfg, adds, 32, 16, "work_stealing")
    sync()
    refs = [p[2].clone() for p in probs] + [a[2].clone() for a in adds]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pg.pgemm_run_grouped(cfg, probs, "bf16_out_bf16", "work_stealing")
            pg.padd_run_multi(cfg, adds, 32, 16, "work_stealing")
    sync()
    outs = [p[2] for p in probs] + [a[2] for a in adds]
    for r in range(4):
        for o in outs:
            o.fill_(float("nan"))
        sync()
        g.replay()
        sync()
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32)), \
                f"replay {r} output {i}"

