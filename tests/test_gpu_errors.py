"""Argument checking of the C ABI on a GPU, and failure detection forced from
the host (stale counters, a straggling program).  Every kernel launched here
exits normally."""
import ctypes

import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from tile_scheduling_persistent_amd import _abi
from oracle import sched_model as sm
from synthetic import bf16_bits_uniform
from tests.gpu_util import config, dev_bf16, note, sync

pytestmark = pytest.mark.gpu


def _status(fn, *a):
    return fn(*a)


def test_config_rejects_small_counter_array():
    h = ctypes.c_void_p()
    X = config().info["num_xcds"]
    assert _abi.lib().pgemm_config_create(0, X - 1, ctypes.byref(h)) == _abi.ERR_INVALID
    assert _abi.lib().pgemm_config_create(99, 0, ctypes.byref(h)) == _abi.ERR_INVALID
    assert _abi.lib().pgemm_config_create(0, 0, None) == _abi.ERR_INVALID
    with pg.Config(0, X) as c:
        assert c.info["counter_capacity"] == X


def test_device_facts():
    info = config().info
    assert info["arch"].startswith("gfx950")
    assert info["num_cus"] >= info["num_xcds"] >= 1
    note(f"device facts {info}")


def test_invalid_arguments_enqueue_nothing():
    cfg = config()
    L = _abi.lib()
    A = torch.zeros(64 * 64, dtype=torch.bfloat16, device="cuda:0")
    B = torch.zeros(64 * 64, dtype=torch.bfloat16, device="cuda:0")
    C = torch.full((64 * 64,), 7.0, dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    a, b, c = A.data_ptr(), B.data_ptr(), C.data_ptr()
    run = lambda *x: L.pgemm_run(cfg.handle, *x)  # noqa: E731
    assert run(None, b, c, 64, 64, 64, 0, 0, None, s) == _abi.ERR_INVALID
    assert run(a, b, c, 0, 64, 64, 0, 0, None, s) == _abi.ERR_INVALID
    assert run(a, b, c, 64, -1, 64, 0, 0, None, s) == _abi.ERR_INVALID
    assert run(a, b, c, 64, 64, 64, 9, 0, None, s) == _abi.ERR_INVALID          # dtype
    assert run(a, b, c, 64, 64, 64, 0, 17, None, s) == _abi.ERR_INVALID         # sched
    assert run(a, b, a, 64, 64, 64, 1, 0, None, s) == _abi.ERR_INVALID          # C aliases A
    host = np.zeros(64 * 64, np.float32)
    assert run(a, b, host.ctypes.data, 64, 64, 64, 0, 0, None, s) == _abi.ERR_INVALID
    args = pg.make_args(tile=(64, 32, 16))
    assert run(a, b, c, 64, 64, 64, 0, 0, ctypes.byref(args), s) == _abi.ERR_UNSUPPORTED
    args = pg.make_args(group_size=-1)
    assert run(a, b, c, 64, 64, 64, 0, 2, ctypes.byref(args), s) == _abi.ERR_INVALID
    args = pg.make_args(grid=cfg.info["num_xcds"] - 1)
    assert run(a, b, c, 64, 64, 64, 0, 3, ctypes.byref(args), s) == _abi.ERR_INVALID
    for order in (-1, 3):                                                     # program_order
        args = pg.make_args(program_order=order)
        assert run(a, b, c, 64, 64, 64, 0, 2, ctypes.byref(args), s) == _abi.ERR_INVALID
        pl = _abi.pgemm_plan()
        assert L.pgemm_plan_gemm(cfg.handle, a, b, c, 64, 64, 64, 0, 2, ctypes.byref(args),
                                 ctypes.byref(pl)) == _abi.ERR_INVALID
    # fp8 without scales, or K not a multiple of 128
    assert run(a, b, c, 64, 64, 128, 2, 0, None, s) == _abi.ERR_INVALID
    sync()
    assert torch.all(C == 7.0)
    X = torch.zeros(100, dtype=torch.float32, device="cuda:0")
    assert L.padd_run(cfg.handle, X.data_ptr(), X.data_ptr(), X.data_ptr(), 10, 10, 7, 7, 0,
                      None, s) == _abi.ERR_UNSUPPORTED
    assert L.padd_run(cfg.handle, X.data_ptr(), X.data_ptr(), X.data_ptr() + 4, 10, 9, 32, 16, 0,
                      None, s) == _abi.ERR_INVALID                              # partial overlap


def test_stale_counters_are_detected():
    """Skipping the counter reset leaves the counters at their final values:
    every claim fails, no tile is computed, and the witness shows it."""
    cfg = config()
    M = N = 1024
    K = 128
    a, b = bf16_bits_uniform((M, K), 1), bf16_bits_uniform((K, N), 2)
    A, B = dev_bf16(a), dev_bf16(b)
    T = 16
    G = pg.plan_gemm(cfg, M, N, K, "bf16_out_f32", "work_stealing")["grid"]
    cfg.witness_enable(T, G)
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda:0")
    flags = _abi.DEBUG_WITNESS
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_f32", "work_stealing", pg.make_args(debug_flags=flags))
    w1 = cfg.witness_read(T, G)
    assert np.all(w1["visits"] == 1)
    C.fill_(-5.0)
    note("work stealing with the reset skipped")
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_f32", "work_stealing",
                 pg.make_args(debug_flags=flags | _abi.DEBUG_SKIP_RESET))
    w2 = cfg.witness_read(T, G)
    sync()
    assert np.all(w2["visits"] == 0)
    assert torch.all(C == -5.0)
    # the normal path resets and recovers
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_f32", "work_stealing", pg.make_args(debug_flags=flags))
    w3 = cfg.witness_read(T, G)
    assert np.all(w3["visits"] == 1)


def test_straggler_rebalanced_by_work_stealing():
    """Program 0 waits 200 us before each tile: under work stealing its XCD
    peers take its share; under blocked ranges it keeps its full share."""
    cfg = config()
    X = cfg.info["num_xcds"]
    M = N = 4096
    K = 256
    tile = (128, 128, 64)
    T = (M // 128) * (N // 128)            # 1024 tiles: T / G per program on average
    G = pg.plan_gemm(cfg, M, N, K, "bf16_out_f32", "blocked", pg.make_args(tile=tile))["grid"]
    a, b = bf16_bits_uniform((M, K), 1), bf16_bits_uniform((K, N), 2)
    A, B = dev_bf16(a), dev_bf16(b)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    cfg.witness_enable(T, G)
    flags = _abi.DEBUG_WITNESS | _abi.DEBUG_STRAGGLER
    res = {}
    for sched in ["blocked", "work_stealing"]:
        note(f"straggler {sched}")
        pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_f32", sched,
                     pg.make_args(tile=tile, debug_flags=flags, straggler_program=0,
                                  straggler_ns=200_000))
        w = cfg.witness_read(T, G)
        assert np.all(w["visits"] == 1)
        res[sched] = int(w["n_tiles"][0])
    assert res["blocked"] == T // G
    peers = [p for p in range(G) if p % X == 0]
    assert res["work_stealing"] < T // G, res


def test_slow_xcc_rebalanced_by_stealing_across_xccs():
    """Every program on hardware XCC 0 waits 100 us before each tile.  Per-XCD
    work stealing leaves XCC 0's range to XCC 0's programs; stealing across
    XCDs lets the others take part of it, and still computes every tile
    once with the exact final counters."""
    cfg = config()
    X = cfg.info["num_xcds"]
    M = N = 4096
    K = 256
    tile = (128, 128, 64)
    T = (M // 128) * (N // 128)
    G = pg.plan_gemm(cfg, M, N, K, "bf16_out_f32", "work_stealing", pg.make_args(tile=tile))["grid"]
    a, b = bf16_bits_uniform((M, K), 1), bf16_bits_uniform((K, N), 2)
    A, B = dev_bf16(a), dev_bf16(b)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    cfg.witness_enable(T, G)
    flags = _abi.DEBUG_WITNESS | _abi.DEBUG_STRAGGLER_XCC
    s0, e0 = sm.ws_ranges(T, X)[0]
    stolen = {}
    for sched in ["work_stealing", "work_stealing_xcc"]:
        note(f"slow XCC 0 under {sched}")
        pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_f32", sched,
                     pg.make_args(tile=tile, debug_flags=flags, straggler_program=0,
                                  straggler_ns=100_000))
        w = cfg.witness_read(T, G)
        assert np.all(w["visits"][:T] == 1)
        xcc = (w["hw_id"][:G] >> 16) & 0xF
        owner = w["owner"][:T]
        stolen[sched] = int(sum(1 for v in range(s0, e0) if xcc[owner[v]] != 0))
        if sched == "work_stealing_xcc":
            homes = [int(h) % X for h in xcc]
            sm.check_wsx_execution(w["visits"][:T].tolist(), owner.tolist(), w["order"][:T].tolist(),
                                   w["counters"].tolist(), homes, T, G, X, claims=w["claims"][:G, :X].tolist())
    note(f"tiles of range 0 computed off XCC 0: {stolen}")
    assert stolen["work_stealing_xcc"] > (e0 - s0) // 4, stolen


def test_plan_matches_launch_shape():
    """The persistent grid starts from CUs x resident workgroups per CU of the
    selected kernel (two for 128x128 GEMM tiles, one for 256x256); the GEMM's
    data-parallel schedulers trim it to the balanced grid of the oracle's
    schedule model, stream-K and the add keep all of it."""
    cfg = config()
    cus, X = cfg.info["num_cus"], cfg.info["num_xcds"]
    big = pg.plan_gemm(cfg, 8192, 8192, 8192, "bf16_out_bf16", "work_stealing")
    small = pg.plan_gemm(cfg, 4096, 4096, 4096, "bf16_out_bf16", "work_stealing",
                         pg.make_args(tile=(128, 128, 64)))
    fp8 = pg.plan_gemm(cfg, 256, 28672, 8192, "fp8_b128_out_bf16", "grouped",
                       pg.make_args(tile=(128, 128, 128)))
    ragged = pg.plan_gemm(cfg, 5120, 5120, 4096, "bf16_out_bf16", "interleaved")
    ragged_sk = pg.plan_gemm(cfg, 5120, 5120, 4096, "bf16_out_bf16", "stream_k")
    add = pg.plan_add(cfg, 8192, 8192, 128, 128, "blocked")
    note(f"plans {big} {small} {fp8} {ragged} {ragged_sk} {add}")
    for pl in (big, small, fp8, ragged):
        assert pl["occupancy"] >= 1
        assert pl["grid"] == sm.balanced_grid(pl["tiles"], cus * pl["occupancy"], X)
    for pl in (ragged_sk, add):
        assert pl["grid"] == cus * pl["occupancy"]
    if cus == 256 and X == 8:
        assert (big["grid"], small["grid"], fp8["grid"], ragged["grid"]) == (256, 512, 448, 200)
    assert big["kernel"] == "bf16_lds" and big["tiles"] == 32 * 32 and big["occupancy"] == 1
    assert small["kernel"] == "bf16_lds" and small["occupancy"] == 2
    assert fp8["kernel"] == "fp8" and fp8["tiles"] == 2 * 224 and fp8["occupancy"] == 2
    assert add["kernel"] == "add" and add["tiles"] == 64 * 64 and add["occupancy"] == 1
    assert pg.plan_gemm(cfg, 100, 100, 100, "bf16_out_bf16", "blocked", pg.make_args(grid=7))["grid"] == 7
    staged = pg.plan_gemm(cfg, 512, 512, 500, "bf16_out_bf16", "blocked")
    assert staged["kernel"] == "bf16_staged"


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    lib.hipFree.argtypes = [ctypes.c_void_p]
    return lib


def test_buffer_ranges_must_lie_in_one_allocation():
    """The library checks each buffer's byte range against the device
    allocation that holds it (the kernels address by the sizes given).  Probed
    with PGEMM_DEBUG_VALIDATE_ONLY, so nothing is launched either way."""
    cfg = config()
    L = _abi.lib()
    hip = _hip()
    size = 4 << 20
    p = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(p), size) == 0
    try:
        base, end = p.value, p.value + size
        s = torch.cuda.current_stream().cuda_stream
        chk = pg.make_args(debug_flags=_abi.DEBUG_VALIDATE_ONLY)
        M, N, K = 256, 512, 1024
        a, b = base, base + M * K * 2                       # A then B, 1.5 MiB
        c_fit = end - M * N * 2                             # bf16 C ending at the allocation's end
        run = lambda A, B, C, dt=1: L.pgemm_run(cfg.handle, A, B, C, M, N, K, dt, 3,  # noqa: E731
                                               ctypes.byref(chk), s)
        assert run(a, b, c_fit) == _abi.OK
        assert run(a, b, c_fit + 256) == _abi.ERR_INVALID          # C runs 256 B past the end
        assert run(a, b, c_fit, dt=0) == _abi.ERR_INVALID           # fp32 C is twice as long
        c_mid = base + (3 << 19)                            # C at 1.5 MiB, clear of A and B below
        assert run(a, b, c_mid) == _abi.OK
        assert run(end - M * K * 2 + 16, b, c_mid) == _abi.ERR_INVALID   # A past the end
        assert run(a, end - K * N * 2 + 2, c_mid) == _abi.ERR_INVALID    # B past the end
        # the add: X, Y, C of rows * cols floats
        r, cc = 64, 1024
        x_fit = end - r * cc * 4
        add = lambda X, Y, C: L.padd_run(cfg.handle, X, Y, C, r, cc, 32, 16, 0,  # noqa: E731
                                        ctypes.byref(chk), s)
        assert add(base, base + r * cc * 4, x_fit) == _abi.OK
        assert add(base, base + r * cc * 4, x_fit + 4) == _abi.ERR_INVALID
        assert add(x_fit + 4, base, base + r * cc * 4) == _abi.ERR_INVALID
        # fp8 scales: [K/128][M] and [K/128][N] bytes
        q = pg.make_args(a_scale=end - (K // 128) * M, b_scale=end - (K // 128) * N - 1,
                         debug_flags=_abi.DEBUG_VALIDATE_ONLY)
        fa, fb, fc = base, base + M * K, base + M * K + K * N
        assert L.pgemm_run(cfg.handle, fa, fb, fc, M, N, K, 2, 3, ctypes.byref(q), s) == _abi.OK
        q.a_scale = end - (K // 128) * M + 1
        assert L.pgemm_run(cfg.handle, fa, fb, fc, M, N, K, 2, 3, ctypes.byref(q), s) == _abi.ERR_INVALID
        sync("validate-only calls")
    finally:
        assert hip.hipFree(p) == 0


def test_counters_zeroed_by_their_last_claim():
    """Per-XCD work stealing zeroes each counter with the last failing claim
    of the launch, so back-to-back launches need no fill kernel: every launch
    of a sequence (bf16 on both pipelines, block-scaled fp8, the add, single
    and paired claims, interleaved with stealing across XCDs, witness and
    skipped-reset launches, which leave the counters dirty and make the next
    call refill them) computes the same bits, and after every launch that
    resets itself the counters read zero."""
    cfg = config()
    X = cfg.info["num_xcds"]
    M, N, K = 1536, 1280, 256
    a, b = bf16_bits_uniform((M, K), 21), bf16_bits_uniform((K, N), 22)
    A, B = dev_bf16(a), dev_bf16(b)
    cfg.witness_enable(64, 1024)

    def counters():
        return cfg.witness_read(0, 0)["counters"][:X]

    def gemm(sched, **kw):
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        note(f"self-reset sequence: {sched} {kw}")
        pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched, pg.make_args(tile=(256, 256, 64), **kw))
        sync()
        return C.view(torch.int16).cpu().numpy()

    ref = gemm("grouped")
    seq = [("work_stealing", {}, True), ("work_stealing", {}, True),
           ("work_stealing", {"claim_chunk": _abi.CLAIM_PAIRS}, True),
           ("work_stealing", {"claim_chunk": 3}, True),
           ("work_stealing", {"pipeline": "pingpong"}, True),
           ("work_stealing_xcc", {}, False), ("work_stealing", {}, True),
           ("work_stealing", {"debug_flags": _abi.DEBUG_WITNESS}, False), ("work_stealing", {}, True),
           ("work_stealing", {"tile": (128, 128, 64)}, True), ("work_stealing", {}, True)]
    for sched, kw, resets in seq:
        kw = dict(kw)
        tile = kw.pop("tile", None)
        if tile:
            C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
            pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched, pg.make_args(tile=tile, **kw))
            sync()
            got = C.view(torch.int16).cpu().numpy()
        else:
            got = gemm(sched, **kw)
        assert np.array_equal(got, ref), (sched, kw)
        c = counters()
        if resets:
            assert np.all(c == 0), (sched, kw, c)
        else:
            assert np.any(c != 0), (sched, kw, c)
    # a skipped reset after a self-resetting launch finds zeroed counters and
    # computes everything; the launch after it refills (the flag marks them dirty)
    gemm("work_stealing")
    assert np.array_equal(gemm("work_stealing", debug_flags=_abi.DEBUG_SKIP_RESET), ref)
    assert np.array_equal(gemm("work_stealing"), ref)
    assert np.all(counters() == 0)
    # the add and block-scaled fp8 on the same counters
    xs = torch.randn(3000, 2000, device="cuda:0")
    ys = torch.randn(3000, 2000, device="cuda:0")
    want = (xs + ys).cpu().numpy().view(np.uint32)
    for _ in range(3):
        z = torch.empty_like(xs)
        pg.padd_run(cfg, xs, ys, z, 3000, 2000, 128, 128, "work_stealing")
        sync()
        assert np.array_equal(z.cpu().numpy().view(np.uint32), want)
        assert np.all(counters() == 0)
    from synthetic import fp8_blockscaled
    qa, sa = fp8_blockscaled(512, 1024, 31, 32, k_major=True)
    qb, sb = fp8_blockscaled(768, 1024, 33, 34, k_major=False)
    fa, fb = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda()
    fsa, fsb = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    outs = []
    for sched in ("grouped", "work_stealing", "work_stealing"):
        C = torch.empty((512, 768), dtype=torch.bfloat16, device="cuda:0")
        pg.pgemm_run(cfg, fa, fb, C, 512, 768, 1024, "fp8_b128_out_bf16", sched,
                     pg.make_args(tile=(128, 128, 128), a_scale=fsa, b_scale=fsb))
        sync()
        outs.append(C.view(torch.int16).cpu().numpy())
        if sched == "work_stealing":
            assert np.all(counters() == 0)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
