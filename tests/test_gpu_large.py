"""GPU parity at sizes past 32-bit byte offsets, through the C ABI.

Each case puts an operand or the output beyond 4 GiB, so any element whose
address were formed in 32 bits would come from (or land at) the wrong place.
Large operands are a seeded block of P rows repeated down the matrix, with P
prime (4099 or 4111), so an address wrapped by 2**32 bytes lands on different
contents.  Rows on both sides of the
4 GiB mark, every ragged edge and a few random rows are checked against the
oracle; guard bands around the output are checked without copying the
output back whole.
"""
import numpy as np
import pytest
import torch

import tile_scheduling_persistent_amd as pg
from oracle import gemm as og
from oracle.add import add_f32
from oracle.codecs import dequant_fp8_a, dequant_fp8_b
from synthetic import bf16_bits_uniform, f32_normal, fp8_blockscaled, rng
from tests.gpu_util import BF16_TOL, FP8_TOL, assert_abs_bound, assert_within, config, note, sync

pytestmark = pytest.mark.gpu

GUARD = 4096
SENT16, SENT32 = 0x7FC1, 0x7FC00001
P_A, P_Y = 4099, 4111   # row periods of the repeated operands (primes)


def repeated(base: np.ndarray, rows: int, torch_dtype) -> torch.Tensor:
    """Device [rows][cols] whose row r is base[r % P]."""
    P = base.shape[0]
    b = torch.from_numpy(np.ascontiguousarray(base)).to("cuda:0").view(torch_dtype)
    out = torch.empty((rows, base.shape[1]), dtype=torch_dtype, device="cuda:0")
    for r0 in range(0, rows, P):
        n = min(P, rows - r0)
        out[r0:r0 + n].copy_(b[:n])
    return out


class BigOut:
    """Output of n elements between guard bands; only the bands and the
    requested rows are ever copied back."""

    def __init__(self, n: int, wide: bool):
        self.n = n
        dt, s = (torch.int32, SENT32) if wide else (torch.int16, SENT16)
        self.sent = s
        self.full = torch.full((n + 2 * GUARD,), s, dtype=dt, device="cuda:0")
        self.body = self.full[GUARD:GUARD + n]

    def guards_intact(self) -> bool:
        lo = self.full[:GUARD].cpu().numpy()
        hi = self.full[GUARD + self.n:].cpu().numpy()
        return bool(np.all(lo == self.sent) and np.all(hi == self.sent))

    def rows(self, rows, width: int) -> torch.Tensor:
        idx = torch.as_tensor(rows, dtype=torch.int64, device="cuda:0")
        return self.body.view(-1, width).index_select(0, idx)


def sample_rows(M: int, row_bytes: int, seed: int) -> np.ndarray:
    """Both ends, every row around the 4 GiB mark and a few random rows."""
    edge = (1 << 32) // row_bytes
    rows = {0, 1, M - 1, M - 2, edge - 1, edge, edge + 1, (M // 256) * 256 - 1, (M // 256) * 256}
    rows |= set(rng(seed).integers(0, M, size=6).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M))


def test_bf16_a_beyond_4gib():
    """A = 139364 x 16384 bf16 (4.57 GB), N = 264 (ragged), K = 16384."""
    M, N, K = 139364, 264, 16384
    cfg = config()
    base = bf16_bits_uniform((P_A, K), 7001)
    b = bf16_bits_uniform((K, N), 7002)
    A = repeated(base.view(np.int16), M, torch.int16).view(torch.bfloat16)
    B = torch.from_numpy(b.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    rows = sample_rows(M, K * 2, 7003)
    assert rows.max() * K * 2 > (1 << 32)
    Cref, Abs = og.gemm_bf16(base[rows % P_A], b)
    for sched, tile in [("work_stealing", (256, 256, 64)), ("grouped", (128, 128, 64)),
                        ("stream_k", (256, 256, 64)), ("work_stealing_xcc", (256, 256, 64))]:
        C = BigOut(M * N, wide=False)
        note(f"pgemm_run bf16 M={M} N={N} K={K} sched={sched} tile={tile}")
        pg.pgemm_run(cfg, A, B, C.body.view(torch.bfloat16), M, N, K, "bf16_out_bf16", sched,
                     pg.make_args(tile=tile))
        sync()
        assert C.guards_intact(), sched
        got = C.rows(rows, N).view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
        assert_abs_bound(got, Cref, Abs, BF16_TOL, f"A > 4 GiB {sched} {tile}")
        del C
    del A
    torch.cuda.empty_cache()


@pytest.mark.parametrize("out", ["bf16_out_bf16", "bf16_out_f32"])
def test_bf16_c_beyond_4gib(out):
    """C = 49163 x 49160 (4.83 GB in bf16, 9.67 GB in fp32), K = 136 (a K tail)."""
    M, N, K = 49163, 49160, 136
    cfg = config()
    a = bf16_bits_uniform((M, K), 7011)
    b = bf16_bits_uniform((K, N), 7012)
    A = torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    B = torch.from_numpy(b.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    wide = out == "bf16_out_f32"
    rows = sample_rows(M, N * (4 if wide else 2), 7013)
    assert rows.max() * N * (4 if wide else 2) > (1 << 32)
    Cref, Abs = og.gemm_bf16(a[rows], b)
    for sched in ["grouped", "work_stealing", "stream_k"]:
        C = BigOut(M * N, wide)
        note(f"pgemm_run M={M} N={N} K={K} {out} sched={sched}")
        view = C.body.view(torch.float32) if wide else C.body.view(torch.bfloat16)
        pg.pgemm_run(cfg, A, B, view, M, N, K, out, sched, pg.make_args(tile=(256, 256, 64)))
        sync()
        assert C.guards_intact(), sched
        r = C.rows(rows, N)
        got = (r.view(torch.float32) if wide else r.view(torch.bfloat16).float()).cpu().numpy()
        # K = 136 keeps |A||B| small, so the bf16 store's own rounding is allowed on top
        assert_within(got.astype(np.float64), Cref, Abs, BF16_TOL, not wide, f"C > 4 GiB {out} {sched}")
        del C, view
        torch.cuda.empty_cache()


def test_fp8_a_beyond_4gib():
    """A = 139364 x 32768 e4m3 (4.57 GB) with its e8m0 scales, N = 256."""
    M, N, K = 139364, 256, 32768
    cfg = config()
    qa_base, sa_base = fp8_blockscaled(P_A, K, 7021, 7022, k_major=True)
    qb, sb = fp8_blockscaled(N, K, 7023, 7024, k_major=False)
    A = repeated(qa_base, M, torch.uint8)
    SA = torch.from_numpy(np.ascontiguousarray(sa_base[:, np.arange(M) % P_A])).to("cuda:0")
    B = torch.from_numpy(qb).to("cuda:0")
    SB = torch.from_numpy(sb).to("cuda:0")
    rows = sample_rows(M, K, 7025)
    assert rows.max() * K > (1 << 32)
    Cref, Abs = og.gemm_f64(dequant_fp8_a(qa_base[rows % P_A], sa_base[:, rows % P_A]),
                            dequant_fp8_b(qb, sb))
    for sched, tile in [("work_stealing", (256, 256, 128)), ("grouped", (128, 128, 128)),
                        ("interleaved", (128, 256, 128)), ("stream_k", (256, 256, 128))]:
        C = BigOut(M * N, wide=False)
        note(f"pgemm_run fp8 M={M} N={N} K={K} sched={sched} tile={tile}")
        pg.pgemm_run(cfg, A, B, C.body.view(torch.bfloat16), M, N, K, "fp8_b128_out_bf16", sched,
                     pg.make_args(tile=tile, a_scale=SA, b_scale=SB))
        sync()
        assert C.guards_intact(), sched
        got = C.rows(rows, N).view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
        assert_abs_bound(got, Cref, Abs, FP8_TOL, f"fp8 A > 4 GiB {sched} {tile}")
        del C
    del A
    torch.cuda.empty_cache()


def test_add_beyond_4gib():
    """X, Y, C = 32771 x 33000 fp32 (4.33 GB each), bit-exact on sampled rows."""
    rows_n, cols = 32771, 33000
    cfg = config()
    xb = f32_normal((P_A, cols), 7031)
    yb = f32_normal((P_Y, cols), 7032)
    X = repeated(xb, rows_n, torch.float32)
    Y = repeated(yb, rows_n, torch.float32)
    rows = sample_rows(rows_n, cols * 4, 7033)
    assert rows.max() * cols * 4 > (1 << 32)
    want = add_f32(xb[rows % P_A], yb[rows % P_Y]).view(np.uint32)
    for sched, tile in [("work_stealing", (128, 128)), ("blocked", (32, 16)),
                        ("interleaved", (64, 64))]:
        C = BigOut(rows_n * cols, wide=True)
        note(f"padd_run {rows_n}x{cols} sched={sched} tile={tile}")
        pg.padd_run(cfg, X, Y, C.body.view(torch.float32), rows_n, cols, tile[0], tile[1], sched)
        sync()
        assert C.guards_intact(), sched
        got = C.rows(rows, cols).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, want), (sched, tile)
        del C
    del X, Y
    torch.cuda.empty_cache()
