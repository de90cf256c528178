"""Persistent tiled GEMM and persistent 2-D add with tile schedulers, for
AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of libpgemm.so (include/pgemm.h): the
functions keep the C names, marshal torch device tensors (or raw device
pointers) and the current HIP stream, and raise PgemmError on a non-zero
status.  Every step of the hot path runs in the library's HIP kernels;
PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _abi
from ._abi import PgemmError, status_str  # noqa: F401

SCHEDULERS = {
    "blocked": _abi.SCHED_BLOCKED,
    "interleaved": _abi.SCHED_INTERLEAVED,
    "grouped": _abi.SCHED_GROUPED,
    "work_stealing": _abi.SCHED_WORK_STEALING,
    "blocked_grouped": _abi.SCHED_BLOCKED_GROUPED,
    "stream_k": _abi.SCHED_STREAM_K,
    "work_stealing_xcc": _abi.SCHED_WORK_STEALING_XCC,
}
DTYPES = {
    "bf16_out_f32": _abi.BF16_OUT_F32,
    "bf16_out_bf16": _abi.BF16_OUT_BF16,
    "fp8_b128_out_bf16": _abi.FP8E4M3_B128_OUT_BF16,
}

__all__ = ["Config", "pgemm_run", "pgemm_run_noalloc", "pgemm_run_grouped", "padd_run", "padd_run_multi", "plan_gemm", "plan_add", "SCHEDULERS",
           "DTYPES", "PgemmError", "status_str", "make_args"]


def _check(where, code):
    if code != _abi.OK:
        raise PgemmError(where, code)


_DTYPES_OF = {}


def _torch_dtypes(names):
    t = _DTYPES_OF.get(names)
    if t is None:
        import torch
        t = _DTYPES_OF[names] = tuple(getattr(torch, n) for n in names if hasattr(torch, n))
    return t


# Element types the calls accept: operands per pgemm_dtype, outputs, adds.
_OPERAND = {_abi.BF16_OUT_F32: ("bfloat16",), _abi.BF16_OUT_BF16: ("bfloat16",),
            _abi.FP8E4M3_B128_OUT_BF16: ("uint8", "float8_e4m3fn")}
_OUTPUT = {_abi.BF16_OUT_F32: ("float32",), _abi.BF16_OUT_BF16: ("bfloat16",),
           _abi.FP8E4M3_B128_OUT_BF16: ("bfloat16",)}
_SCALE = ("uint8",)
_F32 = ("float32",)


def gemm_bytes(M: int, N: int, K: int, dtype) -> dict:
    """Bytes each buffer of a GEMM call spans: A [M][K], B [K][N], C [M][N]
    and (block-scaled fp8) the scales [K/128][M] and [K/128][N]."""
    d = _dtype(dtype)
    esz = 1 if d == _abi.FP8E4M3_B128_OUT_BF16 else 2
    csz = 4 if d == _abi.BF16_OUT_F32 else 2
    out = {"A": M * K * esz, "B": K * N * esz, "C": M * N * csz}
    if d == _abi.FP8E4M3_B128_OUT_BF16:
        out["a_scale"] = (K // 128) * M
        out["b_scale"] = (K // 128) * N
    return out


def _check_tensor(x, what, dtypes=None, nbytes=None):
    """Layout, element type and extent of a tensor argument (host-side checks,
    before any device is involved).  Raw int pointers pass unchecked: the
    library itself checks that every range lies inside one device allocation."""
    if isinstance(x, int):
        return
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor or an int device pointer")
    if not x.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous (row-major)")
    if dtypes is not None and nbytes != 0:  # an empty buffer is never accessed
        allowed = _torch_dtypes(dtypes)
        if x.dtype not in allowed:
            raise ValueError(f"{what}: dtype {x.dtype} not in {allowed}")
    if nbytes is not None and x.numel() * x.element_size() < nbytes:
        raise ValueError(f"{what}: tensor holds {x.numel() * x.element_size()} bytes, "
                         f"the call reads or writes {nbytes}")


def _dev(x, what):
    """Device pointer of a checked tensor argument (or a raw int pointer)."""
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{what}: tensor must live on the GPU")
    return x.data_ptr()


def _ptr(x, what, dtypes=None, nbytes=None):
    """Device pointer of a torch tensor (contiguous, on a GPU, of an allowed
    dtype, at least nbytes long) or a raw int pointer."""
    _check_tensor(x, what, dtypes, nbytes)
    return _dev(x, what)


def _stream(stream, device=None):
    """Raw HIP stream handle: `stream` itself (an int or a torch stream), else
    torch's current stream on `device` (the config's device)."""
    if stream is None:
        import torch
        if device is not None:
            return torch._C._cuda_getCurrentRawStream(device)
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _sched(s):
    return SCHEDULERS[s] if isinstance(s, str) else int(s)


def _dtype(d):
    return DTYPES[d] if isinstance(d, str) else int(d)


ORDERS = {"default": _abi.ORDER_DEFAULT, "dispatch": _abi.ORDER_DISPATCH, "xcd_major": _abi.ORDER_XCD_MAJOR}
PIPELINES = {"default": _abi.PIPELINE_DEFAULT, "four_wave": _abi.PIPELINE_FOUR_WAVE,
             "pingpong": _abi.PIPELINE_PINGPONG}


def make_args(tile=None, group_size=0, grid=0, claim_chunk=0, a_scale=None, b_scale=None,
              debug_flags=0, straggler_program=-1, straggler_ns=0, pipeline="default",
              program_order="default"):
    a = _abi.pgemm_args()
    if tile is not None:
        a.tile_m, a.tile_n, a.tile_k = (tuple(tile) + (0,))[:3]
    a.group_size = group_size
    a.grid = grid
    a.claim_chunk = claim_chunk
    a.a_scale = _ptr(a_scale, "a_scale", _SCALE) if a_scale is not None else None
    a.b_scale = _ptr(b_scale, "b_scale", _SCALE) if b_scale is not None else None
    a._scales = (a_scale, b_scale)  # checked against M, N, K when the call is made
    a.debug_flags = debug_flags
    a.straggler_program = straggler_program
    a.straggler_ns = straggler_ns
    a.pipeline = PIPELINES[pipeline] if isinstance(pipeline, str) else int(pipeline)
    a.program_order = ORDERS[program_order] if isinstance(program_order, str) else int(program_order)
    return a


class Config:
    """pgemm_config: device facts plus the reusable per-XCD counters."""

    def __init__(self, device: int = 0, max_xcds: int = 0):
        h = ctypes.c_void_p()
        _check("pgemm_config_create", _abi.lib().pgemm_config_create(int(device), int(max_xcds),
                                                                      ctypes.byref(h)))
        self.handle = h
        self.device = int(device)
        info = _abi.pgemm_info()
        _check("pgemm_config_query", _abi.lib().pgemm_config_query(h, ctypes.byref(info)))
        self.info = {
            "num_cus": info.num_cus, "num_xcds": info.num_xcds,
            "counter_capacity": info.counter_capacity, "wall_clock_khz": info.wall_clock_khz,
            "clock_khz": info.clock_khz, "lds_bytes_per_cu": info.lds_bytes_per_cu,
            "arch": info.arch.decode(),
        }

    def close(self):
        if self.handle is not None:
            _abi.lib().pgemm_config_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def witness_enable(self, max_tiles: int, max_programs: int):
        _check("pgemm_witness_enable",
               _abi.lib().pgemm_witness_enable(self.handle, int(max_tiles), int(max_programs)))

    def witness_read(self, tiles: int, programs: int, stream=None):
        out = {
            "visits": np.zeros(tiles, np.int32), "owner": np.zeros(tiles, np.int32),
            "order": np.zeros(tiles, np.int32), "t_start": np.zeros(programs, np.int64),
            "t_end": np.zeros(programs, np.int64), "hw_id": np.zeros(programs, np.int32),
            "n_tiles": np.zeros(programs, np.int32),
            "counters": np.zeros(self.info["counter_capacity"], np.int32),
            "cycles": np.zeros(programs, np.int64),
            "claims": np.zeros((programs, _abi.MAX_STEAL_COUNTERS), np.int32),
        }
        w = _abi.pgemm_witness()
        for k in ("visits", "owner", "order", "t_start", "t_end", "hw_id", "n_tiles", "counters",
                  "cycles", "claims"):
            setattr(w, k, out[k].ctypes.data)
        w.tiles = tiles
        w.programs = programs
        _check("pgemm_witness_read",
               _abi.lib().pgemm_witness_read(self.handle, ctypes.byref(w), _stream(stream, self.device)))
        return out


def pgemm_run(cfg: Config, A, B, C, M: int, N: int, K: int, dtype, sched, args=None,
              stream=None):
    """C[M][N] = A[M][K] . B[K][N] on the GPU (asynchronous on `stream`)."""
    code = _abi.lib().pgemm_run(cfg.handle, *_gemm_ptrs(A, B, C, M, N, K, dtype, args),
                                int(M), int(N), int(K), _dtype(dtype), _sched(sched),
                                ctypes.byref(args) if args is not None else None, _stream(stream, cfg.device))
    _check("pgemm_run", code)


def pgemm_run_noalloc(cfg: Config, A, B, C, M: int, N: int, K: int, dtype, sched, args=None,
                      stream=None):
    """pgemm_run without any device allocation: the work-stealing counters and
    the stream-K partial sums come from the library's static per-device
    scratch (calls on one GPU must not overlap)."""
    code = _abi.lib().pgemm_run_noalloc(cfg.handle, *_gemm_ptrs(A, B, C, M, N, K, dtype, args),
                                        int(M), int(N), int(K), _dtype(dtype), _sched(sched),
                                        ctypes.byref(args) if args is not None else None,
                                        _stream(stream, cfg.device))
    _check("pgemm_run_noalloc", code)


def _gemm_ptrs(A, B, C, M, N, K, dtype, args, where=""):
    """Device pointers of a GEMM's A, B, C after every host-side check of
    all its buffers (element types, extents, the scales passed in args)."""
    d = _dtype(dtype)
    nb = gemm_bytes(int(M), int(N), int(K), d) if d in _OPERAND else {}
    if args is not None and "a_scale" in nb:
        for name, t in zip(("a_scale", "b_scale"), getattr(args, "_scales", (None, None))):
            if t is not None:
                _check_tensor(t, name + where, _SCALE, nb[name])
    ops, outs = _OPERAND.get(d), _OUTPUT.get(d)
    _check_tensor(A, "A" + where, ops, nb.get("A"))
    _check_tensor(B, "B" + where, ops, nb.get("B"))
    _check_tensor(C, "C" + where, outs, nb.get("C"))
    return _dev(A, "A" + where), _dev(B, "B" + where), _dev(C, "C" + where)


def _plan_dict(pl) -> dict:
    return {"grid": pl.grid, "occupancy": pl.occupancy, "tiles": pl.tiles,
            "tile": (pl.tile_m, pl.tile_n, pl.tile_k), "threads": pl.threads,
            "lds_bytes": pl.lds_bytes, "kernel": _abi.KERNEL_NAMES.get(pl.kernel, str(pl.kernel)),
            "xcd_major": bool(pl.xcd_major)}


def plan_gemm(cfg: Config, M: int, N: int, K: int, dtype, sched, args=None, A=None, B=None,
              C=None) -> dict:
    """The launch pgemm_run would make (grid, occupancy, tiles, kernel, ...)."""
    pl = _abi.pgemm_plan()
    code = _abi.lib().pgemm_plan_gemm(
        cfg.handle, A.data_ptr() if A is not None else None, B.data_ptr() if B is not None else None,
        C.data_ptr() if C is not None else None, int(M), int(N), int(K), _dtype(dtype),
        _sched(sched), ctypes.byref(args) if args is not None else None, ctypes.byref(pl))
    _check("pgemm_plan_gemm", code)
    return _plan_dict(pl)


def plan_add(cfg: Config, rows: int, cols: int, tile_rows: int, tile_cols: int, sched, args=None,
             X=None, Y=None, C=None) -> dict:
    """The launch padd_run would make."""
    pl = _abi.pgemm_plan()
    code = _abi.lib().pgemm_plan_add(
        cfg.handle, X.data_ptr() if X is not None else None, Y.data_ptr() if Y is not None else None,
        C.data_ptr() if C is not None else None, int(rows), int(cols), int(tile_rows),
        int(tile_cols), _sched(sched), ctypes.byref(args) if args is not None else None,
        ctypes.byref(pl))
    _check("pgemm_plan_add", code)
    return _plan_dict(pl)


def padd_run(cfg: Config, X, Y, C, rows: int, cols: int, tile_rows: int, tile_cols: int, sched,
             args=None, stream=None):
    """C = X + Y (fp32) over tile_rows x tile_cols tiles (asynchronous on `stream`)."""
    nb = int(rows) * int(cols) * 4
    code = _abi.lib().padd_run(cfg.handle, _ptr(X, "X", _F32, nb), _ptr(Y, "Y", _F32, nb),
                               _ptr(C, "C", _F32, nb),
                               int(rows), int(cols), int(tile_rows), int(tile_cols), _sched(sched),
                               ctypes.byref(args) if args is not None else None, _stream(stream, cfg.device))
    _check("padd_run", code)


def padd_run_multi(cfg: Config, problems, tile_rows: int, tile_cols: int, sched, args=None,
                   stream=None):
    """Several adds C_g = X_g + Y_g (fp32) in one persistent launch; `problems`
    is a sequence of (X, Y, C, rows, cols)."""
    n = len(problems)
    arr = (_abi.padd_problem * max(n, 1))()
    for g, (X, Y, C, rows, cols) in enumerate(problems):
        nb = int(rows) * int(cols) * 4
        arr[g].X = _ptr(X, f"X[{g}]", _F32, nb)
        arr[g].Y = _ptr(Y, f"Y[{g}]", _F32, nb)
        arr[g].C = _ptr(C, f"C[{g}]", _F32, nb)
        arr[g].rows = int(rows)
        arr[g].cols = int(cols)
    code = _abi.lib().padd_run_multi(cfg.handle, arr, n, int(tile_rows), int(tile_cols), _sched(sched),
                                     ctypes.byref(args) if args is not None else None, _stream(stream, cfg.device))
    _check("padd_run_multi", code)


def pgemm_run_grouped(cfg: Config, problems, dtype, sched, args=None, stream=None):
    """Several GEMMs C_g = A_g . B_g in one persistent launch; `problems` is a
    sequence of (A, B, C, M, N, K), or (A, B, C, M, N, K, a_scale, b_scale)
    for block-scaled fp8."""
    n = len(problems)
    arr = (_abi.pgemm_problem * max(n, 1))()
    for g, pr in enumerate(problems):
        A, B, C, M, N, K = pr[:6]
        arr[g].A, arr[g].B, arr[g].C = _gemm_ptrs(A, B, C, M, N, K, dtype, None, f"[{g}]")
        arr[g].M, arr[g].N, arr[g].K = int(M), int(N), int(K)
        if len(pr) == 8:
            nb = gemm_bytes(int(M), int(N), int(K), "fp8_b128_out_bf16")
            arr[g].a_scale = _ptr(pr[6], f"a_scale[{g}]", _SCALE, nb["a_scale"])
            arr[g].b_scale = _ptr(pr[7], f"b_scale[{g}]", _SCALE, nb["b_scale"])
    code = _abi.lib().pgemm_run_grouped(cfg.handle, arr, n, _dtype(dtype), _sched(sched),
                                        ctypes.byref(args) if args is not None else None,
                                        _stream(stream, cfg.device))
    _check("pgemm_run_grouped", code)

