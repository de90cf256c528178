"""ctypes declarations of the C ABI in include/pgemm.h (argument marshalling only).

The library is loaded from this package directory; there is no fallback: if
libpgemm.so is missing, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpgemm.so")

# pgemm_status
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_DEVICE, ERR_OOM, ERR_LAUNCH = range(6)
# pgemm_dtype
BF16_OUT_F32, BF16_OUT_BF16, FP8E4M3_B128_OUT_BF16 = range(3)
# pgemm_sched
(SCHED_BLOCKED, SCHED_INTERLEAVED, SCHED_GROUPED, SCHED_WORK_STEALING, SCHED_BLOCKED_GROUPED,
 SCHED_STREAM_K, SCHED_WORK_STEALING_XCC) = range(7)
# debug flags
DEBUG_WITNESS, DEBUG_SKIP_RESET, DEBUG_STRAGGLER, DEBUG_REGISTER_STAGED = 0x1, 0x2, 0x4, 0x8
DEBUG_STRAGGLER_XCC = 0x10
DEBUG_VALIDATE_ONLY = 0x20
# pgemm_args.claim_chunk value for paired claims
CLAIM_PAIRS = -1
# pgemm_kernel
KERNEL_BF16_LDS, KERNEL_BF16_STAGED, KERNEL_FP8, KERNEL_ADD, KERNEL_BF16_PINGPONG = range(5)
KERNEL_NAMES = {KERNEL_BF16_LDS: "bf16_lds", KERNEL_BF16_STAGED: "bf16_staged", KERNEL_FP8: "fp8",
                KERNEL_ADD: "add", KERNEL_BF16_PINGPONG: "bf16_pingpong"}
# pgemm_args.pipeline
PIPELINE_DEFAULT, PIPELINE_FOUR_WAVE, PIPELINE_PINGPONG = 0, 1, 2
# pgemm_args.program_order
ORDER_DEFAULT, ORDER_DISPATCH, ORDER_XCD_MAJOR = 0, 1, 2


class pgemm_args(ctypes.Structure):
    _fields_ = [
        ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
        ("group_size", ctypes.c_int), ("grid", ctypes.c_int), ("claim_chunk", ctypes.c_int),
        ("a_scale", ctypes.c_void_p), ("b_scale", ctypes.c_void_p),
        ("debug_flags", ctypes.c_uint),
        ("straggler_program", ctypes.c_int), ("straggler_ns", ctypes.c_int),
        ("pipeline", ctypes.c_int), ("program_order", ctypes.c_int),
    ]


class pgemm_info(ctypes.Structure):
    _fields_ = [
        ("num_cus", ctypes.c_int), ("num_xcds", ctypes.c_int), ("counter_capacity", ctypes.c_int),
        ("wall_clock_khz", ctypes.c_int), ("clock_khz", ctypes.c_int),
        ("lds_bytes_per_cu", ctypes.c_int), ("arch", ctypes.c_char * 64),
    ]


class pgemm_witness(ctypes.Structure):
    _fields_ = [
        ("visits", ctypes.c_void_p), ("owner", ctypes.c_void_p), ("order", ctypes.c_void_p),
        ("tiles", ctypes.c_int64),
        ("t_start", ctypes.c_void_p), ("t_end", ctypes.c_void_p),
        ("hw_id", ctypes.c_void_p), ("n_tiles", ctypes.c_void_p),
        ("programs", ctypes.c_int32), ("counters", ctypes.c_void_p),
        ("cycles", ctypes.c_void_p), ("claims", ctypes.c_void_p),
    ]


MAX_STEAL_COUNTERS = 8  # columns of pgemm_witness.claims


class pgemm_plan(ctypes.Structure):
    _fields_ = [
        ("grid", ctypes.c_int), ("occupancy", ctypes.c_int), ("tiles", ctypes.c_int64),
        ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
        ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int), ("kernel", ctypes.c_int),
        ("xcd_major", ctypes.c_int),
    ]


PADD_MAX_PROBLEMS = 8


class padd_problem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


PGEMM_MAX_PROBLEMS = 8
# bytes of the static device scratch pgemm_run_noalloc uses on each device
NOALLOC_SCRATCH_BYTES = (64 << 20) + 4096


class pgemm_problem(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_scale", ctypes.c_void_p), ("b_scale", ctypes.c_void_p)]


_cfg_p = ctypes.c_void_p
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m tile_scheduling_persistent_amd.build` "
            "(or __graft_entry__.build()); there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    L.pgemm_status_str.argtypes = [st]
    L.pgemm_status_str.restype = ctypes.c_char_p
    L.pgemm_config_create.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(_cfg_p)]
    L.pgemm_config_create.restype = st
    L.pgemm_config_query.argtypes = [_cfg_p, ctypes.POINTER(pgemm_info)]
    L.pgemm_config_query.restype = st
    L.pgemm_config_destroy.argtypes = [_cfg_p]
    L.pgemm_config_destroy.restype = st
    L.pgemm_run.argtypes = [_cfg_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                            ctypes.c_int, ctypes.POINTER(pgemm_args), ctypes.c_void_p]
    L.pgemm_run.restype = st
    L.pgemm_run_noalloc.argtypes = L.pgemm_run.argtypes
    L.pgemm_run_noalloc.restype = st
    L.padd_run.argtypes = [_cfg_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int, ctypes.POINTER(pgemm_args), ctypes.c_void_p]
    L.padd_run.restype = st
    L.padd_run_multi.argtypes = [_cfg_p, ctypes.POINTER(padd_problem), ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, ctypes.POINTER(pgemm_args),
                                 ctypes.c_void_p]
    L.padd_run_multi.restype = st
    L.pgemm_run_grouped.argtypes = [_cfg_p, ctypes.POINTER(pgemm_problem), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.POINTER(pgemm_args), ctypes.c_void_p]
    L.pgemm_run_grouped.restype = st
    L.pgemm_witness_enable.argtypes = [_cfg_p, ctypes.c_int64, ctypes.c_int]
    L.pgemm_witness_enable.restype = st
    L.pgemm_witness_read.argtypes = [_cfg_p, ctypes.POINTER(pgemm_witness), ctypes.c_void_p]
    L.pgemm_witness_read.restype = st
    L.pgemm_plan_gemm.argtypes = [_cfg_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_int, ctypes.POINTER(pgemm_args), ctypes.POINTER(pgemm_plan)]
    L.pgemm_plan_gemm.restype = st
    L.pgemm_plan_add.argtypes = [_cfg_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.POINTER(pgemm_args), ctypes.POINTER(pgemm_plan)]
    L.pgemm_plan_add.restype = st
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().pgemm_status_str(int(code)).decode()


class PgemmError(RuntimeError):
    def __init__(self, where: str, code: int):
        super().__init__(f"{where}: {status_str(code)} (status {code})")
        self.code = code
