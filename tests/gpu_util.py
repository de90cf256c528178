"""Helpers for the GPU parity tests: device copies of the seeded inputs,
guard-banded outputs and the elementwise tolerance checks.  Imported only by
tests marked gpu."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import tile_scheduling_persistent_amd as pg

BF16_TOL = 1e-3     # |C - C_ref| <= 1e-3 * (|A|.|B|)_ij  (bf16 operands)
FP8_TOL = 2e-2      # |C - C_ref| <= 2e-2 * (|A|.|B|)_ij  (block-scaled e4m3 operands)
GUARD = 4096        # elements of guard band on each side of an output
SENTINEL_U16 = 0x7FC1
SENTINEL_F32 = 0x7FC00001

# Host-side deadline on every wait for GPU work in the tests: a launch that
# never finishes fails its test with the name of the call instead of blocking
# until an outer time limit kills the run.
SYNC_DEADLINE_S = 90.0

_CFG = None
_LAST = "(no call noted yet)"


class GpuDeadline(AssertionError):
    """GPU work did not finish within the tests' deadline."""


def note(msg: str) -> None:
    global _LAST
    _LAST = msg
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def sync(what: str | None = None, timeout_s: float = SYNC_DEADLINE_S, stream=None) -> None:
    """Wait for the work queued so far on `stream` (default: the current
    stream), polling an event against a deadline; raise GpuDeadline naming
    `what` (default: the last noted call) if it does not complete in time.
    Then synchronise the device (every other stream)."""
    ev = torch.cuda.Event()
    ev.record(stream if stream is not None else torch.cuda.current_stream())
    t0 = time.monotonic()
    while not ev.query():
        if time.monotonic() - t0 > timeout_s:
            raise GpuDeadline(f"GPU work not finished after {timeout_s:.0f} s: {what or _LAST}")
        time.sleep(0.0005)
    torch.cuda.synchronize()


def config() -> pg.Config:
    global _CFG
    if _CFG is None:
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU visible to torch")
        _CFG = pg.Config(0)
    return _CFG


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda:0").view(torch.bfloat16)


def dev_u8(q: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q)).to("cuda:0")


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


class Guarded:
    """Output buffer of n elements with guard bands of sentinel bits around it."""

    def __init__(self, n: int, kind: str):
        self.n = n
        self.kind = kind
        if kind == "bf16":
            self.full = torch.full((n + 2 * GUARD,), SENTINEL_U16, dtype=torch.int16, device="cuda:0")
            self.view = self.full[GUARD:GUARD + n].view(torch.bfloat16)
        else:
            self.full = torch.full((n + 2 * GUARD,), SENTINEL_F32, dtype=torch.int32, device="cuda:0")
            self.view = self.full[GUARD:GUARD + n].view(torch.float32)

    def guards_intact(self) -> bool:
        h = self.full.cpu().numpy()
        s = SENTINEL_U16 if self.kind == "bf16" else SENTINEL_F32
        return bool(np.all(h[:GUARD] == s) and np.all(h[GUARD + self.n:] == s))

    def body_bits(self) -> np.ndarray:
        return self.full[GUARD:GUARD + self.n].cpu().numpy()

    def as_f64(self) -> np.ndarray:
        return self.view.float().cpu().numpy().astype(np.float64)


def assert_within(C: np.ndarray, Cref: np.ndarray, Abs: np.ndarray, tol: float,
                  out_bf16: bool, what: str = "") -> None:
    """|C - Cref| <= tol * Abs elementwise; for a bf16 result the final rounding
    of the stored value (one bf16 ulp at |Cref|) is allowed on top."""
    C = np.asarray(C, np.float64)
    err = np.abs(C - Cref)
    bound = tol * Abs
    if out_bf16:
        e = np.floor(np.log2(np.maximum(np.abs(Cref), 1e-300)))
        bound = bound + np.where(Cref != 0, np.exp2(e - 7), 0.0)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = [(tuple(i), C[tuple(i)], Cref[tuple(i)], Abs[tuple(i)]) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside tolerance, e.g. {rows}")


def assert_abs_bound(C: np.ndarray, Cref: np.ndarray, Abs: np.ndarray, tol: float,
                      what: str = "") -> None:
    """The plain bound |C - Cref| <= tol * Abs, final rounding included."""
    err = np.abs(np.asarray(C, np.float64) - Cref)
    bad = ~(err <= tol * Abs)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside {tol}*|A||B|, e.g. "
                             f"{[(tuple(i), C[tuple(i)], Cref[tuple(i)], Abs[tuple(i)]) for i in idx]}")
