"""The C-ABI library loads without a GPU and exports every entry point that
include/pgemm.h declares; host-side behaviour that needs no device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgemm.h")
LIB = os.path.join(ROOT, "tile_scheduling_persistent_amd", "libpgemm.so")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PGEMM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ["pgemm_config_create", "pgemm_config_query", "pgemm_config_destroy", "pgemm_run",
              "padd_run", "pgemm_status_str", "pgemm_witness_enable", "pgemm_witness_read"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    L = ctypes.CDLL(LIB)
    for n in declared():
        assert hasattr(L, n), n
    syms = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                          check=True).stdout
    exported = {l.split()[-1] for l in syms.splitlines() if " T " in l}
    assert set(declared()) <= exported
    # nothing but the C ABI is exported
    assert exported == set(declared()), sorted(exported - set(declared()))


def test_header_compiles_as_c():
    src = '#include "pgemm.h"\nint main(void){ pgemm_args a = {0}; (void)a; return 0; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        f"-I{os.path.dirname(HEADER)}", "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings_and_null_handling():
    import tile_scheduling_persistent_amd as pg
    from tile_scheduling_persistent_amd import _abi
    L = _abi.lib()
    assert pg.status_str(_abi.OK) == "ok"
    assert "invalid" in pg.status_str(_abi.ERR_INVALID)
    assert pg.status_str(99) == "unknown status"
    assert L.pgemm_config_destroy(None) == _abi.OK
    assert L.pgemm_config_query(None, None) == _abi.ERR_INVALID
    assert L.pgemm_run(None, None, None, None, 1, 1, 1, 0, 0, None, None) == _abi.ERR_INVALID
    assert L.padd_run(None, None, None, None, 1, 1, 32, 16, 0, None, None) == _abi.ERR_INVALID
    assert L.pgemm_config_create(0, 0, None) == _abi.ERR_INVALID


def test_binding_rejects_host_tensors():
    import torch
    import tile_scheduling_persistent_amd as pg
    with pytest.raises(ValueError):
        pg._ptr(torch.zeros(4), "A")
    with pytest.raises(TypeError):
        pg._ptr([1, 2], "A")


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU path")
def test_config_create_without_gpu_reports_error():
    import tile_scheduling_persistent_amd as pg
    with pytest.raises(pg.PgemmError):
        pg.Config(0)


def test_binding_checks_dtype_and_extent_before_any_device_call():
    """The binding refuses a tensor of the wrong element type, or one too
    short for the bytes the call would read or write, before the library is
    called (a too-short output would otherwise be written past its end)."""
    import torch
    import tile_scheduling_persistent_amd as pg
    M, N, K = 64, 48, 256
    nb = pg.gemm_bytes(M, N, K, "bf16_out_bf16")
    assert nb == {"A": M * K * 2, "B": K * N * 2, "C": M * N * 2}
    assert pg.gemm_bytes(M, N, K, "bf16_out_f32")["C"] == M * N * 4
    f8 = pg.gemm_bytes(M, N, K, "fp8_b128_out_bf16")
    assert (f8["A"], f8["B"], f8["a_scale"], f8["b_scale"]) == (M * K, K * N, 2 * M, 2 * N)
    ok = torch.empty(M * K, dtype=torch.bfloat16)
    pg._check_tensor(ok, "A", ("bfloat16",), nb["A"])
    with pytest.raises(ValueError, match="bytes"):
        pg._check_tensor(torch.empty(M * K - 1, dtype=torch.bfloat16), "A", ("bfloat16",), nb["A"])
    with pytest.raises(ValueError, match="dtype"):
        pg._check_tensor(torch.empty(M * K, dtype=torch.float16), "A", ("bfloat16",), nb["A"])
    with pytest.raises(ValueError, match="contiguous"):
        pg._check_tensor(torch.empty(K, M, dtype=torch.bfloat16).t(), "A", ("bfloat16",), nb["A"])
    # an fp32 C is twice a bf16 C: a bf16 buffer of M*N elements is too short for it
    with pytest.raises(ValueError):
        pg._check_tensor(torch.empty(M * N, dtype=torch.bfloat16), "C", ("float32",),
                         pg.gemm_bytes(M, N, K, "bf16_out_f32")["C"])
    # the whole GEMM argument set: a short C is caught before anything is launched
    A = torch.empty(M * K, dtype=torch.bfloat16)
    B = torch.empty(K * N, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="C"):
        pg._gemm_ptrs(A, B, torch.empty(M * N - 8, dtype=torch.bfloat16), M, N, K, "bf16_out_bf16", None)
    with pytest.raises(ValueError, match="dtype"):
        pg._gemm_ptrs(A, B, torch.empty(M * N, dtype=torch.float32), M, N, K, "bf16_out_bf16", None)
    # scales given to make_args are checked against M, N, K of the call
    qa = torch.empty(M * K, dtype=torch.uint8)
    qb = torch.empty(K * N, dtype=torch.uint8)
    short = torch.empty((K // 128) * M - 1, dtype=torch.uint8)
    args = pg._abi.pgemm_args()
    args._scales = (short, torch.empty((K // 128) * N, dtype=torch.uint8))
    with pytest.raises(ValueError, match="a_scale"):
        pg._gemm_ptrs(qa, qb, torch.empty(M * N, dtype=torch.bfloat16), M, N, K, "fp8_b128_out_bf16", args)
    # host tensors that pass every other check are still refused
    with pytest.raises(ValueError, match="GPU"):
        pg._gemm_ptrs(A, B, torch.empty(M * N, dtype=torch.bfloat16), M, N, K, "bf16_out_bf16", None)
