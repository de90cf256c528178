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
