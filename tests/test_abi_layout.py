"""The ctypes mirrors of the C ABI's structs (tile_scheduling_persistent_amd/
_abi.py) against the header itself: a small C program built with gcc from
include/pgemm.h prints every field's offset and every struct's size, which
must equal what ctypes computes.  Catches a field added, dropped, reordered
or retyped on one side only."""
import ctypes
import os
import subprocess

import pytest

from tile_scheduling_persistent_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = ["pgemm_args", "pgemm_info", "pgemm_witness", "pgemm_plan", "padd_problem", "pgemm_problem"]


@pytest.fixture(scope="module")
def c_layout(tmp_path_factory):
    d = tmp_path_factory.mktemp("abi")
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "pgemm.h"', "int main(void) {"]
    for name in STRUCTS:
        lines.append(f'  printf("{name} sizeof %zu\\n", sizeof({name}));')
        for field, _ in getattr(_abi, name)._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["  return 0;", "}"]
    src, exe = d / "layout.c", d / "layout"
    src.write_text("\n".join(lines) + "\n")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return {(a, b): int(c) for a, b, c in (line.split() for line in out.strip().splitlines())}


@pytest.mark.parametrize("name", STRUCTS)
def test_struct_layout_matches_header(c_layout, name):
    st = getattr(_abi, name)
    assert c_layout[(name, "sizeof")] == ctypes.sizeof(st), name
    for field, _ in st._fields_:
        assert c_layout[(name, field)] == getattr(st, field).offset, (name, field)


def test_every_header_struct_is_mirrored():
    """Each struct typedef of the header has a ctypes mirror (the opaque
    config aside), so no struct can be left out of the layout check."""
    import re
    text = open(os.path.join(ROOT, "include", "pgemm.h")).read()
    names = set(re.findall(r"^\}\s*(\w+);", text, re.M)) - {"pgemm_status", "pgemm_dtype", "pgemm_sched",
                                                            "pgemm_kernel"}
    assert names == set(STRUCTS)
