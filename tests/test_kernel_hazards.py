"""Checks on the machine code of the direct-to-LDS bf16 kernel (CPU only: the
kernel is compiled to gfx950 assembly here, nothing runs on a GPU).

The kernel issues its 16x16x32 MFMAs as inline assembly so that the
accumulators stay in AGPRs; the compiler's hazard logic does not look inside
inline assembly, so the kernel's own code has to keep every register an MFMA
reads (operands and accumulator input) clear of VALU writes in the wait
states before it.  These tests read the built code and require at least
MIN_WAIT_STATES between any VALU write (v_accvgpr_write included) and an
MFMA reading that register, and no scratch traffic (no register spills) in
any instantiation of the kernel."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tile_scheduling_persistent_amd", "csrc", "gemm_bf16_lds.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL = "gemm_bf16_lds_kernel"
# VALU write -> MFMA read of that VGPR/AGPR needs 2 wait states on this
# architecture; ask for twice that.
MIN_WAIT_STATES = 4


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def functions(asm, name):
    """Instruction lists of the functions whose symbol contains `name`."""
    out = {}
    for fn in re.findall(r"^(_Z\S*" + name + r"\S*):", asm, re.M):
        i = asm.index(fn + ":")
        j = asm.index(".Lfunc_end", i)
        ins = []
        for line in asm[i:j].splitlines():
            line = line.split(";")[0].strip()
            if line and not line.startswith(".") and not line.endswith(":"):
                ins.append(line)
        out[fn] = ins
    return out


def mfma_hazards(ins, need):
    """(MFMAs seen, list of (writer, mfma, wait states)) for VALU writes that
    reach an MFMA's source registers fewer than `need` wait states before it,
    walking back through the straight-line code (s_nop N counts N + 1)."""
    found, nmf = [], 0
    for k, line in enumerate(ins):
        if not line.startswith("v_mfma"):
            continue
        nmf += 1
        ops = [o for o in re.split(r"[ ,]+", line)[1:] if o]
        srcs = set().union(*[_regs(o) for o in ops[1:4]])
        ws = 0
        for b in range(k - 1, max(-1, k - 4 * need - 8), -1):
            q = ins[b]
            if q.startswith("s_nop"):
                ws += int(q.split()[1]) + 1
            else:
                if q.startswith("v_") and not q.startswith("v_mfma") and len(q.split()) > 1:
                    if _regs(re.split(r"[ ,]+", q)[1]) & srcs:
                        found.append((q, line, ws))
                ws += 1
            if ws >= need:
                break
    return nmf, found


@pytest.fixture(scope="module")
def kernel_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               f"-I{os.path.join(ROOT, 'include')}", "-S", "--cuda-device-only", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def test_no_valu_write_close_before_an_mfma_read(kernel_asm):
    fns = functions(kernel_asm, KERNEL)
    assert len(fns) >= 16, sorted(fns)  # tiles x outputs x witness / stream-K / grouped
    total = 0
    for fn, ins in fns.items():
        nmf, found = mfma_hazards(ins, MIN_WAIT_STATES)
        total += nmf
        assert nmf > 0, fn
        assert not found, (fn, found[:3])
    assert total >= 16 * 64


def test_no_register_spills_to_scratch(kernel_asm):
    for fn, ins in functions(kernel_asm, KERNEL).items():
        assert not [q for q in ins if q.startswith("scratch_")], fn


def test_hazard_check_catches_planted_writes():
    ins = ["v_accvgpr_write_b32 a1, 0",
           "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
           "v_mov_b32 v5, 0", "s_nop 0",
           "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], a[4:7]",
           "v_mov_b32 v6, 0", "s_nop 3",
           "v_mfma_f32_16x16x32_bf16 a[8:11], v[0:3], v[4:7], a[8:11]",
           "v_mov_b32 v40, 0",
           "v_mfma_f32_16x16x32_bf16 a[12:15], v[0:3], v[4:7], a[12:15]"]
    nmf, found = mfma_hazards(ins, MIN_WAIT_STATES)
    assert nmf == 4
    assert [(w, ws) for w, _, ws in found] == [("v_accvgpr_write_b32 a1, 0", 0), ("v_mov_b32 v5, 0", 1)]
