"""CPU check of the built library's gfx950 code: every write of m0 (the LDS
destination of a buffer_load ... lds) is followed by exactly one s_nop and
then its load, and nothing else reads or writes m0.

The K/V and Q/dO tiles reach LDS through inline-asm buffer loads that write
m0 and load in one statement.  m0 is a register the compiler reserves and
does not track across asm statements, so that form is safe only while no
other instruction of the kernels uses m0.  An LDS-bound buffer load also
needs one wait state after a scalar write of m0 before it reads it; the
compiler's hazard recognizer does not look into inline assembly, so the
statement carries its own s_nop (the compiler emits the same nop after its
m0 write for the builtin form of the load).  This test disassembles the
library's own code objects (built here from source) and checks both.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bf16_attention_forward_amd", "libattn_fwd.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

INSN = re.compile(r"^\s+([a-z_0-9]+)\b([^/]*)")


def gfx950_listings(tmp_path):
    lib = tmp_path / "lib.so"
    shutil.copy(LIB, lib)
    # --offloading writes each bundle next to its input, i.e. into tmp_path
    subprocess.run([OBJDUMP, "--offloading", str(lib)], check=True, capture_output=True, timeout=300)
    bundles = sorted(p for p in os.listdir(tmp_path) if p.endswith("gfx950"))
    assert bundles, "no gfx950 code object in the library"
    for b in bundles:
        out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(tmp_path / b)], check=True,
                             capture_output=True, text=True, timeout=300).stdout
        insns = []
        for line in out.splitlines():
            m = INSN.match(line)
            if m:
                insns.append((m.group(1), m.group(2).strip()))
        yield b, insns


def is_lds_load(op, args):
    return op.startswith("buffer_load_dword") and re.search(r"\blds\b", args) is not None


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(OBJDUMP),
                    reason="library not built or llvm-objdump absent")
def test_m0_write_is_followed_by_a_wait_state_then_its_lds_load(tmp_path):
    n_loads = 0
    for name, insns in gfx950_listings(tmp_path):
        for i, (op, args) in enumerate(insns):
            uses_m0 = re.search(r"\bm0\b", args) is not None
            if is_lds_load(op, args):
                n_loads += 1
                assert i > 1 and insns[i - 1][0] == "s_nop", (name, i, insns[i - 1], op, args)
                assert insns[i - 2][0] == "s_mov_b32" and insns[i - 2][1].startswith("m0,"), \
                    (name, i, insns[i - 2], op, args)
            if uses_m0:
                assert op == "s_mov_b32" and args.startswith("m0,"), (name, i, op, args)
                assert insns[i + 1][0] == "s_nop", (name, i, insns[i + 1])
                assert is_lds_load(*insns[i + 2]), (name, i, insns[i + 2])
    assert n_loads > 0
