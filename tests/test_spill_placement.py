"""CPU check of the built forward kernels: no register spill traffic in a
steady-state loop.

The persistent attention variants (8 waves, head dimension 128) hold state
across their item loop, and the register file is nearly full: the compiler
spills a few values in an item's last iteration.  That is cheap only where
it runs once per item; a scratch store or reload inside the key loop would
run once per key tile.  This test disassembles the library's own gfx950
code (built here from source), finds each function's loops from its
backward branches, and checks that no scratch instruction sits inside an
innermost loop of any attn_fwd_main variant.  A planted listing checks the
checker.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bf16_attention_forward_amd", "libattn_fwd.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

FUNC = re.compile(r"^([0-9a-f]+) <(\S+)>:$")
INSN = re.compile(r"^\s+([a-z_0-9]+)\b(.*?)\s*//\s*([0-9A-F]+):(.*)$")
TARGET = re.compile(r"<(\S+)\+0x([0-9a-f]+)>")


def functions(tmp_path, key):
    """{name: [(address, opcode, branch target or None)]} for functions whose name holds key."""
    lib = tmp_path / "lib.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], check=True, capture_output=True, timeout=300)
    funcs = {}
    for b in sorted(p for p in os.listdir(tmp_path) if p.endswith("gfx950")):
        out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(tmp_path / b)], check=True,
                             capture_output=True, text=True, timeout=300).stdout
        name, base = None, 0
        for line in out.splitlines():
            f = FUNC.match(line)
            if f:
                name, base = f.group(2), int(f.group(1), 16)
                if key in name:
                    funcs[name] = []
                continue
            m = INSN.match(line)
            if m and name in funcs:
                tgt = None
                if m.group(1).startswith(("s_cbranch", "s_branch")):
                    t = TARGET.search(m.group(4))
                    if t and t.group(1) == name:
                        tgt = base + int(t.group(2), 16)
                funcs[name].append((int(m.group(3), 16), m.group(1), tgt))
    return funcs


def innermost_loops(insns):
    """Address ranges [head, back-branch] of loops that contain no other loop."""
    loops = sorted({(tgt, addr) for addr, op, tgt in insns if tgt is not None and tgt <= addr})
    return [(h, e) for h, e in loops
            if not any((h2, e2) != (h, e) and h <= h2 and e2 <= e for h2, e2 in loops)]


def spills_in_loops(insns):
    loops = innermost_loops(insns)
    return [(addr, op) for addr, op, _ in insns
            if op.startswith("scratch_") and any(h <= addr <= e for h, e in loops)]


def test_checker_flags_a_spill_inside_a_loop():
    planted = [(0, "s_mov_b32", None), (4, "scratch_store_dword", None),      # before the loop: allowed
               (8, "v_mfma_f32_16x16x32_bf16", None), (12, "scratch_load_dword", None),
               (16, "s_cbranch_scc1", 8), (20, "s_endpgm", None)]
    assert innermost_loops(planted) == [(8, 16)]
    assert spills_in_loops(planted) == [(12, "scratch_load_dword")]
    nested = [(0, "v_add_f32", None), (4, "scratch_load_dword", None), (8, "v_mfma_f32_16x16x32_bf16", None),
              (12, "s_cbranch_scc1", 8), (16, "s_cbranch_scc1", 0)]
    assert innermost_loops(nested) == [(8, 12)]                              # the outer loop may spill
    assert spills_in_loops(nested) == []


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(OBJDUMP),
                    reason="library not built or llvm-objdump absent")
def test_no_spill_in_the_forward_key_loops(tmp_path):
    funcs = functions(tmp_path, "attn_fwd_main")
    assert funcs, "no attn_fwd_main in the library"
    for name, insns in funcs.items():
        assert innermost_loops(insns), name                                   # every variant has its key loop
        assert spills_in_loops(insns) == [], name

