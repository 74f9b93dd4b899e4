"""CPU check of the built library's gfx950 code: the dK/dV kernel's
inline-assembly products keep the distances the hardware needs.

The backward's dK/dV kernel accumulates dK and dV in AGPRs with MFMAs
written as inline assembly, which the compiler's hazard recognizer does
not look into.  The CDNA3 instruction-set manual lists the software wait
states around MFMAs: a VALU write of a VGPR (or a v_accvgpr_write of an
AGPR) needs 2 before an MFMA reads it as an operand, and a read of an MFMA
result by v_accvgpr_read needs up to 18 (16-pass products).  The kernel
keeps these distances by construction (its operands are made a phase
earlier, its accumulators are read after an explicit wait); this test
disassembles the library's own code objects and checks, in every dK/dV
kernel variant, that

  * no VALU instruction writes an operand register of an AGPR-destination
    MFMA within the 4 wait states before it (2 required),
  * no v_accvgpr_read reads an AGPR written by an MFMA within the 19 wait
    states before it (18 required),
  * no AGPR-destination MFMA is entered by a branch within those 4 wait
    states (the window would then depend on the path), and
  * no accumulator is the destination of two MFMAs fewer than 16 products
    apart.
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
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")

VALU_TO_MFMA = 4      # wait states checked (2 required)
MFMA_TO_READ = 19     # wait states checked (18 required)
MIN_ACC_DISTANCE = 16


def regs(text):
    out = set()
    for m in REG.finditer(text):
        lo = int(m.group(2) if m.group(2) is not None else m.group(4))
        hi = int(m.group(3) if m.group(3) is not None else m.group(4))
        out |= {(m.group(1), r) for r in range(lo, hi + 1)}
    return out


def dkdv_functions(tmp_path):
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
                if "attn_bwd_dkdv" in name:
                    funcs[name] = {"base": base, "insns": [], "targets": set()}
                continue
            m = INSN.match(line)
            if m and name in funcs:
                fn = funcs[name]
                fn["insns"].append((int(m.group(3), 16), m.group(1), m.group(2).strip()))
                if m.group(1).startswith(("s_cbranch", "s_branch")):
                    t = TARGET.search(m.group(4))
                    if t and t.group(1) == name:
                        fn["targets"].add(fn["base"] + int(t.group(2), 16))
    return funcs


def wait_states(op, args):
    if op == "s_nop":
        return int(args.split()[0], 0) + 1
    return 1


def split_operands(args):
    # "a[0:3], v[2:5], v[6:9], a[0:3]" -> the four operand texts
    parts, depth, cur = [], 0, ""
    for ch in args:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            parts.append(cur.strip())
            cur = ""
        else:
            cur += ch
    parts.append(cur.strip())
    return parts


def violations(name, fn):
    """The distance violations in one function's instruction list."""
    out = []
    insns = fn["insns"]
    last_acc_write = {}
    mfma_count = 0
    for i, (addr, op, args) in enumerate(insns):
        if op.startswith("v_mfma"):
            mfma_count += 1
        if op.startswith("v_mfma") and args.startswith("a"):
            ops = split_operands(args)
            dst, srcs = regs(ops[0]), set().union(*(regs(o) for o in ops[1:]))
            ws, j = 0, i - 1
            while j >= 0 and ws < VALU_TO_MFMA:
                if insns[j + 1][0] in fn["targets"]:
                    out.append((name, hex(addr), "branch target in window"))
                jop, jargs = insns[j][1], insns[j][2]
                if jop.startswith("v_") and not jop.startswith(("v_mfma", "v_cmp")):
                    if regs(split_operands(jargs)[0]) & srcs:
                        out.append((name, hex(addr), op, args, "operand written by", jop, jargs, ws))
                ws += wait_states(jop, jargs)
                j -= 1
            for r in dst:
                if r in last_acc_write and mfma_count - last_acc_write[r] < MIN_ACC_DISTANCE:
                    out.append((name, hex(addr), "accumulator reused", r))
                last_acc_write[r] = mfma_count
        if op == "v_accvgpr_read_b32":
            src = regs(split_operands(args)[1])
            ws, j = 0, i - 1
            while j >= 0 and ws < MFMA_TO_READ:
                jop, jargs = insns[j][1], insns[j][2]
                if jop.startswith("v_mfma") and regs(split_operands(jargs)[0]) & src:
                    out.append((name, hex(addr), args, "read too soon after", jop, jargs, ws))
                ws += wait_states(jop, jargs)
                j -= 1
    return out


def test_checker_finds_planted_hazards():
    """The checker on hand-written sequences: each planted hazard is found,
    the same sequence with enough distance is not."""
    def fn(lines, targets=()):
        return {"insns": [(4 * i, op, args) for i, (op, args) in enumerate(lines)], "targets": set(targets)}
    mfma = ("v_mfma_f32_16x16x32_bf16", "a[0:3], v[2:5], v[6:9], a[0:3]")
    assert violations("f", fn([("v_cvt_pk_bf16_f32", "v7, v1, v2"), mfma]))
    assert violations("f", fn([("v_accvgpr_write_b32", "a1, 0"), ("s_nop", "0"), mfma]))
    assert not violations("f", fn([("v_cvt_pk_bf16_f32", "v7, v1, v2"), ("s_nop", "3"), mfma]))
    assert not violations("f", fn([("v_cvt_pk_bf16_f32", "v17, v1, v2"), mfma]))
    assert violations("f", fn([("s_nop", "0"), mfma], targets={4}))
    assert violations("f", fn([mfma, ("s_nop", "7"), ("v_accvgpr_read_b32", "v1, a2")]))
    assert not violations("f", fn([mfma, ("s_nop", "7"), ("s_nop", "7"), ("s_nop", "7"),
                                   ("v_accvgpr_read_b32", "v1, a2")]))
    assert violations("f", fn([mfma, mfma]))


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(OBJDUMP),
                    reason="library not built or llvm-objdump absent")
def test_dkdv_inline_mfma_distances(tmp_path):
    funcs = dkdv_functions(tmp_path)
    assert len(funcs) == 4, sorted(funcs)          # head dimension 128 / 64, causal or not
    for name, fn in funcs.items():
        assert any(op.startswith("v_mfma") and a.startswith("a") for _, op, a in fn["insns"]), name
        assert violations(name, fn) == []
