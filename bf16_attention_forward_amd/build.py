"""Build the gfx950 HIP library (libattn_fwd.so) in-tree with hipcc.

Usage: python -m bf16_attention_forward_amd.build            (or build() from Python)
       python -m bf16_attention_forward_amd.build --table    (build, then print a
                                                               per-kernel resource table)
The compiler's raw resource-usage remarks (VGPR/AGPR/SGPR counts, LDS,
scratch, occupancy per kernel) are written to _build/ at the repository root,
a build folder kept out of version control; resource_table() condenses them
into one markdown row per kernel.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_fwd.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
REPORT = os.path.join(BUILD_DIR, "libattn_fwd.resource-usage.txt")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_fwd_kernel.hip", "attn_bwd_kernel.hip", "attn_gather_kernel.hip", "attn_api.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ALU ops are kept off: hipcc must not emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # built-in MFMAs keep their results in VGPRs: the backward's dK/dV kernel
    # binds its accumulators to AGPRs itself (inline assembly), and its S and
    # dP feed VALU work; without the option the compiler moves every MFMA of
    # that kernel to the AGPR form and copies S and dP back (the other kernels
    # compile to the same code either way)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Rpass-analysis=kernel-resource-usage",
]


def build(extra_flags=None, out=None, quiet=True) -> str:
    out = out or LIB
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libattn_fwd.so")
    os.replace(out + ".tmp", out)
    lines = [ln for ln in res.stderr.splitlines() if "remark:" in ln]
    report = REPORT if out == LIB else out + ".resource-usage.txt"
    os.makedirs(os.path.dirname(report), exist_ok=True)
    with open(report, "w") as f:
        f.write("\n".join(lines) + "\n")
    if not quiet:
        print("\n".join(lines))
    return out


FIELDS = (("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"), ("SGPRs Spill", "SGPR spill"),
          ("VGPRs Spill", "VGPR spill"),
          ("ScratchSize [bytes/lane]", "scratch B/lane"), ("LDS Size [bytes/block]", "LDS B/block"),
          ("Occupancy [waves/SIMD]", "waves/SIMD"))


def _demangle(names):
    tool = shutil.which("llvm-cxxfilt") or "/opt/rocm/llvm/bin/llvm-cxxfilt"
    if not os.path.exists(tool):
        tool = shutil.which("c++filt")
    if not tool:
        return names
    res = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
    out = res.stdout.splitlines()
    return out if len(out) == len(names) else names


def resource_table(report: str = REPORT) -> str:
    """One markdown row per kernel from the compiler's resource-usage remarks."""
    kernels, cur = [], None
    pat = re.compile(r"remark:\s+(.*?):\s+(\S+)\s+\[-Rpass")
    for ln in open(report):
        m = pat.search(ln)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = {"name": val}
            kernels.append(cur)
        elif cur is not None:
            cur[key] = val
    names = _demangle([k["name"] for k in kernels])
    head = "| kernel | " + " | ".join(h for _, h in FIELDS) + " |"
    rows = [head, "|" + "---|" * (len(FIELDS) + 1)]
    for k, nm in sorted(zip(kernels, names), key=lambda kn: kn[1]):
        nm = nm.replace("attn::", "").replace("attn_bwd::", "").replace("(attn::AttnParams)", "")
        nm = re.sub(r"\(attn_bwd::BwdParams\)", "", nm)
        rows.append(f"| `{nm}` | " + " | ".join(k.get(f, "") for f, _ in FIELDS) + " |")
    return "\n".join(rows) + "\n"


if __name__ == "__main__":
    path = build(quiet="--table" in sys.argv)
    if "--table" in sys.argv:
        print(resource_table())
    else:
        print(path)
