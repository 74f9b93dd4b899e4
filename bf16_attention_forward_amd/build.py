"""Build the gfx950 HIP library (libattn_fwd.so) in-tree with hipcc.

Usage: python -m bf16_attention_forward_amd.build   (or build() from Python)
The resource-usage report of the kernels (VGPR/AGPR/SGPR counts, LDS,
scratch, occupancy) is written next to the library as
libattn_fwd.resource-usage.txt.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_fwd.so")
REPORT = os.path.join(HERE, "libattn_fwd.resource-usage.txt")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_fwd_kernel.hip", "attn_bwd_kernel.hip", "attn_api.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ALU ops are kept off: hipcc must not emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
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
    with open(REPORT if out == LIB else out + ".resource-usage.txt", "w") as f:
        f.write("\n".join(lines) + "\n")
    if not quiet:
        print("\n".join(lines))
    return out


if __name__ == "__main__":
    print(build(quiet=False))
