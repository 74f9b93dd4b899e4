"""rocprofv3 helpers: a calibration copy kernel and summaries of profiler output.

  python -m bf16_attention_forward_amd.profiling copy --mib 1024 --iters 5
      Plain device-to-device copy of a known size, profiled next to the
      attention kernel so FETCH_SIZE / WRITE_SIZE can be scaled to bytes.

  python -m bf16_attention_forward_amd.profiling stats --dir D --out F --command C
      Per-kernel duration summary (from --kernel-trace --stats CSV output).

  python -m bf16_attention_forward_amd.profiling counters --dir D --out F --command C
      Per-kernel average of every collected counter (from --pmc CSV output).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys
from collections import defaultdict


def _find(d: str, suffix: str):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits


def short_name(name: str) -> str:
    if "attn_fwd_main" in name:
        return "attn_fwd_main"
    if "attn_fwd_combine" in name:
        return "attn_fwd_combine"
    if "copy" in name.lower() or "elementwise" in name.lower():
        return "copy:" + name[:60]
    return name[:80]


def kernel_stats(d: str) -> dict:
    """{kernel: {calls, avg_ns, min_ns, max_ns, total_ns}} from the kernel trace CSV."""
    rows = []
    for f in _find(d, "kernel_trace.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    per = defaultdict(list)
    for r in rows:
        per[short_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: {"calls": len(v), "avg_ns": statistics.fmean(v), "median_ns": statistics.median(v),
                "min_ns": min(v), "max_ns": max(v), "total_ns": sum(v)} for k, v in per.items()}


def counter_means(d: str) -> dict:
    """{kernel: {counter: mean per dispatch}} from the counter collection CSV."""
    per = defaultdict(lambda: defaultdict(list))
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                per[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    # several rows per dispatch when a counter is reported per dimension: sum within dispatch is
    # already done by rocprofv3 for derived counters; average over dispatches here
    return {k: {c: statistics.fmean(v) for c, v in cs.items()} for k, cs in per.items()}


def do_copy(mib: int, iters: int):
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(iters):
        torch.neg(src, out=dst)   # elementwise kernel: reads n bytes, writes n bytes
    torch.cuda.synchronize()
    print(f"copied {n} bytes x {iters}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--iters", type=int, default=5)
    for name in ("stats", "counters"):
        s = sub.add_parser(name)
        s.add_argument("--dir", required=True)
        s.add_argument("--out", required=True)
        s.add_argument("--command", required=True)
        s.add_argument("--title", default="")
    a = ap.parse_args()
    if a.cmd == "copy":
        do_copy(a.mib, a.iters)
        return
    lines = [f"# {a.title}".rstrip(), "", f"command: {a.command}", ""]
    if a.cmd == "stats":
        st = kernel_stats(a.dir)
        lines.append(f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        for k, v in sorted(st.items(), key=lambda kv: -kv[1]["total_ns"]):
            lines.append(f"{k:40s} {v['calls']:6d} {v['avg_ns'] / 1e3:10.2f} {v['median_ns'] / 1e3:10.2f} "
                         f"{v['min_ns'] / 1e3:10.2f} {v['max_ns'] / 1e3:10.2f}")
    else:
        cm = counter_means(a.dir)
        for k, cs in sorted(cm.items()):
            lines.append(f"[{k}]")
            for cn, val in sorted(cs.items()):
                lines.append(f"  {cn:40s} {val:20.3f}")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
