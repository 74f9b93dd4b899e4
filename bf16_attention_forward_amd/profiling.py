"""rocprofv3 helpers: a calibration copy kernel and summaries of profiler output.

  python -m bf16_attention_forward_amd.profiling copy --mib 1024 --iters 5
      Plain device-to-device copy of a known size, profiled next to the
      attention kernel so FETCH_SIZE / WRITE_SIZE can be scaled to bytes.

  python -m bf16_attention_forward_amd.profiling stats --dir D --out F --command C
      Per-kernel duration summary (from --kernel-trace --stats CSV output).

  python -m bf16_attention_forward_amd.profiling counters --dir D --out F --command C
      Per-kernel average of every collected counter (from --pmc CSV output).

  python -m bf16_attention_forward_amd.profiling traffic --fetch D1 --write D2 \
        --copy-fetch D3 --copy-write D4 --copy-mib 1024 --workload NAME --out JSON
      HBM bytes per launch of attn_fwd_main: FETCH_SIZE and WRITE_SIZE (KiB per
      dispatch) each divided by what the same counter reads per byte of the
      calibration copy, recorded with the kernel source hash it was taken on.
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
    if "attn_gather_kv" in name:
        return "attn_gather_kv"
    for k in ("attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_delta"):
        if k in name:
            return k + ("<causal>" if "<true>" in name else "")
    if "copy" in name.lower() or "elementwise" in name.lower():
        return "copy:" + name[:60]
    return name[:80]


def kernel_stats(d: str, last: int = 0) -> dict:
    """{kernel: {calls, avg_ns, min_ns, max_ns, total_ns}} from the kernel trace CSV
    (dispatch order; with last > 0 only each kernel's last `last` dispatches)."""
    rows = []
    for f in _find(d, "kernel_trace.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = defaultdict(list)
    for r in rows:
        per[short_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if last > 0:
        per = {k: v[-last:] for k, v in per.items()}
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


# MI355X: 8 XCDs (GRBM_GUI_ACTIVE is summed over them), 256 CUs, 4 SIMDs each
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def derived_lines(cs: dict) -> list:
    """Utilisation figures from the per-dispatch means of one kernel."""
    out = []
    gui = cs.get("GRBM_GUI_ACTIVE")
    if not gui:
        return out
    cyc = gui / N_XCD
    out.append(f"  GPU cycles per dispatch (GRBM_GUI_ACTIVE / {N_XCD} XCDs) = {cyc:,.0f}")
    mb = cs.get("SQ_VALU_MFMA_BUSY_CYCLES")
    if mb:
        out.append(f"  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {N_SIMD} SIMDs) = {mb / (cyc * N_SIMD):.3f}")
        if cs.get("SQ_INSTS_MFMA"):
            out.append(f"     ({mb / cs['SQ_INSTS_MFMA']:.1f} busy cycles charged per MFMA instruction)")
    co = cs.get("SQ_VALU_MFMA_COEXEC_CYCLES")
    if co is not None:
        out.append(f"  VALU issued while MFMA busy = SQ_VALU_MFMA_COEXEC_CYCLES / (cycles x {N_SIMD}) = {co / (cyc * N_SIMD):.3f}")
    waves = cs.get("SQ_WAVES")
    if waves:
        per = [f"{n} per wave = {cs[c] / waves:,.0f}" for n, c in
               (("MFMA", "SQ_INSTS_MFMA"), ("VALU incl. MFMA", "SQ_INSTS_VALU"), ("LDS", "SQ_INSTS_LDS")) if c in cs]
        if per:
            out.append("  instructions: " + "; ".join(per))
    lds = cs.get("SQ_LDS_IDX_ACTIVE")
    if lds:
        out.append(f"  LDS busy = SQ_LDS_IDX_ACTIVE / (cycles x {N_CU} CUs) = {lds / (cyc * N_CU):.3f}")
    if "SQ_LDS_BANK_CONFLICT" in cs:
        out.append(f"  LDS bank-conflict cycles per dispatch = {cs['SQ_LDS_BANK_CONFLICT']:,.0f}")
    av = cs.get("SQ_ACTIVE_INST_VALU")
    if av:
        out.append(f"  VALU active (quad-cycles x 4) / (cycles x {N_SIMD}) = {4 * av / (cyc * N_SIMD):.3f}")
    hit, miss = cs.get("TCC_HIT_sum"), cs.get("TCC_MISS_sum")
    if hit is not None and miss is not None and hit + miss > 0:
        out.append(f"  L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) = {hit / (hit + miss):.3f}")
    if "SQ_LDS_BANK_CONFLICT" in cs and cs.get("SQ_INSTS_LDS"):
        out.append(f"  LDS bank-conflict cycles per LDS instruction = {cs['SQ_LDS_BANK_CONFLICT'] / cs['SQ_INSTS_LDS']:.4f}")
    wl = cs.get("SQ_WAIT_INST_LDS")
    if wl is not None:
        out.append(f"  wave-cycles waiting for LDS issue (x 4) / (cycles x waves resident) = "
                   f"{4 * wl / (cyc * 2 * N_SIMD):.3f}")
    return out


def kernel_source_sha(root: str) -> str:
    """Hash of the kernel sources with comments and blank space removed, so a
    record stays valid across comment edits and goes stale on code changes."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("attn_fwd_kernel.hip", "attn_fwd_internal.h"):
        with open(os.path.join(root, "bf16_attention_forward_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib, workload, out, command):
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    f = counter_means(fetch_dir)["attn_fwd_main"]["FETCH_SIZE"]
    w = counter_means(write_dir)["attn_fwd_main"]["WRITE_SIZE"]
    cf = [v["FETCH_SIZE"] for k, v in counter_means(cfetch_dir).items() if k.startswith("copy:")][0]
    cw = [v["WRITE_SIZE"] for k, v in counter_means(cwrite_dir).items() if k.startswith("copy:")][0]
    copy_bytes = copy_mib * 1024 * 1024
    f_scale = cf * 1024.0 / copy_bytes      # counter bytes per true byte read
    w_scale = cw * 1024.0 / copy_bytes
    rec = {}
    if os.path.exists(out):
        with open(out) as fh:
            rec = json.load(fh)
    sha = kernel_source_sha(root)
    if rec.get("kernel_source_sha") != sha:
        rec = {"kernel_source_sha": sha, "workloads": {}}
    rec["workloads"][workload] = {
        "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w,
        "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": copy_bytes,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_read_bytes_per_launch": f * 1024.0 / f_scale,
        "hbm_write_bytes_per_launch": w * 1024.0 / w_scale,
        "hbm_bytes_per_launch": f * 1024.0 / f_scale + w * 1024.0 / w_scale,
        "command": command,
    }
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec["workloads"][workload], indent=1))


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
        s.add_argument("--dir", required=True, nargs="+")
        s.add_argument("--out", required=True)
        s.add_argument("--command", required=True)
        s.add_argument("--title", default="")
        s.add_argument("--last", type=int, default=0, help="also summarise each kernel's last N dispatches")
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy-fetch", "copy-write", "workload", "out", "command"):
        t.add_argument("--" + n, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    a = ap.parse_args()
    if a.cmd == "traffic":
        traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.workload, a.out, a.command)
        return
    if a.cmd == "copy":
        do_copy(a.mib, a.iters)
        return
    lines = [f"# {a.title}".rstrip(), "", f"command: {a.command}", ""]
    if a.cmd == "stats":
        for label, last in (("all dispatches", 0), (f"last {a.last} dispatches (the timed steps)", a.last)):
            if label.startswith("last") and last <= 0:
                continue
            st = kernel_stats(a.dir[0], last)
            lines.append(f"## {label}")
            lines.append(f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} {'max_us':>10s}")
            for k, v in sorted(st.items(), key=lambda kv: -kv[1]["total_ns"]):
                lines.append(f"{k:40s} {v['calls']:6d} {v['avg_ns'] / 1e3:10.2f} {v['median_ns'] / 1e3:10.2f} "
                             f"{v['min_ns'] / 1e3:10.2f} {v['max_ns'] / 1e3:10.2f}")
            lines.append("")
    else:
        cm = defaultdict(dict)
        for d in a.dir:
            for k, cs in counter_means(d).items():
                cm[k].update(cs)
        for k, cs in sorted(cm.items()):
            lines.append(f"[{k}] per-dispatch means")
            for cn, val in sorted(cs.items()):
                lines.append(f"  {cn:40s} {val:20.3f}")
            if "GRBM_GUI_ACTIVE" in cs and not k.startswith("copy:"):
                lines += ["", "Derived:"] + derived_lines(cs)
            lines.append("")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
