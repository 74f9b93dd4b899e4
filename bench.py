#!/usr/bin/env python3
"""Benchmark: bf16 attention forward on one MI355X through the C ABI.

One "step" is one call of attn_fwd_bf16 (the whole hot path: key/value
staging, both MFMA products, the online softmax, the rounding epilogue and,
when the planner splits keys, the combine kernel) over one batch of seeded
synthetic input already resident in HBM.

Default workload: the largest single-GPU configuration, video-diffusion
self-attention, BSHD, B=1, H=12, Sq=Skv=32760 (a 21x30x52 latent grid), head
dim 128, Q/K/V ~ N(0,1)*0.5, RTNE output.  The other workloads are timed too
and reported under "workloads".  Methodology follows the HipKittens summary's
experiments section: warm-up launches, then timed launches on N(0,1)-style
inputs; before the warm-up the workload runs back to back for a few seconds
so the timed launches see the clock the GPU settles at under this load, and
the shader clock is sampled during the timed launches.

Prints ONE JSON line:
  value        = algorithmic TFLOP/s (4*B*H*Sq*Skv*128 / wall time per step)
  roofline     = the main kernel's achieved TFLOP/s (HIP events around each
                 launch on the launch stream) against the dense bf16 MFMA peak
  cpu_baseline = the fp64 oracle timed on a bounded row sample on the host
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4 SIMD x 1024 flop/clk x 2.4 GHz (dense, published 2.5 PFLOP/s)
HBM_PEAK_GBS = 8000.0


def measured_traffic(workload_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_main_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from bf16_attention_forward_amd.profiling import kernel_source_sha
    ent = rec.get("workloads", {}).get(workload_name)
    if not ent or rec.get("kernel_source_sha") != kernel_source_sha(ROOT):
        return None
    return ent.get("hbm_bytes_per_launch")


def time_workload(w, mode, steps, warmup, kv_splits=0, round_weights=False, block_order=0, settle_s=0.0,
                  sample_clock=False):
    """Time `steps` launches of workload w after `warmup` untimed ones (and,
    with settle_s > 0, after running it back to back for that many seconds
    first).  Returns wall seconds of the timed launches, per-launch ms from
    HIP events recorded on the launch stream, and (sample_clock) the shader
    clock levels read while the timed launches ran."""
    import threading
    import torch
    from bf16_attention_forward_amd import attn_fwd_bf16, attn_fwd_bf16_gqa, attn_fwd_bf16_hd
    from bf16_attention_forward_amd import workloads as wl

    q, k, v = wl.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    stream = torch.cuda.current_stream(dev)

    def step():
        if w.D != 128:
            attn_fwd_bf16_hd(qd, kd, vd, od, layout=w.layout, round_mode=mode, stream=stream, causal=w.causal,
                             scale=w.scale, round_weights=round_weights)
        elif w.causal or w.Hkv:
            attn_fwd_bf16_gqa(qd, kd, vd, od, layout=w.layout, round_mode=mode, stream=stream, causal=w.causal,
                              round_weights=round_weights)
        else:
            attn_fwd_bf16(qd, kd, vd, od, layout=w.layout, round_mode=mode, stream=stream, kv_splits=kv_splits,
                          block_order=block_order,
                          round_weights=round_weights)

    if settle_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # per-launch HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    clocks, done = [], threading.Event()

    def sampler():
        while not done.wait(0.05):
            mhz = read_sclk_mhz()
            if mhz is not None:
                clocks.append(mhz)

    th = threading.Thread(target=sampler, daemon=True) if sample_clock else None
    torch.cuda.synchronize()
    if th:
        th.start()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if th:
        done.set()
        th.join()
    per = [a.elapsed_time(b) for a, b in evs]   # ms
    return {"wall_s": wall, "ms": per, "flops": w.flops, "sclk_mhz": clocks}


def time_cold(w, mode, steps, warmup=20):
    """Per-launch ms of workload w with the caches cleared before every launch:
    a 512 MiB fill on the launch stream (outside the events) evicts the L2s
    and the last-level cache, so every launch reads Q, K, V from HBM."""
    import torch
    from bf16_attention_forward_amd import attn_fwd_bf16
    from bf16_attention_forward_amd import workloads as wl

    q, k, v = wl.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        attn_fwd_bf16(qd, kd, vd, od, layout=w.layout, round_mode=mode, stream=stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        flush.fill_(i & 0xff)
        a.record(stream)
        attn_fwd_bf16(qd, kd, vd, od, layout=w.layout, round_mode=mode, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def read_sclk_mhz():
    """The GPU's current shader clock level in MHz, read from the driver's
    sysfs table of clock levels (the line marked '*') for this device's PCI
    address; None when it cannot be read.  A plain file read: no child
    program is started."""
    import re
    import torch
    try:
        pr = torch.cuda.get_device_properties(0)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        with open(f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk") as fh:
            text = fh.read()
    except Exception:
        return None
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*mhz", line.lower())
            return int(m.group(1)) if m else None
    return None


# algorithmic FLOPs of the backward pass: five products of the forward's
# size (the recomputed S, dP, dV, dQ, dK) against the forward's two
BWD_FLOP_FACTOR = 2.5


def time_paged(steps, warmup):
    """Median ms of attn_fwd_bf16_paged on the paged-cache workload (the whole
    call: with its 256-row pages the kernel reads the cache in place)."""
    import torch
    from bf16_attention_forward_amd import attn_fwd_bf16_paged
    from bf16_attention_forward_amd import workloads as wl

    c = wl.PAGED
    pk = wl.make_paged_kv(c["B"], c["H"], c["kv_lens"], c["page_size"], seed=c["seed"])
    q = wl.random_qkv("bshd", c["B"], c["H"], c["Sq"], 1, c["seed"])[0]
    dev = torch.device("cuda:0")
    qd, kc, vc = q.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev)
    bt, kl = pk.block_table.to(dev), pk.kv_lens.to(dev)
    od = torch.empty_like(qd)
    run = lambda: attn_fwd_bf16_paged(qd, kc, vc, bt, kl, od, max_kv_len=pk.max_kv_len, layout="bshd")
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) for a, b in evs])


def time_varlen(steps, warmup):
    """Median ms of attn_fwd_bf16_varlen on the packed-sequence workload."""
    import torch
    from bf16_attention_forward_amd import attn_fwd_bf16_varlen
    from bf16_attention_forward_amd import workloads as wl

    c = wl.VARLEN
    pk = wl.make_packed(c["H"], c["H"], c["lens"], c["lens"], seed=c["seed"], q_factor=0.5, k_factor=0.5,
                        v_factor=0.5)
    dev = torch.device("cuda:0")
    qd, kd, vd = pk.q.to(dev), pk.k.to(dev), pk.v.to(dev)
    cq, ck = pk.cu_q.to(dev), pk.cu_k.to(dev)
    od = torch.empty_like(qd)
    m = max(c["lens"])
    run = lambda: attn_fwd_bf16_varlen(qd, kd, vd, cq, ck, od, max_seqlen_q=m, max_seqlen_k=m)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) for a, b in evs])


def time_backward(w, steps, warmup):
    """Median ms of attn_bwd_bf16 on workload w (O and lse from the forward)."""
    import torch
    from bf16_attention_forward_amd import attn_bwd_bf16, attn_fwd_bf16_hd
    from bf16_attention_forward_amd import workloads as wl

    q, k, v = wl.make_inputs(w)
    do = wl.random_qkv(w.layout, w.B, w.H, w.Sq, 1, w.seed + 5000, D=w.D)[0]
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = attn_fwd_bf16_hd(qd, kd, vd, layout=w.layout, scale=w.scale, causal=w.causal, return_lse=True)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    bwd = lambda: attn_bwd_bf16(qd, kd, vd, o, dod, lse, layout=w.layout, scale=w.scale, causal=w.causal,
                                dq=dq, dk=dk, dv=dv)
    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        bwd()
        b.record()
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) for a, b in evs])


def cpu_baseline(w, budget_s: float):
    import numpy as np
    import oracle
    from bf16_attention_forward_amd import workloads as wl
    q, k, v = wl.make_inputs(w)
    qb, kb, vb = wl.bits(q), wl.bits(k), wl.bits(v)
    threads = os.cpu_count() or 1
    total_rows = w.B * w.H * w.Sq
    rng = np.random.default_rng(w.seed)
    calib = np.sort(rng.choice(total_rows, size=min(256, total_rows), replace=False))
    t = time.perf_counter()
    oracle.attention(qb, kb, vb, layout=w.layout, scale=wl.DEFAULT_SCALE, rows=calib, method=False, nthreads=threads)
    dt = max(time.perf_counter() - t, 1e-6)
    n = int(min(total_rows, max(256, len(calib) * budget_s / dt)))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False))
    t = time.perf_counter()
    oracle.attention(qb, kb, vb, layout=w.layout, scale=wl.DEFAULT_SCALE, rows=rows, method=False, nthreads=threads)
    dt = time.perf_counter() - t
    flops = 4.0 * n * w.Skv * 128
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {total_rows} query rows (seeded uniform sample) of {w.name}, all {w.Skv} keys, "
                      f"fp64, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=3, help="workload number (1..9)")
    ap.add_argument("--settle", type=float, default=3.0,
                    help="seconds of back-to-back launches before the warm-up (clock settling)")
    ap.add_argument("--block-order", choices=["planner", "naive", "xcd"], default="planner",
                    help="work-group order of the plain entry point (an ablation of the XCD-aware order)")
    ap.add_argument("--sq", type=int, default=0,
                    help="override the workload's query length (e.g. for a ragged last round of work items)")
    ap.add_argument("--kv-splits", type=int, default=0,
                    help="key splits of the plain entry point: 0 = planner, 1 = never (an ablation of the tail split)")
    ap.add_argument("--mode", default="rtne")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--backward", action="store_true",
                    help="time only the backward pass of the workload (one JSON line of its own)")
    ap.add_argument("--paged", action="store_true",
                    help="time only the paged key/value cache workload (one JSON line of its own)")
    ap.add_argument("--varlen", action="store_true",
                    help="time only the packed-sequence workload (one JSON line of its own)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the work shards over (batch, head, query tile) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bf16_attention_forward_amd import workloads as wl
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)

    w = wl.WORKLOADS[args.workload]
    if args.sq:
        import dataclasses
        w = dataclasses.replace(w, Sq=args.sq, name=f"{w.name}_sq{args.sq}")
    if args.backward:
        if w.D not in (128, 64):
            print(f"the backward pass covers head dimensions 128 and 64; not {w.name}", file=sys.stderr)
            sys.exit(2)
        em = time_backward(w, steps=args.steps, warmup=args.warmup)
        tf = BWD_FLOP_FACTOR * w.flops / (em * 1e-3) / 1e12
        print(json.dumps({"metric": "attention bwd TFLOPS (2.5 x 4*B*H*Sq*Skv*d) and % of bf16 MFMA peak",
                          "value": round(tf, 2), "unit": "TFLOP/s", "median_ms": round(em, 5),
                          "steps": args.steps, "warmup": args.warmup,
                          "frac_of_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "config": {**w.describe(), "pass": "backward"}}), flush=True)
        return
    if args.paged:
        c = wl.PAGED
        em = time_paged(steps=args.steps, warmup=args.warmup)
        tf = wl.paged_flops(c["H"], c["Sq"], c["kv_lens"]) / (em * 1e-3) / 1e12
        print(json.dumps({"metric": "paged-cache attention fwd TFLOPS (sum over entries of 4*H*Sq*kv_len*d), "
                                    "the whole call",
                          "value": round(tf, 2), "unit": "TFLOP/s", "median_ms": round(em, 5),
                          "steps": args.steps, "warmup": args.warmup,
                          "frac_of_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "config": {"workload": c["name"], "B": c["B"], "H": c["H"], "Sq": c["Sq"],
                                     "kv_lens": list(c["kv_lens"]), "page_size": c["page_size"],
                                     "head_dim": 128, "layout": "bshd", "round_mode": "rtne"}}), flush=True)
        return
    if args.varlen:
        c = wl.VARLEN
        em = time_varlen(steps=args.steps, warmup=args.warmup)
        tf = wl.varlen_flops(c["H"], c["lens"], c["lens"]) / (em * 1e-3) / 1e12
        print(json.dumps({"metric": "packed-sequence attention fwd TFLOPS (sum over sequences of 4*H*len^2*d)",
                          "value": round(tf, 2), "unit": "TFLOP/s", "median_ms": round(em, 5),
                          "steps": args.steps, "warmup": args.warmup,
                          "frac_of_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "config": {"workload": c["name"], "H": c["H"], "lens": list(c["lens"]),
                                     "head_dim": 128, "layout": "thd", "round_mode": "rtne"}}), flush=True)
        return
    sclk_idle = read_sclk_mhz()
    order = {"planner": 0, "naive": 1, "xcd": 2}[args.block_order]
    r = time_workload(w, args.mode, args.steps, args.warmup, block_order=order, kv_splits=args.kv_splits,
                      settle_s=args.settle, sample_clock=True)
    ms_step = r["wall_s"] * 1e3 / args.steps
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    ev_mean = statistics.fmean(r["ms"])
    achieved = w.flops / (ev_mean * 1e-3) / 1e12
    srt = sorted(r["ms"])
    traffic = measured_traffic(w.name)
    sk = sorted(r["sclk_mhz"])
    clocks = {"sclk_mhz_idle_before": sclk_idle,
              "sclk_mhz_timed_median": sk[len(sk) // 2] if sk else None,
              "sclk_mhz_timed_min": sk[0] if sk else None, "sclk_mhz_timed_max": sk[-1] if sk else None,
              "sclk_samples": len(sk), "settle_s": args.settle,
              "source": "sysfs pp_dpm_sclk (current level), sampled every 50 ms during the timed launches"}
    if sk:
        # dense bf16 peak at the clock the timed launches ran at
        clocks["peak_tflops_at_timed_median_clock"] = round(MFMA_BF16_PEAK_TFLOPS * clocks["sclk_mhz_timed_median"]
                                                            / 2400.0, 1)

    extra = {}
    if not args.no_extra:
        # caches cleared before every launch (the timed value above runs warm,
        # as the HipKittens experiments do)
        cold = sorted(time_cold(w, args.mode, steps=10 if w.flops > 2e12 else 30))
        em = statistics.median(cold)
        extra[f"{w.name}:cold_cache"] = {"mode": args.mode, "median_ms": round(em, 4), "min_ms": round(cold[0], 4),
                                         "tflops": round(w.flops / (em * 1e-3) / 1e12, 1),
                                         "frac_peak": round(w.flops / (em * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        # every other workload in each of its rounding modes
        for num in sorted(wl.WORKLOADS):
            ww = wl.WORKLOADS[num]
            # sub-millisecond launches need more warm-up than the long ones
            # to reach a steady clock (100 launches of them take < 0.1 s)
            short = ww.flops < 2e12
            for mode in ww.modes:
                if ww.name == w.name and mode == args.mode:
                    continue
                rr = time_workload(ww, mode, steps=100 if short else 20, warmup=200 if short else 10,
                                   settle_s=0.5)
                em = statistics.median(rr["ms"])
                extra[f"{ww.name}:{mode}"] = {"mode": mode, "median_ms": round(em, 4),
                                              "tflops": round(ww.flops / (em * 1e-3) / 1e12, 1),
                                              "frac_peak": round(ww.flops / (em * 1e-3) / 1e12 /
                                                                 MFMA_BF16_PEAK_TFLOPS, 4)}
        # the option that rounds the in-loop weights with the output's mode,
        # on the 4096^2 self-attention workload
        w2 = wl.WORKLOADS[2]
        for mode in w2.modes:
            rr = time_workload(w2, mode, steps=100, warmup=200, round_weights=True, settle_s=0.5)
            em = statistics.median(rr["ms"])
            extra[f"{w2.name}:{mode}+weights"] = {"mode": mode, "round_weights": True, "median_ms": round(em, 4),
                                                  "tflops": round(w2.flops / (em * 1e-3) / 1e12, 1)}

        # backward pass of the 4096^2 workloads (plain, causal, head dim 64) and the grouped causal one
        for ww in (wl.WORKLOADS[2], wl.WORKLOADS[7], wl.WORKLOADS[6], wl.WORKLOADS[8]):
            em = time_backward(ww, steps=20, warmup=5)
            tf = BWD_FLOP_FACTOR * ww.flops / (em * 1e-3) / 1e12
            extra[f"{ww.name}:backward"] = {"median_ms": round(em, 4), "tflops": round(tf, 1),
                                            "frac_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}

        # the paged key/value cache (per-entry lengths, 256-token pages)
        c = wl.PAGED
        em = time_paged(steps=20, warmup=5)
        tf = wl.paged_flops(c["H"], c["Sq"], c["kv_lens"]) / (em * 1e-3) / 1e12
        extra[f"{c['name']}:rtne"] = {"median_ms": round(em, 4), "tflops": round(tf, 1),
                                      "frac_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                      "note": "the whole call (keys and values read in place from the pages)"}
        # packed sequences of different lengths
        c = wl.VARLEN
        em = time_varlen(steps=20, warmup=5)
        tf = wl.varlen_flops(c["H"], c["lens"], c["lens"]) / (em * 1e-3) / 1e12
        extra[f"{c['name']}:rtne"] = {"median_ms": round(em, 4), "tflops": round(tf, 1),
                                      "frac_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget)

    factors = {"q": w.q_factor, "k": w.k_factor, "v": w.v_factor}
    scaled = ", ".join(f"{n.upper()} x{f:g}" for n, f in factors.items() if f != 1.0)
    out = {
        "metric": "attention fwd TFLOPS (4*B*H*Sq*Skv*d) and % of bf16 MFMA peak, d=128",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs" + (f", {scaled}" if scaled else "") + ")",
        "config": {**w.describe(), "round_mode": args.mode, "parallelism": "single GPU",
                   **({"block_order": args.block_order} if args.block_order != "planner" else {}),
                   **({"kv_splits": args.kv_splits} if args.kv_splits else {})},
        "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernel_ms": {"mean": round(ev_mean, 5), "median": round(statistics.median(srt), 5),
                      "min": round(srt[0], 5), "p90": round(srt[int(0.9 * (len(srt) - 1))], 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_main",
                     "algorithmic_flops_per_launch": w.flops},
        "cpu_baseline": cpu,
        "clocks": clocks,
        "workloads": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
