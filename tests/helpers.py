"""Shared helpers for the GPU parity tests (test-side only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import gate
from bf16_attention_forward_amd import workloads as wl


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda", non_blocking=False).contiguous()


def run_hip(q, k, v, layout, mode="rtne", scale=None, **kw) -> np.ndarray:
    """Run the HIP path on CPU bf16 tensors; return output bf16 bits (numpy uint16)."""
    from bf16_attention_forward_amd import attn_fwd_bf16
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = attn_fwd_bf16(qd, kd, vd, layout=layout, round_mode=mode,
                      scale=wl.DEFAULT_SCALE if scale is None else scale, **kw)
    torch.cuda.synchronize()
    return wl.bits(o.cpu())


def run_hip_gqa(q, k, v, layout, mode="rtne", causal=False, scale=None) -> np.ndarray:
    """attn_fwd_bf16_gqa on CPU bf16 tensors (k, v may have fewer heads); output bits."""
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = attn_fwd_bf16_gqa(qd, kd, vd, layout=layout, round_mode=mode, causal=causal,
                          scale=wl.DEFAULT_SCALE if scale is None else scale)
    torch.cuda.synchronize()
    return wl.bits(o.cpu())


def check(o_bits, q, k, v, layout, mode, *, rows=None, scale=None, label="", oracle_res=None, causal=False,
          weights_mode="rtne"):
    """Gate the HIP output against the oracle on all rows (rows=None) or a sample.

    Returns (stats, oracle result).  stats holds the definition gate (ULP
    floor 2 sigma against the exact output) and, under "method", the
    tighter gate against the oracle's method companion (bf16 weights rounded
    in `weights_mode`, normalised by their own sum; floor 1 sigma of that
    companion).  assert_gates() checks both."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
    else:
        B, H, Sq, _ = q.shape
    sc = wl.DEFAULT_SCALE if scale is None else scale
    res = oracle_res
    if res is None or res.o_method is None:
        res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=sc, rows=rows,
                               method=True, l_from_rounded=True, p_round=weights_mode, causal=causal)
    if rows is None:
        g = wl.gather_rows(o_bits, layout, B, H, Sq, np.arange(B * H * Sq))
    else:
        g = wl.gather_rows(o_bits, layout, B, H, Sq, rows)
    st = gate.compare(g, res.o_exact, res.sigma, mode)
    sm = gate.compare(g, res.o_method, res.sigma_method, mode, floor_factor=1.0)
    st["method"] = {k_: sm[k_] for k_ in ("nonfinite_match", "max_D", "frac_D_gt1", "frac_D_gt2",
                                          "literal_max_steps", "literal_frac_gt1", "passed")}
    say(f"[gate] {label} mode={mode} rows={len(res.rows)} {st}")
    return st, res


def assert_gates(st):
    """Both gates of check(): every finite element within 2 ULP, at least
    99.9% within 1, NaN/Inf positions identical -- against the exact output
    (floor 2 sigma) and against the method companion (floor 1 sigma)."""
    for s in (st, st["method"]):
        assert s["nonfinite_match"], st
        assert s["max_D"] <= 2.0, st
        assert s["frac_D_gt1"] <= 1e-3, st
