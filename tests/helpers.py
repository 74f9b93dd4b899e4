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


def check(o_bits, q, k, v, layout, mode, *, rows=None, scale=None, label="", oracle_res=None, causal=False):
    """Gate the HIP output against the oracle on all rows (rows=None) or a sample."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
    else:
        B, H, Sq, _ = q.shape
    sc = wl.DEFAULT_SCALE if scale is None else scale
    res = oracle_res if oracle_res is not None else oracle.attention(
        wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=sc, rows=rows, method=False, causal=causal)
    if rows is None:
        g = wl.gather_rows(o_bits, layout, B, H, Sq, np.arange(B * H * Sq))
    else:
        g = wl.gather_rows(o_bits, layout, B, H, Sq, rows)
    st = gate.compare(g, res.o_exact, res.sigma, mode)
    say(f"[gate] {label} mode={mode} rows={len(res.rows)} {st}")
    return st, res
