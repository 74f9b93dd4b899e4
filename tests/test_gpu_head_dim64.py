"""GPU parity of head dimension 64 (attn_fwd_bf16_hd), through the C ABI,
against the fp64 oracle at D = 64: every finite element within 2 bf16 ULP, at
least 99.9% within 1, NaN/Inf positions identical; plus the identity that the
64-dimension kernel gives the first 64 dimensions of the 128-dimension kernel
on inputs zero-padded to 128: the scores, weights and weighted sums are the
same numbers, only the row sums add the same weights in another order (on the
matrix core at 64, on the vector ALU at 128), so an output may move by one
bf16 step where it lies within fp32 rounding of a bf16 boundary."""
import numpy as np
import pytest
import torch

import oracle
from oracle import gate
from bf16_attention_forward_amd import workloads as wl
from tests.helpers import say, to_dev

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")
SCALE64 = float(np.float32(0.125))


def run64(q, k, v, layout, mode="rtne", causal=False, scale=SCALE64, lse=False, **kw):
    from bf16_attention_forward_amd import attn_fwd_bf16_hd
    out = attn_fwd_bf16_hd(to_dev(q), to_dev(k), to_dev(v), layout=layout, round_mode=mode, causal=causal,
                           scale=scale, return_lse=lse, **kw)
    torch.cuda.synchronize()
    if lse:
        return wl.bits(out[0].cpu()), out[1].cpu().numpy().reshape(-1)
    return wl.bits(out.cpu())


def gate_all(o_bits, q, k, v, layout, mode, causal=False, scale=SCALE64, rows=None):
    if layout == "bshd":
        B, Sq, H, _ = q.shape
    else:
        B, H, Sq, _ = q.shape
    res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=scale, method=True,
                           l_from_rounded=True, causal=causal, rows=rows)
    g = wl.gather_rows(o_bits, layout, B, H, Sq, np.arange(B * H * Sq) if rows is None else rows)
    st = gate.compare(g, res.o_exact, res.sigma, mode)
    # the tighter gate against the method companion (bf16 weights, their own sum)
    sm = gate.compare(g, res.o_method, res.sigma_method, mode, floor_factor=1.0)
    st["method"] = sm
    st["passed"] = bool(st["passed"] and sm["passed"])
    return st, res


CASES = [
    # layout, B, Hq, Hkv, Sq, Skv, causal
    ("bshd", 2, 3, 3, 257, 130, False),     # ragged query and key tails
    ("bhsd", 1, 2, 2, 300, 1000, False),    # few work items: the planner splits the keys
    ("bhsd", 1, 4, 2, 300, 300, True),      # grouped heads, causal
    ("bshd", 1, 2, 1, 333, 130, True),      # Sq > Skv: leading rows see no key
    ("bhsd", 1, 3, 1, 1, 1, False),         # single query, single key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_Hq{c[2]}Hkv{c[3]}_{c[4]}x{c[5]}{'_causal' if c[6] else ''}")
@pytest.mark.parametrize("mode", MODES)
def test_d64_small_shapes_all_rows(case, mode):
    layout, B, Hq, Hkv, Sq, Skv, causal = case
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 900 + Sq, 1.0, 2.0, 1.0, Hkv=Hkv, D=64)
    say(f"[case] d64 {case} {mode}")
    o = run64(q, k, v, layout, mode, causal=causal)
    st, _ = gate_all(o, q, k, v, layout, mode, causal=causal)
    say(f"[gate] d64 {case} {mode} {st}")
    assert st["passed"], st


def test_d64_lse():
    q, k, v = wl.random_qkv("bhsd", 1, 4, 300, 700, 91, 1.0, 2.0, 1.0, Hkv=2, D=64)
    o, lse = run64(q, k, v, "bhsd", causal=True, lse=True)
    res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=SCALE64, method=False,
                           causal=True)
    fin = np.isfinite(res.lse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(res.lse))
    assert np.all(np.abs(lse[fin] - res.lse[fin]) <= 2.0 ** -8 + 2.0 ** -20 * np.abs(res.lse[fin]))


@pytest.mark.parametrize("case", [("bshd", 2, 3, 257, 130, False), ("bhsd", 1, 4, 300, 1000, False),
                                  ("bhsd", 1, 2, 300, 300, True)])
def test_d64_equals_d128_zero_padded(case):
    layout, B, H, Sq, Skv, causal = case
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 95, 1.0, 2.0, 1.0, D=64)
    pad = lambda t: torch.nn.functional.pad(t, (0, 64))
    o64 = run64(q, k, v, layout, causal=causal)
    o128 = run64(pad(q), pad(k), pad(v), layout, causal=causal)
    assert np.all(o128[..., 64:] == 0)
    steps = np.abs(gate.ordinal(o128[..., :64]).astype(np.int64) - gate.ordinal(o64).astype(np.int64))
    say(f"[pad] {case}: differing elements {np.mean(steps > 0):.2e}, max steps {steps.max()}")
    assert steps.max() <= 1 and np.mean(steps > 0) <= 1e-3


def test_d64_nonfinite_positions():
    from tests.test_oracle_attention import closed_form_mask
    layout, B, H, Sq, Skv = "bhsd", 1, 4, 512, 512
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 97, 1.0, 2.0, 1.0, D=64)
    inj = wl.inject_nonfinite(q, v, layout, 97)
    expect = closed_form_mask(inj, B, H, Sq, D=64)
    for mode in MODES:
        o = run64(q, k, v, layout, mode).reshape(B, H, Sq, 64)
        vals = (o.astype(np.uint32) << 16).view(np.float32)
        got = np.where(np.isnan(vals), 1, np.where(np.isposinf(vals), 2, np.where(np.isneginf(vals), 3, 0)))
        assert np.array_equal(got, expect), f"{mode}: NaN/Inf pattern differs in {(got != expect).sum()} places"
        assert np.all(o[np.isnan(vals)] == 0x7FC0)


@pytest.mark.parametrize("num", [8, 9])
def test_d64_full_size_sampled_rows(num):
    w = wl.WORKLOADS[num]
    q, k, v = wl.make_inputs(w)
    rows = wl.sample_rows(w.B, w.H, w.Sq, 4, w.seed)
    say(f"[case] {w.name} sampled rows {len(rows)}")
    o = run64(q, k, v, w.layout, w.modes[0], scale=w.scale)
    st, _ = gate_all(o, q, k, v, w.layout, w.modes[0], scale=w.scale, rows=rows)
    say(f"[gate] {w.name} {st}")
    assert st["passed"], st
