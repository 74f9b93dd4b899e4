"""GPU parity of the option that rounds the in-loop softmax weights with the
output's rounding mode (ATTN_ROUND_WEIGHTS), through the C ABI.

Two bars: the plain definition (every finite element within 2 bf16 ULP, at
least 99.9% within 1, NaN/Inf positions identical), and the oracle's method
companion whose bf16 weights are rounded in the same mode (normalised by the
sum of those rounded weights), which the kernel follows closely.  With the
values the identity over the keys the output is the rounded weights over their
sum, so truncated weights are visible directly (up to the rare weight whose
fp32 exponential rounds differently from the fp64 one)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import gate
from bf16_attention_forward_amd import workloads as wl
from tests.helpers import say, to_dev

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")


def run(q, k, v, layout, mode, causal=False, Hkv=None, **kw):
    from bf16_attention_forward_amd import attn_fwd_bf16, attn_fwd_bf16_gqa
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    if causal or Hkv is not None:
        o = attn_fwd_bf16_gqa(qd, kd, vd, layout=layout, round_mode=mode, causal=causal, round_weights=True)
    else:
        o = attn_fwd_bf16(qd, kd, vd, layout=layout, round_mode=mode, round_weights=True, **kw)
    torch.cuda.synchronize()
    return wl.bits(o.cpu())


CASES = [
    # layout, B, H, Hkv, Sq, Skv, causal, kv_splits
    ("bhsd", 1, 2, None, 300, 1000, False, 0),    # few work items: the planner splits the keys
    ("bshd", 2, 3, None, 257, 130, False, 1),     # ragged query and key tails, unsplit
    ("bhsd", 1, 4, 2, 300, 300, True, 0),         # grouped heads, causal
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_{c[4]}x{c[5]}{'_causal' if c[6] else ''}")
@pytest.mark.parametrize("mode", MODES)
def test_weights_rounded_in_mode(case, mode):
    layout, B, H, Hkv, Sq, Skv, causal, splits = case
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 700 + Sq, 1.0, 2.0, 1.0, Hkv=Hkv)
    kw = {} if (causal or Hkv is not None) else {"kv_splits": splits}
    g_bits = run(q, k, v, layout, mode, causal=causal, Hkv=Hkv, **kw)
    res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=wl.DEFAULT_SCALE,
                           method=True, l_from_rounded=True, p_round=mode, causal=causal)
    Hq = H
    g = wl.gather_rows(g_bits, layout, B, Hq, Sq, np.arange(B * Hq * Sq))
    st = gate.compare(g, res.o_exact, res.sigma, mode)
    sm = gate.compare(g, res.o_method, res.sigma_method, mode, floor_factor=1.0)
    say(f"[wround] {case} {mode} definition max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f} | "
        f"method max_D={sm['max_D']:.2f} >1={sm['frac_D_gt1']:.5f}")
    assert st["passed"], st
    assert sm["nonfinite_match"] and sm["max_D"] <= 2.0 and sm["frac_D_gt1"] <= 1e-3, sm


@pytest.mark.parametrize("mode", MODES)
def test_identity_values_show_the_weights(mode):
    """V = identity over 128 keys: o_j = pt_j / sum pt.  The output must follow
    the weights of its own mode; with truncated weights it must differ from
    the nearest-even weights' result on a sizeable share of elements."""
    Sq, Skv = 200, 128
    q, k, _ = wl.random_qkv("bhsd", 1, 2, Sq, Skv, 71, 1.0, 3.0, 1.0)
    vv = np.zeros((1, 2, Skv, 128), np.float32)
    vv[0, :, np.arange(Skv), np.arange(Skv)] = 1.0
    v = torch.from_numpy(vv).to(torch.bfloat16)
    g_bits = run(q, k, v, "bhsd", mode)
    g = wl.gather_rows(g_bits, "bhsd", 1, 2, Sq, np.arange(2 * Sq))
    same = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=wl.DEFAULT_SCALE,
                            method=True, l_from_rounded=True, p_round=mode)
    nearest = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=wl.DEFAULT_SCALE,
                               method=True, l_from_rounded=True, p_round="rtne")
    exp_same = oracle.round_bf16(same.o_method, mode)
    exp_near = oracle.round_bf16(nearest.o_method, mode)
    match_same = float(np.mean(g == exp_same))
    match_near = float(np.mean(g == exp_near))
    st = gate.compare(g, same.o_method, same.sigma_method, mode, floor_factor=1.0)
    say(f"[wround] identity {mode}: equal to own-mode weights {match_same:.4f}, to nearest-even weights "
        f"{match_near:.4f}, max_D={st['max_D']:.2f}")
    # a weight whose fp32 exponential lies on the other side of a bf16
    # rounding boundary than the fp64 one (about 2^-14 of them) moves its
    # output by one weight ulp: at most 2 output steps, rarely
    assert st["max_D"] <= 2.0 and st["frac_D_gt1"] <= 1e-3, st
    assert match_same >= 0.99
    if mode == "rtz":
        assert match_near < match_same - 0.05


def test_nonfinite_positions_with_rounded_weights():
    """NaN/+-Inf planted in Q and V of the self-attention workload: with the
    weights rounded in each mode the output's NaN/Inf pattern is still the
    closed form implied by IEEE arithmetic on the definition."""
    from tests.test_oracle_attention import closed_form_mask
    w = wl.WORKLOADS[2]
    q, k, v = wl.make_inputs(w)
    inj = wl.inject_nonfinite(q, v, w.layout, w.seed)
    expect = closed_form_mask(inj, w.B, w.H, w.Sq)
    for mode in MODES:
        say(f"[case] nonfinite, weights rounded {mode}")
        o = run(q, k, v, w.layout, mode).reshape(w.B, w.H, w.Sq, 128)
        vals = (o.astype(np.uint32) << 16).view(np.float32)
        got = np.where(np.isnan(vals), 1, np.where(np.isposinf(vals), 2, np.where(np.isneginf(vals), 3, 0)))
        assert np.array_equal(got, expect), f"{mode}: NaN/Inf pattern differs in {(got != expect).sum()} places"
        assert np.all(o[np.isnan(vals)] == 0x7FC0)


def test_growing_scores_with_rounded_weights():
    """Scores that keep outgrowing the softmax offset (the re-offset path)."""
    from tests.test_gpu_special import ramp_inputs
    q, k, v = ramp_inputs("bhsd", 1, 2, 300, 1000, 73)
    for mode in MODES:
        g_bits = run(q, k, v, "bhsd", mode, kv_splits=0)
        res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=wl.DEFAULT_SCALE,
                               method=False)
        g = wl.gather_rows(g_bits, "bhsd", 1, 2, 300, np.arange(600))
        st = gate.compare(g, res.o_exact, res.sigma, mode)
        say(f"[wround] ramp {mode} max_D={st['max_D']:.2f}")
        assert st["passed"], st
