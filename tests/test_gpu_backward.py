"""GPU parity of the backward pass (attn_bwd_bf16), through the C ABI.

The backward starts from the forward's output O and log-sum-exp; here both
come from the oracle (its fp64 output rounded to bf16, and its fp64 lse as
fp32), and the oracle's gradients take delta_i = <dO_i, O_i> from that same O.
Every gradient element is gated like the forward output: within 2 bf16 ULP
and at least 99.9% within 1, the ULP taken at max(|exact|, 2 sigma), sigma the
RMS size of the terms its sum adds.  The kernels feed P and dS to the MFMAs as
bf16, which is what the sigma floor absorbs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import gate
from bf16_attention_forward_amd import workloads as wl
from tests.helpers import say, to_dev

pytestmark = pytest.mark.gpu
SCALE = wl.DEFAULT_SCALE


def rows_first(bits, layout):
    """[B,S,H,D] or [B,H,S,D] bits -> [(b*H + h)*S + s, D]."""
    if layout == "bshd":
        bits = bits.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(bits).reshape(-1, bits.shape[-1])


def case_inputs(layout, B, H, Sq, Skv, seed, causal=False, Hkv=None, D=128, scale=SCALE):
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, seed, 1.0, 2.0, 1.0, Hkv=Hkv, D=D)
    do = wl.random_qkv(layout, B, H, Sq, 1, seed + 5000, D=D)[0]
    fwd = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=scale, method=False,
                           causal=causal)
    o_rows = fwd.rounded("rtne").reshape(B, H, Sq, D)
    o_bits = o_rows.transpose(0, 2, 1, 3).copy() if layout == "bshd" else o_rows.copy()
    o = torch.from_numpy(o_bits.view(np.int16)).view(torch.bfloat16)
    lse = torch.from_numpy(fwd.lse.astype(np.float32).reshape(B, H, Sq))
    return q, k, v, do, o, o_bits, lse


def run_bwd(q, k, v, o, do, lse, layout, causal=False, scale=SCALE):
    from bf16_attention_forward_amd import attn_bwd_bf16
    dq, dk, dv = attn_bwd_bf16(to_dev(q), to_dev(k), to_dev(v), to_dev(o), to_dev(do), to_dev(lse),
                               layout=layout, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return wl.bits(dq.cpu()), wl.bits(dk.cpu()), wl.bits(dv.cpu())


CASES = [
    ("bshd", 2, 3, 257, 130),    # ragged query and key tails
    ("bhsd", 1, 2, 300, 1000),   # several key blocks and query tiles
    ("bhsd", 1, 2, 64, 64),      # one tile each
    ("bhsd", 1, 1, 700, 333),    # Sq > Skv
    ("bshd", 1, 2, 1, 77),       # a single query
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}H{c[2]}_{c[3]}x{c[4]}")
def test_backward_matches_oracle(case):
    layout, B, H, Sq, Skv = case
    q, k, v, do, o, o_bits, lse = case_inputs(layout, B, H, Sq, Skv, 300 + Sq + Skv)
    say(f"[case] backward {case}")
    gq, gk, gv = run_bwd(q, k, v, o, do, lse, layout)
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                               o=o_bits)
    for name, g, exact, sig in (("dq", gq, ref.dq, ref.sdq), ("dk", gk, ref.dk, ref.sdk), ("dv", gv, ref.dv, ref.sdv)):
        st = gate.compare(rows_first(g, layout), exact, sig, "rtne")
        say(f"[gate] backward {case} {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)


CAUSAL_CASES = [
    ("bhsd", 1, 2, 300, 300),    # square: the diagonal crosses tiles of both kernels
    ("bshd", 2, 3, 200, 333),    # Sq < Skv: queries are the last positions
    ("bhsd", 1, 2, 333, 130),    # Sq > Skv: leading rows see no key (lse -inf, dQ = 0)
    ("bhsd", 1, 1, 600, 100),    # a whole dQ work-group of rows sees no key
    ("bshd", 1, 2, 64, 1000),    # most keys before the queries; dK/dV work-groups start late
    ("bhsd", 1, 2, 70, 700),     # the first dK/dV work-groups see every query
]


@pytest.mark.parametrize("case", CAUSAL_CASES, ids=lambda c: f"{c[0]}_B{c[1]}H{c[2]}_{c[3]}x{c[4]}_causal")
def test_causal_backward_matches_oracle(case):
    """The causal mask of the forward (bottom-right aligned): O and lse from
    the oracle's masked forward, gradients against its masked backward."""
    layout, B, H, Sq, Skv = case
    q, k, v, do, o, o_bits, lse = case_inputs(layout, B, H, Sq, Skv, 700 + Sq + Skv, causal=True)
    say(f"[case] causal backward {case}")
    gq, gk, gv = run_bwd(q, k, v, o, do, lse, layout, causal=True)
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                               o=o_bits, causal=True)
    # A row that sees exactly one key (row Sq - Skv) is the single-key case:
    # its exact dQ is 0, the kernel's is fp32 rounding noise (bound as in
    # test_single_key_backward); every other element meets the gate.
    one = Skv - Sq
    seen1 = np.zeros((B * H, Sq), bool)
    if 0 <= -one < Sq:
        seen1[:, -one] = True
    gq_rows = rows_first(gq, layout)
    keep = ~seen1.reshape(-1)
    for name, g, exact, sig in (("dq", gq_rows[keep], ref.dq[keep], ref.sdq[keep]),
                                ("dk", rows_first(gk, layout), ref.dk, ref.sdk),
                                ("dv", rows_first(gv, layout), ref.dv, ref.sdv)):
        st = gate.compare(g, exact, sig, "rtne")
        say(f"[gate] causal backward {case} {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)
    if seen1.any():
        assert np.all(ref.dq[~keep] == 0)
        mx = lambda t: float(t.float().abs().max())
        bound = SCALE * 2.0 ** -9 * mx(do) * mx(v) * mx(k)
        assert np.all(np.abs(oracle.bf16_bits_to_f64(gq_rows[~keep])) <= bound)
    # rows that see no key (Sq > Skv) have dQ = 0 exactly
    no_key = np.arange(Sq) + (Skv - Sq) < 0
    assert np.all(gq_rows.reshape(B * H, Sq, 128)[:, no_key] == 0)


def test_causal_forward_then_backward_on_the_gpu():
    """End to end under the mask: the GPU causal forward's O and lse feed the
    GPU causal backward, against the oracle's gradients for that same O (its
    delta from the GPU's O).  Against the gradients of the exact output the
    first rows fail the gate: a row that sees few keys has dP - delta
    cancel, which magnifies the rounding of O inside delta."""
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa, attn_bwd_bf16
    layout, B, H, Sq, Skv = "bshd", 1, 2, 400, 400
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 49, 1.0, 2.0, 1.0)
    do = wl.random_qkv(layout, B, H, Sq, 1, 5049)[0]
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = attn_fwd_bf16_gqa(qd, kd, vd, layout=layout, causal=True, return_lse=True)
    dq, dk, dv = attn_bwd_bf16(qd, kd, vd, o, dod, lse, layout=layout, causal=True)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                               o=wl.bits(o.cpu()), causal=True)
    # row 0 sees one key: its exact dQ is 0 (checked in the test above)
    keep = np.ones(B * H * Sq, bool)
    keep[np.arange(B * H) * Sq] = False
    dq_rows = rows_first(wl.bits(dq.cpu()), layout)
    for name, g, exact, sig in (("dq", dq_rows[keep], ref.dq[keep], ref.sdq[keep]),
                                ("dk", rows_first(wl.bits(dk.cpu()), layout), ref.dk, ref.sdk),
                                ("dv", rows_first(wl.bits(dv.cpu()), layout), ref.dv, ref.sdv)):
        st = gate.compare(g, exact, sig, "rtne")
        say(f"[gate] causal fwd+bwd {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)


GQA_CASES = [
    # layout, B, Hq, Hkv, Sq, Skv, causal
    ("bhsd", 1, 4, 1, 300, 500, False),    # one key/value head for four query heads
    ("bshd", 2, 6, 2, 257, 130, False),    # ragged tails, three query heads per group
    ("bhsd", 1, 4, 2, 300, 300, True),     # with the causal mask
    ("bshd", 1, 8, 2, 200, 333, True),     # Sq < Skv under the mask
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: f"{c[0]}_B{c[1]}Hq{c[2]}Hkv{c[3]}_{c[4]}x{c[5]}_{'causal' if c[6] else 'full'}")
def test_grouped_heads_backward_matches_oracle(case):
    """Grouped-query heads: dQ per query head from its key/value head, dK and
    dV of a key/value head summed over its query heads (O and lse from the
    oracle's grouped forward)."""
    layout, B, Hq, Hkv, Sq, Skv, causal = case
    q, k, v, do, o, o_bits, lse = case_inputs(layout, B, Hq, Sq, Skv, 900 + Sq + Skv, causal=causal, Hkv=Hkv)
    say(f"[case] grouped backward {case}")
    gq, gk, gv = run_bwd(q, k, v, o, do, lse, layout, causal=causal)
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                               o=o_bits, causal=causal)
    gq_rows = rows_first(gq, layout)
    keep = np.ones(B * Hq * Sq, bool)
    if causal and 0 <= Sq - Skv < Sq:
        keep.reshape(B * Hq, Sq)[:, Sq - Skv] = False     # rows that see one key: exact dQ 0 (noise bound below)
    for name, g, exact, sig in (("dq", gq_rows[keep], ref.dq[keep], ref.sdq[keep]),
                                ("dk", rows_first(gk, layout), ref.dk, ref.sdk),
                                ("dv", rows_first(gv, layout), ref.dv, ref.sdv)):
        st = gate.compare(g, exact, sig, "rtne")
        say(f"[gate] grouped backward {case} {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)
    if not keep.all():
        mx = lambda t: float(t.float().abs().max())
        bound = SCALE * 2.0 ** -9 * mx(do) * mx(v) * mx(k)
        assert np.all(np.abs(oracle.bf16_bits_to_f64(gq_rows[~keep])) <= bound)


def test_grouped_forward_then_backward_on_the_gpu():
    """End to end with grouped heads: the GPU grouped forward's O and lse feed
    the GPU backward; the oracle's gradients for that same O."""
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa, attn_bwd_bf16
    layout, B, Hq, Hkv, Sq, Skv = "bhsd", 1, 4, 2, 300, 700
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 51, 1.0, 2.0, 1.0, Hkv=Hkv)
    do = wl.random_qkv(layout, B, Hq, Sq, 1, 5051)[0]
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = attn_fwd_bf16_gqa(qd, kd, vd, layout=layout, return_lse=True)
    dq, dk, dv = attn_bwd_bf16(qd, kd, vd, o, dod, lse, layout=layout)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                               o=wl.bits(o.cpu()))
    for name, g, exact, sig in (("dq", dq, ref.dq, ref.sdq), ("dk", dk, ref.dk, ref.sdk), ("dv", dv, ref.dv, ref.sdv)):
        st = gate.compare(rows_first(wl.bits(g.cpu()), layout), exact, sig, "rtne")
        say(f"[gate] grouped fwd+bwd {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)


D64_CASES = [
    # layout, B, Hq, Hkv, Sq, Skv, causal
    ("bhsd", 1, 2, 2, 300, 500, False),
    ("bshd", 2, 3, 3, 257, 130, False),    # ragged tails
    ("bshd", 1, 4, 2, 257, 257, True),     # grouped heads and the causal mask
    ("bhsd", 1, 2, 1, 333, 130, True),     # Sq > Skv: rows without keys
]
SCALE64 = float(np.float32(0.125))


@pytest.mark.parametrize("case", D64_CASES, ids=lambda c: f"{c[0]}_B{c[1]}Hq{c[2]}Hkv{c[3]}_{c[4]}x{c[5]}_{'causal' if c[6] else 'full'}_d64")
def test_head_dim_64_backward_matches_oracle(case):
    """Head dimension 64 (128-byte rows, the backward's 8-position LDS
    swizzle), against the oracle's backward at D = 64."""
    layout, B, Hq, Hkv, Sq, Skv, causal = case
    q, k, v, do, o, o_bits, lse = case_inputs(layout, B, Hq, Sq, Skv, 1100 + Sq + Skv, causal=causal, Hkv=Hkv,
                                              D=64, scale=SCALE64)
    say(f"[case] d64 backward {case}")
    gq, gk, gv = run_bwd(q, k, v, o, do, lse, layout, causal=causal, scale=SCALE64)
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE64,
                               o=o_bits, causal=causal)
    gq_rows = rows_first(gq, layout)
    keep = np.ones(B * Hq * Sq, bool)
    if causal and 0 <= Sq - Skv < Sq:
        keep.reshape(B * Hq, Sq)[:, Sq - Skv] = False     # rows that see one key: exact dQ 0
    for name, g, exact, sig in (("dq", gq_rows[keep], ref.dq[keep], ref.sdq[keep]),
                                ("dk", rows_first(gk, layout), ref.dk, ref.sdk),
                                ("dv", rows_first(gv, layout), ref.dv, ref.sdv)):
        st = gate.compare(g, exact, sig, "rtne")
        say(f"[gate] d64 backward {case} {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)
    if not keep.all():
        mx = lambda t: float(t.float().abs().max())
        bound = SCALE64 * 2.0 ** -9 * mx(do) * mx(v) * mx(k)
        assert np.all(np.abs(oracle.bf16_bits_to_f64(gq_rows[~keep])) <= bound)
    if causal:   # rows that see no key (Sq > Skv under the mask) have dQ = 0 exactly
        no_key = np.arange(Sq) + (Skv - Sq) < 0
        assert np.all(gq_rows.reshape(B * Hq, Sq, 64)[:, no_key] == 0)


def test_head_dim_64_forward_then_backward_on_the_gpu():
    """End to end at head dimension 64: attn_fwd_bf16_hd's O and lse feed the
    backward; the oracle's gradients for that same O."""
    from bf16_attention_forward_amd import attn_fwd_bf16_hd, attn_bwd_bf16
    layout, B, H, Sq, Skv = "bshd", 1, 4, 400, 600
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 53, 1.0, 2.0, 1.0, D=64)
    do = wl.random_qkv(layout, B, H, Sq, 1, 5053, D=64)[0]
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = attn_fwd_bf16_hd(qd, kd, vd, layout=layout, scale=SCALE64, return_lse=True)
    dq, dk, dv = attn_bwd_bf16(qd, kd, vd, o, dod, lse, layout=layout, scale=SCALE64)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE64,
                               o=wl.bits(o.cpu()))
    for name, g, exact, sig in (("dq", dq, ref.dq, ref.sdq), ("dk", dk, ref.dk, ref.sdk), ("dv", dv, ref.dv, ref.sdv)):
        st = gate.compare(rows_first(wl.bits(g.cpu()), layout), exact, sig, "rtne")
        say(f"[gate] d64 fwd+bwd {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f}")
        assert st["passed"], (name, st)


@pytest.mark.parametrize("sq", [1, 70])
def test_single_key_backward(sq):
    """One key: the softmax is constant, so dS = P (dP - delta) = 0 and dQ = dK
    = 0 exactly, while dV is the sum of dO over the queries.  The kernel forms
    dP and delta as two fp32 dot products of the same 128 products in different
    orders; each is within 128 u (u = 2^-24) of the sum of the absolute
    products (at most 128 max|dO| max|V|), so |dP - delta| <= 2^-9 max|dO|
    max|V|, and with P <= 1 the gradients stay below scale 2^-9 max|dO| max|V|
    times max|K| (dQ) or Sq max|Q| (dK)."""
    layout, B, H = "bhsd", 1, 2
    q, k, v, do, o, o_bits, lse = case_inputs(layout, B, H, sq, 1, 57 + sq)
    gq, gk, gv = run_bwd(q, k, v, o, do, lse, layout)
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                               o=o_bits)
    assert np.all(ref.dq == 0) and np.all(ref.dk == 0)
    mx = lambda t: float(t.float().abs().max())
    noise = SCALE * 2.0 ** -9 * mx(do) * mx(v)
    f = lambda bits: oracle.bf16_bits_to_f64(bits)
    say(f"[gate] single key sq={sq}: max|dq| {np.abs(f(gq)).max():.2e} max|dk| {np.abs(f(gk)).max():.2e} "
        f"bounds {noise * mx(k):.2e} {noise * mx(q) * sq:.2e}")
    assert np.all(np.abs(f(gq)) <= noise * mx(k))
    assert np.all(np.abs(f(gk)) <= noise * mx(q) * sq)
    st = gate.compare(rows_first(gv, layout), ref.dv, ref.sdv, "rtne")
    assert st["passed"], st


def test_backward_deterministic():
    layout, B, H, Sq, Skv = "bhsd", 1, 2, 300, 400
    q, k, v, do, o, _, lse = case_inputs(layout, B, H, Sq, Skv, 41)
    a = run_bwd(q, k, v, o, do, lse, layout)
    b = run_bwd(q, k, v, o, do, lse, layout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_forward_then_backward_on_the_gpu():
    """End to end: the GPU forward's O and lse feed the GPU backward, compared
    with the oracle's gradients for the exact output.  lse is formed from the
    bf16 weights (error below 2^-8, a common factor on each row's weights) and O
    is rounded, yet the gradients still meet the same gate."""
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa, attn_bwd_bf16
    layout, B, H, Sq, Skv = "bhsd", 1, 2, 300, 500
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 47, 1.0, 2.0, 1.0)
    do = wl.random_qkv(layout, B, H, Sq, 1, 5047)[0]
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = attn_fwd_bf16_gqa(qd, kd, vd, layout=layout, return_lse=True)
    dq, dk, dv = attn_bwd_bf16(qd, kd, vd, o, dod, lse, layout=layout)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE)
    for name, g, exact, sig in (("dq", dq, ref.dq, ref.sdq), ("dk", dk, ref.dk, ref.sdk), ("dv", dv, ref.dv, ref.sdv)):
        st = gate.compare(rows_first(wl.bits(g.cpu()), layout), exact, sig, "rtne")
        say(f"[gate] fwd+bwd {name} max_D={st['max_D']:.2f} >1={st['frac_D_gt1']:.5f} >2={st['frac_D_gt2']:.5f}")
        assert st["passed"], (name, st)
