"""Pins of the oracle's backward pass (gradients of the plain operation).

The backward is pinned against a library routine (torch autograd through
softmax(Q K^T * scale) V in float64), a closed form (a single key: the softmax
is constant, so dQ = dK = 0 and dV is the sum of dO over the queries), and
the exact effect of starting from a given (rounded) forward output o: only the
row term delta_i = <dO_i, o_i> changes, by a known amount."""
import numpy as np
import pytest
import torch

import oracle
from bf16_attention_forward_amd import workloads as wl

SCALE = float(np.float32(1.0 / np.sqrt(128)))


def f64(t):
    return t.to(torch.float64)


def heads_first(t, layout):
    return t.permute(0, 2, 1, 3) if layout == "bshd" else t


def autograd_grads(q, k, v, do, layout, scale, causal):
    Q, K, V, G = (heads_first(f64(t), layout).clone().requires_grad_(i < 3) for i, t in enumerate((q, k, v, do)))
    group = Q.shape[1] // K.shape[1]
    # grouped heads: each key/value head serves `group` consecutive query
    # heads; autograd adds the repeated heads' gradients into the original
    Kr, Vr = K.repeat_interleave(group, dim=1), V.repeat_interleave(group, dim=1)
    S = scale * (Q @ Kr.transpose(-1, -2))
    keep = torch.ones(S.shape[-2:], dtype=torch.bool)
    if causal:
        sq, skv = Q.shape[2], K.shape[2]
        i = torch.arange(sq)[:, None]; j = torch.arange(skv)[None, :]
        keep = j <= i + (skv - sq)
    # rows that see no key get weights 0 (a finite stand-in score, then masked
    # by multiplication, so no NaN enters the graph)
    has_key = keep.any(dim=-1, keepdim=True)
    S = torch.where(keep | ~has_key, S, torch.full_like(S, float("-inf")))
    P = torch.softmax(S, dim=-1) * has_key
    O = P @ Vr
    (O * G).sum().backward()
    D = q.shape[-1]
    return (Q.grad.reshape(-1, D).numpy(), K.grad.reshape(-1, D).numpy(), V.grad.reshape(-1, D).numpy(),
            O.detach())


def inputs(layout, B, H, sq, skv, seed, D=128):
    q, k, v = wl.random_qkv(layout, B, H, sq, skv, seed, k_factor=2.0, D=D)
    do = wl.random_qkv(layout, B, H, sq, 1, seed + 1000, D=D)[0]
    return q, k, v, do


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("causal,sq,skv", [(False, 23, 41), (True, 37, 37), (True, 20, 53), (True, 41, 17)])
def test_matches_torch_autograd_float64(layout, causal, sq, skv):
    q, k, v, do = inputs(layout, 2, 3, sq, skv, 5)
    g = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                             causal=causal)
    dq, dk, dv, _ = autograd_grads(q, k, v, do, layout, SCALE, causal)
    for got, ref in ((g.dq, dq), (g.dk, dk), (g.dv, dv)):
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-12), np.abs(got - ref).max()


@pytest.mark.parametrize("layout,hkv,causal", [("bhsd", 1, False), ("bshd", 2, True), ("bhsd", 3, True)])
def test_grouped_heads_match_torch_autograd_float64(layout, hkv, causal):
    """Grouped-query heads (6 query heads on hkv key/value heads): dK and dV of
    a key/value head sum over its query heads -- autograd through the
    repeated heads, a derivation independent of the oracle's loops."""
    q, k, v, do = inputs(layout, 2, 6, 29, 35, 13)
    keep = slice(0, hkv)
    k, v = (t[:, :, keep] if layout == "bshd" else t[:, keep] for t in (k, v))
    k, v = k.contiguous(), v.contiguous()
    g = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                             causal=causal)
    dq, dk, dv, _ = autograd_grads(q, k, v, do, layout, SCALE, causal)
    assert g.dk.shape == (2 * hkv * 35, 128)
    for got, ref in ((g.dq, dq), (g.dk, dk), (g.dv, dv)):
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-12), np.abs(got - ref).max()


def test_head_dim_64_matches_autograd():
    q, k, v, do = inputs("bhsd", 1, 2, 30, 45, 7, D=64)
    s = float(np.float32(0.125))
    g = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout="bhsd", scale=s)
    dq, dk, dv, _ = autograd_grads(q, k, v, do, "bhsd", s, False)
    for got, ref in ((g.dq, dq), (g.dk, dk), (g.dv, dv)):
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_single_key_closed_form():
    q, k, v, do = inputs("bhsd", 1, 2, 9, 1, 11)
    g = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout="bhsd", scale=SCALE)
    assert np.all(np.abs(g.dq) < 1e-15) and np.all(np.abs(g.dk) < 1e-15)
    assert np.allclose(g.dv, f64(do).sum(dim=2).reshape(-1, 128).numpy(), rtol=1e-15, atol=1e-15)


def test_given_output_changes_only_delta():
    """With o given (the exact output rounded to bf16), dv is unchanged and
    dq, dk move by exactly the delta correction: with e_i = <dO_i, o_i - O_i>,
    dq_i -= scale e_i sum_j p_ij k_j and dk_j -= scale sum_i e_i p_ij q_i."""
    layout, B, H, sq, skv = "bshd", 1, 2, 19, 33
    q, k, v, do = inputs(layout, B, H, sq, skv, 13)
    exact = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE)
    fwd = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=SCALE, method=False)
    o_bits = fwd.rounded("rtne").reshape(B, H, sq, 128).transpose(0, 2, 1, 3).copy()   # [B,S,H,D] bits
    given = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                                 o=o_bits)
    assert np.array_equal(given.dv, exact.dv)
    Q, K, G = (heads_first(f64(t), layout) for t in (q, k, do))
    P = torch.softmax(SCALE * (Q @ K.transpose(-1, -2)), dim=-1)
    O = P @ heads_first(f64(v), layout)
    Og = heads_first(f64(torch.from_numpy(oracle.bf16_bits_to_f64(o_bits))), layout)
    e = ((Og - O) * G).sum(-1, keepdim=True)                     # [B,H,Sq,1]
    ddq = -SCALE * e * (P @ K)
    ddk = -SCALE * (P * e).transpose(-1, -2) @ Q
    assert np.allclose(given.dq - exact.dq, ddq.reshape(-1, 128).numpy(), rtol=1e-9, atol=1e-14)
    assert np.allclose(given.dk - exact.dk, ddk.reshape(-1, 128).numpy(), rtol=1e-9, atol=1e-14)
    assert np.abs(given.dq - exact.dq).max() > 0


# ------------------------------------------------- the sigmas of the gradients
# Each gradient element is a sum of terms (dq_id: scale ds_ij k_jd over keys j;
# dk_jd: scale ds_ij q_id over queries i of every query head of the group;
# dv_jd: p_ij do_id), and the oracle returns next to it the RMS size of those
# terms, sqrt(sum of squares), which sets the ULP floor of the backward gate.
# Two pins independent of the oracle's loops: float64 matrix products of the
# squared factors, and 50-digit decimal brute force on tiny shapes.
def reference_grad_sigmas(q, k, v, do, layout, scale, causal):
    """sdq, sdk, sdv as matrix products of squares (torch float64):
    sdq = |scale| sqrt(dS^2 K^2), sdk = |scale| sqrt(sum_group dS^2T Q^2),
    sdv = sqrt(sum_group P^2T dO^2)."""
    Q, K, V, G = (heads_first(f64(t), layout) for t in (q, k, v, do))
    group = Q.shape[1] // K.shape[1]
    Kr, Vr = K.repeat_interleave(group, dim=1), V.repeat_interleave(group, dim=1)
    S = scale * (Q @ Kr.transpose(-1, -2))
    sq, skv = Q.shape[2], K.shape[2]
    keep = torch.ones(sq, skv, dtype=torch.bool)
    if causal:
        i = torch.arange(sq)[:, None]; j = torch.arange(skv)[None, :]
        keep = j <= i + (skv - sq)
    has_key = keep.any(dim=-1, keepdim=True)
    S = torch.where(keep | ~has_key, S, torch.full_like(S, float("-inf")))
    P = torch.softmax(S, dim=-1) * has_key
    O = P @ Vr
    delta = (G * O).sum(-1, keepdim=True)
    dP = G @ Vr.transpose(-1, -2)
    dS = P * (dP - delta)
    sdq = abs(scale) * torch.sqrt((dS * dS) @ (Kr * Kr))
    B, Hq, _, D = Q.shape
    Hk = K.shape[1]
    sk2 = ((dS * dS).transpose(-1, -2) @ (Q * Q)).reshape(B, Hk, group, skv, D).sum(2)
    sv2 = ((P * P).transpose(-1, -2) @ (G * G)).reshape(B, Hk, group, skv, D).sum(2)
    return (sdq.reshape(-1, D).numpy(), (abs(scale) * torch.sqrt(sk2)).reshape(-1, D).numpy(),
            torch.sqrt(sv2).reshape(-1, D).numpy())


@pytest.mark.parametrize("layout,H,hkv,causal,sq,skv", [("bhsd", 3, 3, False, 23, 41), ("bshd", 3, 3, True, 37, 37),
                                                        ("bshd", 6, 2, True, 29, 35), ("bhsd", 4, 1, False, 19, 50)])
def test_gradient_sigmas_match_float64_products(layout, H, hkv, causal, sq, skv):
    q, k, v, do = inputs(layout, 2, H, sq, skv, 17)
    if hkv != H:
        keep = slice(0, hkv)
        k, v = ((t[:, :, keep] if layout == "bshd" else t[:, keep]).contiguous() for t in (k, v))
    g = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout=layout, scale=SCALE,
                             causal=causal)
    for got, ref in zip((g.sdq, g.sdk, g.sdv), reference_grad_sigmas(q, k, v, do, layout, SCALE, causal)):
        assert got.shape == ref.shape
        assert np.all(np.isfinite(got)) and np.all(got >= 0)
        assert np.allclose(got, ref, rtol=1e-10, atol=1e-300), np.abs(got - ref).max()


def test_gradient_sigmas_scale_with_the_scale_and_dO():
    """sdq and sdk carry |scale| once more than the weights' own dependence,
    sdv does not; doubling dO doubles every gradient and every sigma."""
    q, k, v, do = inputs("bhsd", 1, 2, 15, 21, 23)
    a = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout="bhsd", scale=SCALE)
    do2 = (do.float() * 2).to(torch.bfloat16)
    b = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do2), layout="bhsd", scale=SCALE)
    for x, y in ((a.sdq, b.sdq), (a.sdk, b.sdk), (a.sdv, b.sdv), (a.dq, b.dq), (a.dk, b.dk), (a.dv, b.dv)):
        assert np.allclose(2 * x, y, rtol=1e-13, atol=0)


def decimal_grads(Q, K, V, G, scale):
    """dq, sdq, dk, sdk, dv, sdv of one head by the chain rule in 50-digit
    decimal arithmetic (exact rational scores)."""
    from decimal import Decimal, getcontext
    from fractions import Fraction
    getcontext().prec = 50
    sq, skv, D = Q.shape[0], K.shape[0], Q.shape[1]
    dec = lambda x: Decimal(x.numerator) / Decimal(x.denominator) if isinstance(x, Fraction) else Decimal(float(x))
    sc = Fraction(float(np.float32(scale)))
    P = []
    for i in range(sq):
        s = [sc * sum(Fraction(float(Q[i, d])) * Fraction(float(K[j, d])) for d in range(D)) for j in range(skv)]
        m = max(s)
        e = [(dec(x) - dec(m)).exp() for x in s]
        l = sum(e)
        P.append([x / l for x in e])
    O = [[sum(P[i][j] * dec(V[j, d]) for j in range(skv)) for d in range(D)] for i in range(sq)]
    delta = [sum(dec(G[i, d]) * O[i][d] for d in range(D)) for i in range(sq)]
    dS = [[P[i][j] * (sum(dec(G[i, d]) * dec(V[j, d]) for d in range(D)) - delta[i]) for j in range(skv)]
          for i in range(sq)]
    scd = dec(sc)
    out = {n: np.zeros((sq if n in ("dq", "sdq") else skv, D)) for n in ("dq", "sdq", "dk", "sdk", "dv", "sdv")}
    for d in range(D):
        for i in range(sq):
            t = [scd * dS[i][j] * dec(K[j, d]) for j in range(skv)]
            out["dq"][i, d] = float(sum(t)); out["sdq"][i, d] = float(sum(x * x for x in t).sqrt())
        for j in range(skv):
            tk = [scd * dS[i][j] * dec(Q[i, d]) for i in range(sq)]
            tv = [P[i][j] * dec(G[i, d]) for i in range(sq)]
            out["dk"][j, d] = float(sum(tk)); out["sdk"][j, d] = float(sum(x * x for x in tk).sqrt())
            out["dv"][j, d] = float(sum(tv)); out["sdv"][j, d] = float(sum(x * x for x in tv).sqrt())
    return out


@pytest.mark.parametrize("sq,skv", [(2, 3), (3, 2), (1, 3)])
def test_gradients_and_sigmas_bruteforce_decimal(sq, skv):
    q, k, v, do = inputs("bhsd", 1, 1, sq, skv, 31, D=128)
    g = oracle.attention_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), layout="bhsd", scale=SCALE)
    Q, K, V, G = (oracle.bf16_bits_to_f64(wl.bits(t))[0, 0] for t in (q, k, v, do))
    ref = decimal_grads(Q, K, V, G, SCALE)
    for name in ("dq", "dk", "dv"):
        got, sig = getattr(g, name), ref["s" + name]
        # the gradients cancel; compare against the size of their terms
        assert np.all(np.abs(got - ref[name]) <= 1e-12 * sig + 1e-300), name
        assert np.allclose(getattr(g, "s" + name), sig, rtol=1e-12, atol=0), "s" + name
