"""Pins for the fp64 attention oracle.

The pages print no worked example, so the oracle is pinned against things
the mathematics fixes (the definition is the fused softmax(Q K^T scale) V of
the MoonMath AI MI300X attention article's opening paragraphs):

- brute force in 50-digit decimal arithmetic on tiny inputs (exact rational
  scores, decimal exp), for the output and for sigma;
- a library routine that reduces to the same definition:
  torch.nn.functional.scaled_dot_product_attention in float64 on the CPU;
- closed forms: Skv = 1 returns V's row; constant V returns the constant;
  equal scores (Q = 0 or scale = 0) return the exact mean of V; a score gap
  above 800 nats returns the dominant key's V row bit for bit; V = identity
  returns the softmax weights, which sum to one;
- invariances: a joint permutation of the key/value rows, BSHD vs BHSD
  storage of the same data, additivity in V over disjoint supports;
- the NaN/Inf pattern implied by IEEE arithmetic on the definition,
  computed in closed form from the injection sites.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bf16_attention_forward_amd import workloads as wl

SCALE = wl.DEFAULT_SCALE


def bf(x) -> np.ndarray:
    """float array -> bf16 bit patterns (torch's RTNE cast)."""
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def run(q, k, v, layout="bhsd", scale=SCALE, **kw):
    return oracle.attention(q, k, v, layout=layout, scale=scale, **kw)


# ---------------------------------------------------------------- brute force
def decimal_attention_row(qrow, K, V, scale):
    """Definition evaluated with exact rationals and 50-digit decimal exp."""
    getcontext().prec = 50
    qf = [Fraction(float(x)) for x in qrow]
    sc = Fraction(float(np.float32(scale)))
    s = []
    for j in range(K.shape[0]):
        s.append(sc * sum(qf[d] * Fraction(float(K[j, d])) for d in range(len(qf))))
    m = max(s)
    p = [(Decimal(x.numerator) / Decimal(x.denominator) - Decimal(m.numerator) / Decimal(m.denominator)).exp() for x in s]
    l = sum(p)
    o, sg = [], []
    for d in range(V.shape[1]):
        num = sum(p[j] * Decimal(float(V[j, d])) for j in range(K.shape[0]))
        sq = sum((p[j] * Decimal(float(V[j, d]))) ** 2 for j in range(K.shape[0]))
        o.append(num / l)
        sg.append(sq.sqrt() / l)
    return np.array([float(x) for x in o]), np.array([float(x) for x in sg])


@pytest.mark.parametrize("skv", [1, 2, 3, 5])
@pytest.mark.parametrize("seed", [1, 2])
def test_bruteforce_decimal(skv, seed):
    q, k, v = wl.random_qkv("bhsd", 1, 1, 2, skv, seed, k_factor=2.0)
    qb, kb, vb = wl.bits(q), wl.bits(k), wl.bits(v)
    res = run(qb, kb, vb)
    Q, K, V = f64(qb)[0, 0], f64(kb)[0, 0], f64(vb)[0, 0]
    for i in range(Q.shape[0]):
        o_ref, s_ref = decimal_attention_row(Q[i], K, V, SCALE)
        scale_o = np.maximum(np.abs(o_ref), s_ref) + 1e-300
        assert np.all(np.abs(res.o_exact[i] - o_ref) <= 1e-13 * scale_o + 1e-15 * np.abs(V).max())
        assert np.allclose(res.sigma[i], s_ref, rtol=1e-12, atol=0)


# ------------------------------------------------------------- library routine
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_matches_torch_sdpa_float64(layout):
    q, k, v = wl.random_qkv(layout, 2, 3, 37, 211, 11, k_factor=2.0)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout)
    to_bhsd = (lambda t: t.permute(0, 2, 1, 3)) if layout == "bshd" else (lambda t: t)
    Q, K, V = (to_bhsd(t).to(torch.float64).contiguous() for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=float(SCALE))
    ref = ref.reshape(-1, 128).numpy()   # rows in (b, h, i) order == oracle's flat row ids
    assert np.max(np.abs(res.o_exact - ref)) <= 1e-12 * float(V.abs().max())


# ----------------------------------------------------------------- closed forms
def test_single_key_returns_value_row():
    q, k, v = wl.random_qkv("bshd", 1, 2, 9, 1, 5)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd")
    V = f64(wl.bits(v))            # [1,1,2,128]
    for h in range(2):
        assert np.array_equal(res.o_exact[h * 9:(h + 1) * 9], np.broadcast_to(V[0, 0, h], (9, 128)))
        for mode in ("rtne", "rtna", "rtz"):
            assert np.array_equal(res.rounded(mode)[h * 9:(h + 1) * 9], np.broadcast_to(wl.bits(v)[0, 0, h], (9, 128)))


@pytest.mark.parametrize("c", [1.0, -0.375, 3.140625, 2.0 ** -20])
def test_constant_value_returns_constant(c):
    q, k, _ = wl.random_qkv("bhsd", 1, 1, 7, 50, 6, k_factor=2.0)
    vb = np.full((1, 1, 50, 128), bf([c])[0], dtype=np.uint16)
    res = run(wl.bits(q), wl.bits(k), vb)
    assert np.allclose(res.o_exact, c, rtol=4e-16 * 50, atol=0)
    for mode in ("rtne", "rtna"):
        assert np.all(res.rounded(mode) == bf([c])[0])


@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_equal_scores_return_exact_mean(how):
    skv = 64
    q, k, v = wl.random_qkv("bhsd", 1, 1, 3, skv, 8)
    qb = wl.bits(q).copy()
    scale = SCALE
    if how == "zero_q":
        qb[:] = 0
    else:
        scale = 0.0
    vb = wl.bits(v)
    res = run(qb, wl.bits(k), vb, scale=scale)
    V = f64(vb)[0, 0]
    mean = np.array([float(sum(Fraction(x) for x in V[:, d]) / skv) for d in range(128)])
    assert np.all(np.abs(res.o_exact - mean) <= 1e-15 * np.abs(V).max())
    # the method companion is exact here too (every weight is 1)
    assert np.array_equal(res.o_method, res.o_exact)


def test_equal_scores_tie_rounding():
    # V rows alternate 1 and 1 + 2^-7 -> mean 1 + 2^-8, a tie between two bf16 values
    skv = 8
    qb = np.zeros((1, 1, 1, 128), np.uint16)
    kb = bf(np.ones((1, 1, skv, 128)))
    vals = np.where(np.arange(skv) % 2 == 0, 1.0, 1.0 + 2.0 ** -7)
    vb = bf(np.broadcast_to(vals[None, None, :, None], (1, 1, skv, 128)))
    res = run(qb, kb, vb)
    assert np.all(res.o_exact == 1.0 + 2.0 ** -8)
    assert np.all(res.rounded("rtne") == 0x3F80)
    assert np.all(res.rounded("rtna") == 0x3F81)
    assert np.all(res.rounded("rtz") == 0x3F80)


@pytest.mark.parametrize("j0", [0, 17, 40])
def test_one_hot_dominant_score_selects_row(j0):
    skv = 41
    _, _, v = wl.random_qkv("bhsd", 1, 1, 1, skv, 9)
    qv = np.zeros((1, 1, 1, 128)); qv[..., 0] = 128.0
    kv = np.zeros((1, 1, skv, 128)); kv[0, 0, j0, 0] = 128.0
    kv[0, 0, :, 1] = 1.0   # other scores 0; dominant score 128*128*scale ~ 1448
    res = run(bf(qv), bf(kv), wl.bits(v))
    vb = wl.bits(v)[0, 0, j0]
    assert np.array_equal(res.o_exact[0], f64(vb))
    for mode in ("rtne", "rtna", "rtz"):
        assert np.array_equal(res.rounded(mode)[0], vb)


def test_identity_values_give_softmax_weights():
    skv = 100
    q, k, _ = wl.random_qkv("bhsd", 1, 2, 5, skv, 10, k_factor=2.0)
    vv = np.zeros((1, 2, skv, 128)); vv[0, :, np.arange(skv), np.arange(skv)] = 1.0
    res = run(wl.bits(q), wl.bits(k), bf(vv))
    w = res.o_exact[:, :skv]
    assert np.all(w > 0)
    assert np.all(res.o_exact[:, skv:] == 0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=skv * 2.0 ** -52)
    # ratio of two weights is exp of the score difference (scores from exact products)
    Q = f64(wl.bits(q))[0, 0, 0]; K = f64(wl.bits(k))[0, 0]
    s = np.array([float(sum(Fraction(Q[d]) * Fraction(K[j, d]) for d in range(128)) * Fraction(float(SCALE))) for j in (3, 71)])
    assert np.isclose(w[0, 3] / w[0, 71], np.exp(s[0] - s[1]), rtol=1e-13)


# ------------------------------------------------------------------ invariances
def test_joint_key_value_permutation_invariance():
    q, k, v = wl.random_qkv("bhsd", 1, 2, 6, 77, 12, k_factor=2.0)
    perm = np.random.default_rng(0).permutation(77)
    a = run(wl.bits(q), wl.bits(k), wl.bits(v))
    b = run(wl.bits(q), wl.bits(k)[:, :, perm], wl.bits(v)[:, :, perm])
    assert np.allclose(a.o_exact, b.o_exact, rtol=1e-13, atol=1e-15)
    # a permutation of only K (not V) must change the result
    c = run(wl.bits(q), wl.bits(k)[:, :, perm], wl.bits(v))
    assert not np.allclose(a.o_exact, c.o_exact, rtol=1e-6, atol=1e-6)


def test_layouts_agree_bitwise():
    q, k, v = wl.random_qkv("bshd", 2, 3, 19, 23, 13)
    a = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd")
    perm = lambda t: wl.bits(t.permute(0, 2, 1, 3).contiguous())
    b = run(perm(q), perm(k), perm(v), layout="bhsd")
    assert np.array_equal(a.o_exact, b.o_exact)
    assert np.array_equal(a.sigma, b.sigma)


def test_additive_in_values_over_disjoint_supports():
    q, k, v = wl.random_qkv("bhsd", 1, 1, 4, 30, 14)
    vb = wl.bits(v)
    mask = (np.arange(128) % 3 == 0)
    v1 = np.where(mask, vb, 0).astype(np.uint16)
    v2 = np.where(~mask, vb, 0).astype(np.uint16)
    a = run(wl.bits(q), wl.bits(k), vb).o_exact
    b = run(wl.bits(q), wl.bits(k), v1).o_exact + run(wl.bits(q), wl.bits(k), v2).o_exact
    assert np.array_equal(a, b)   # each column is computed independently of the others


def test_row_subset_matches_full():
    q, k, v = wl.random_qkv("bshd", 2, 2, 11, 13, 15)
    full = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd")
    rows = np.array([0, 5, 21, 43, 12])
    sub = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd", rows=rows)
    assert np.array_equal(sub.o_exact, full.o_exact[rows])


# -------------------------------------------------------------------- NaN / Inf
def closed_form_mask(inj, B, H, Sq, D=128):
    """Expected output class per (b, h, i, d): 0 finite, 1 NaN, 2 +Inf, 3 -Inf."""
    out = np.zeros((B, H, Sq, D), np.int8)
    col = {}
    for (b, h, j, d, val) in inj.v_sites:
        st = col.setdefault((b, h, d), set())
        st.add("nan" if np.isnan(val) else ("+" if val > 0 else "-"))
    for (b, h, d), st in col.items():
        cls = 1 if ("nan" in st or {"+", "-"} <= st) else (2 if "+" in st else 3)
        out[b, h, :, d] = cls
    for (b, h, i, d, val) in inj.q_sites:
        out[b, h, i, :] = 1
    return out


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_nonfinite_positions_closed_form(layout):
    B, H, Sq, Skv = 2, 3, 21, 33
    q, k, v = wl.random_qkv(layout, B, H, Sq, Skv, 16, k_factor=2.0)
    inj = wl.inject_nonfinite(q, v, layout, 16)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout)
    o = res.o_exact.reshape(B, H, Sq, 128)
    got = np.where(np.isnan(o), 1, np.where(np.isposinf(o), 2, np.where(np.isneginf(o), 3, 0)))
    assert np.array_equal(got, closed_form_mask(inj, B, H, Sq))
    assert res.rounded("rtne")[np.isnan(res.o_exact)].tolist() == [0x7FC0] * int(np.isnan(res.o_exact).sum())


# ------------------------------------------------------------- method companion
def test_method_companion_close_to_exact():
    q, k, v = wl.random_qkv("bhsd", 1, 2, 16, 300, 17, k_factor=2.0)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v))
    # bf16 weights carry a relative error of at most 2^-9 each
    assert np.all(np.abs(res.o_method - res.o_exact) <= 2.0 ** -9 * np.sqrt(300) * res.sigma * 1.01 + 1e-300)
    assert not np.array_equal(res.o_method, res.o_exact)


@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
def test_method_weights_rounded_in_mode(mode):
    """Method companion with the weights rounded in a given mode (the reading in
    which the MoonMath article's per-mode speeds come from rounding the weights
    in the loop): with V the identity over the keys and L the sum of the
    rounded weights, o_method is pt_j / sum pt with pt_j = mode(2^(x_j - M)),
    rebuilt here from exact (rational) scores and the grid-search rounding."""
    from tests.test_oracle_round import reference_round
    skv, sq = 100, 3
    q, k, _ = wl.random_qkv("bhsd", 1, 1, sq, skv, 61, k_factor=2.0)
    vv = np.zeros((1, 1, skv, 128)); vv[0, 0, np.arange(skv), np.arange(skv)] = 1.0
    res = run(wl.bits(q), wl.bits(k), bf(vv), method=True, l_from_rounded=True, p_round=mode)
    Q = f64(wl.bits(q))[0, 0]; K = f64(wl.bits(k))[0, 0]
    log2e = 1.4426950408889634
    differs_from_rtne = 0
    for i in range(sq):
        s = np.array([float(sum(Fraction(Q[i, d]) * Fraction(K[j, d]) for d in range(128)) * Fraction(float(SCALE)))
                      for j in range(skv)])
        x = s * log2e
        p = np.exp2(x - np.ceil(x.max()))
        pt = oracle.bf16_bits_to_f64(reference_round(p, mode))
        assert np.allclose(res.o_method[i, :skv], pt / pt.sum(), rtol=1e-14, atol=0)
        assert np.all(res.o_method[i, skv:] == 0)
        differs_from_rtne += int(np.sum(pt != oracle.bf16_bits_to_f64(reference_round(p, "rtne"))))
    # truncation changes most weights; the two nearest modes differ only on
    # exact ties, which fp64 powers of two of these scores never hit
    assert (differs_from_rtne > 0) == (mode == "rtz")


@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
@pytest.mark.parametrize("l_from_rounded", [True, False])
def test_method_companion_and_its_sigma_rebuilt(mode, l_from_rounded):
    """o_method and sigma_method for general V, rebuilt from exact (rational)
    scores, the grid-search rounding of the weights pt_j = mode(2^(x_j - M))
    and plain matrix products: o_method = (pt V) / L and sigma_method =
    sqrt(pt^2 V^2) / L, L = sum pt (l_from_rounded) or sum 2^(x_j - M).
    sigma_method sets the ULP floor of the method gate."""
    from tests.test_oracle_round import reference_round
    sq, skv = 3, 70
    q, k, v = wl.random_qkv("bhsd", 1, 1, sq, skv, 67, k_factor=2.0)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), method=True, l_from_rounded=l_from_rounded, p_round=mode)
    Q, K, V = (f64(wl.bits(t))[0, 0] for t in (q, k, v))
    log2e = 1.4426950408889634
    for i in range(sq):
        s = np.array([float(sum(Fraction(Q[i, d]) * Fraction(K[j, d]) for d in range(128)) * Fraction(float(SCALE)))
                      for j in range(skv)])
        x = s * log2e
        pm = np.exp2(x - np.ceil(x.max()))
        pt = oracle.bf16_bits_to_f64(reference_round(pm, mode))
        L = pt.sum() if l_from_rounded else pm.sum()
        assert np.allclose(res.o_method[i], (pt @ V) / L, rtol=1e-12, atol=1e-14 * np.abs(V).max())
        assert np.allclose(res.sigma_method[i], np.sqrt((pt * pt) @ (V * V)) / L, rtol=1e-12, atol=0)
    # the companion's sigma stays within the weights' rounding of the exact one
    assert np.all(np.abs(res.sigma_method - res.sigma) <= 2.0 ** -7 * res.sigma + 1e-300) or not l_from_rounded


def test_sigma_bounds_the_output():
    """|o_d| <= sqrt(Skv) sigma_d (Cauchy-Schwarz on the sum of Skv terms) and
    sigma_d <= max_j |v_jd| (the weights sum to one), for o and o_method."""
    skv = 50
    q, k, v = wl.random_qkv("bshd", 1, 2, 20, skv, 69, k_factor=2.0)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd", method=True, l_from_rounded=True)
    vmax = np.abs(f64(wl.bits(v))).max(axis=1).reshape(2, 128)           # [h, d]
    for o, sg in ((res.o_exact, res.sigma), (res.o_method, res.sigma_method)):
        assert np.all(np.abs(o) <= np.sqrt(skv) * sg * (1 + 1e-12))
        assert np.all(sg.reshape(2, 20, 128) <= vmax[:, None, :] * (1 + 1e-12))


# ------------------------------------------- grouped-query heads, causal mask
# The pages list causal masking and grouped-query attention as limitations of
# the kernel they describe (MoonMath article, limitations paragraph); the
# oracle's extension is pinned like the plain operation: a library routine
# (SDPA in float64 with an explicit boolean mask), decimal brute force on the
# admissible keys, closed forms, and the identity GQA = MHA on repeated heads.
def repeat_kv_heads(t: np.ndarray, layout: str, group: int) -> np.ndarray:
    """Key/value head h -> query heads h*group .. h*group+group-1."""
    return np.repeat(t, group, axis=2 if layout == "bshd" else 1)


def causal_mask(Sq: int, Skv: int) -> torch.Tensor:
    """Bottom-right aligned: query i sees keys j <= i + Skv - Sq."""
    return torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq)


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("hq,hkv", [(6, 2), (6, 3), (4, 1)])
def test_gqa_equals_mha_on_repeated_heads(layout, hq, hkv):
    q, k, v = wl.random_qkv(layout, 2, hq, 19, 45, 21, k_factor=2.0, Hkv=hkv)
    qb, kb, vb = wl.bits(q), wl.bits(k), wl.bits(v)
    res = run(qb, kb, vb, layout=layout)
    ref = run(qb, repeat_kv_heads(kb, layout, hq // hkv), repeat_kv_heads(vb, layout, hq // hkv), layout=layout)
    assert np.array_equal(res.o_exact, ref.o_exact)
    assert np.array_equal(res.sigma, ref.sigma)


@pytest.mark.parametrize("sq,skv", [(37, 37), (20, 53), (53, 20), (1, 9)])
def test_causal_matches_torch_sdpa_float64(sq, skv):
    layout, B, H, hkv = "bhsd", 1, 4, 2
    q, k, v = wl.random_qkv(layout, B, H, sq, skv, 31, k_factor=2.0, Hkv=hkv)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, causal=True)
    Q = q.to(torch.float64)
    K = torch.repeat_interleave(k.to(torch.float64), H // hkv, dim=1).contiguous()
    V = torch.repeat_interleave(v.to(torch.float64), H // hkv, dim=1).contiguous()
    mask = causal_mask(sq, skv)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=float(SCALE))
    ref = ref.reshape(-1, 128).numpy()
    has_key = np.tile(mask.any(dim=1).numpy(), B * H)
    assert np.max(np.abs(res.o_exact[has_key] - ref[has_key])) <= 1e-12 * float(V.abs().max())
    assert np.all(res.o_exact[~has_key] == 0.0) and np.all(res.sigma[~has_key] == 0.0)


@pytest.mark.parametrize("sq,skv", [(3, 4), (4, 3), (2, 2)])
def test_causal_bruteforce_decimal(sq, skv):
    q, k, v = wl.random_qkv("bhsd", 1, 1, sq, skv, 41, k_factor=2.0)
    qb, kb, vb = wl.bits(q), wl.bits(k), wl.bits(v)
    res = run(qb, kb, vb, causal=True)
    Q, K, V = f64(qb)[0, 0], f64(kb)[0, 0], f64(vb)[0, 0]
    for i in range(sq):
        n = min(skv, i + skv - sq + 1)
        if n <= 0:
            assert np.all(res.o_exact[i] == 0.0)
            continue
        o_ref, s_ref = decimal_attention_row(Q[i], K[:n], V[:n], SCALE)
        scale_o = np.maximum(np.abs(o_ref), s_ref) + 1e-300
        assert np.all(np.abs(res.o_exact[i] - o_ref) <= 1e-13 * scale_o + 1e-15 * np.abs(V).max())
        assert np.allclose(res.sigma[i], s_ref, rtol=1e-12, atol=0)


def test_causal_first_query_sees_only_first_key():
    """Sq == Skv: query 0 has one admissible key, so its output is V's row 0
    exactly, in every rounding mode."""
    q, k, v = wl.random_qkv("bshd", 1, 2, 40, 40, 43, Hkv=1)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd", causal=True)
    V = f64(wl.bits(v))                       # [1, 40, 1, 128]
    for h in range(2):
        assert np.array_equal(res.o_exact[h * 40], V[0, 0, 0])
        for mode in ("rtne", "rtna", "rtz"):
            assert np.array_equal(res.rounded(mode)[h * 40], wl.bits(v)[0, 0, 0])


def test_causal_last_query_sees_every_key():
    """The last query row is unmasked: it equals the plain operation's row."""
    q, k, v = wl.random_qkv("bhsd", 1, 2, 30, 70, 44, k_factor=2.0)
    qb, kb, vb = wl.bits(q), wl.bits(k), wl.bits(v)
    rows = np.array([29, 59])
    a = run(qb, kb, vb, causal=True, rows=rows)
    b = run(qb, kb, vb, causal=False, rows=rows)
    assert np.array_equal(a.o_exact, b.o_exact)


# -------------------------------------------------------------- log-sum-exp
@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_torch_logsumexp(causal):
    layout, B, H, hkv, sq, skv = "bshd", 2, 4, 2, 23, 41
    q, k, v = wl.random_qkv(layout, B, H, sq, skv, 51, k_factor=2.0, Hkv=hkv)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, causal=causal)
    Q = q.to(torch.float64).permute(0, 2, 1, 3)
    K = torch.repeat_interleave(k.to(torch.float64).permute(0, 2, 1, 3), H // hkv, dim=1)
    S = float(SCALE) * (Q @ K.transpose(-1, -2))
    if causal:
        S = S.masked_fill(~causal_mask(sq, skv), float("-inf"))
    ref = torch.logsumexp(S, dim=-1).reshape(-1).numpy()
    assert np.allclose(res.lse, ref, rtol=1e-14, atol=1e-13)


def test_lse_closed_forms():
    # one key: lse is that key's scaled score; equal scores: log(Skv) + score
    q, k, v = wl.random_qkv("bhsd", 1, 1, 5, 1, 52)
    res = run(wl.bits(q), wl.bits(k), wl.bits(v))
    s0 = float(SCALE) * (f64(wl.bits(q))[0, 0] @ f64(wl.bits(k))[0, 0, 0])
    assert np.allclose(res.lse, s0, rtol=1e-15, atol=0)
    q0 = np.zeros((1, 1, 3, 128), np.uint16)
    _, k2, v2 = wl.random_qkv("bhsd", 1, 1, 3, 37, 53)
    res = run(q0, wl.bits(k2), wl.bits(v2))
    assert np.allclose(res.lse, np.log(37.0), rtol=1e-15, atol=0)
    # causal rows that see no key
    q3, k3, v3 = wl.random_qkv("bhsd", 1, 1, 9, 4, 54)
    res = run(wl.bits(q3), wl.bits(k3), wl.bits(v3), causal=True)
    assert np.all(np.isneginf(res.lse[:5])) and np.all(np.isfinite(res.lse[5:]))


# ------------------------------------------------------- head dimension 64
# The HipKittens summary's kernel suite lists attention forward for head
# dimensions 64 and 128; the oracle takes D as a parameter and is pinned at
# D = 64 like at 128: the library routine in float64, brute force in decimal,
# and the identity that zero-padding Q, K, V to 128 dimensions changes no score.
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("causal,hkv", [(False, 3), (True, 1)])
def test_d64_matches_torch_sdpa_float64(layout, causal, hkv):
    B, H, sq, skv = 2, 3, 37, 53
    q, k, v = wl.random_qkv(layout, B, H, sq, skv, 81, k_factor=2.0, Hkv=hkv, D=64)
    scale = float(np.float32(0.125))
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=scale, causal=causal)
    assert res.o_exact.shape == (B * H * sq, 64)
    perm = (0, 2, 1, 3) if layout == "bshd" else (0, 1, 2, 3)
    Q = q.to(torch.float64).permute(*perm)
    K = torch.repeat_interleave(k.to(torch.float64).permute(*perm), H // hkv, dim=1)
    V = torch.repeat_interleave(v.to(torch.float64).permute(*perm), H // hkv, dim=1)
    mask = causal_mask(sq, skv) if causal else None
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    assert np.allclose(res.o_exact, ref.reshape(-1, 64).numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("skv", [1, 3])
def test_d64_bruteforce_decimal(skv):
    q, k, v = wl.random_qkv("bhsd", 1, 1, 2, skv, 82, D=64)
    scale = float(np.float32(0.125))
    res = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=scale)
    Q = f64(wl.bits(q))[0, 0]; K = f64(wl.bits(k))[0, 0]; V = f64(wl.bits(v))[0, 0]
    for i in range(2):
        o_ref, s_ref = decimal_attention_row(Q[i], K, V, scale)
        scale_o = np.maximum(np.abs(o_ref), s_ref) + 1e-300
        assert np.all(np.abs(res.o_exact[i] - o_ref) <= 1e-13 * scale_o + 1e-15 * np.abs(V).max())
        assert np.allclose(res.sigma[i], s_ref, rtol=1e-12, atol=0)


def test_d64_equals_d128_zero_padded():
    q, k, v = wl.random_qkv("bshd", 1, 2, 40, 70, 83, k_factor=2.0, D=64)
    pad = lambda t: torch.nn.functional.pad(t, (0, 64))
    scale = float(np.float32(0.125))
    r64 = run(wl.bits(q), wl.bits(k), wl.bits(v), layout="bshd", scale=scale, method=True)
    r128 = run(wl.bits(pad(q)), wl.bits(pad(k)), wl.bits(pad(v)), layout="bshd", scale=scale, method=True)
    assert np.array_equal(r128.o_exact[:, :64], r64.o_exact) and np.all(r128.o_exact[:, 64:] == 0)
    assert np.array_equal(r128.sigma[:, :64], r64.sigma)
    assert np.array_equal(r128.o_method[:, :64], r64.o_method)
