"""GPU parity of attn_fwd_bf16_gqa: grouped-query heads and the causal mask
(query i sees keys j <= i + Skv - Sq), against the fp64 oracle, through the
C ABI.  Same bar as the plain path: every finite element within 2 bf16 ULP,
at least 99.9% within 1, NaN/Inf positions identical, rows that see no key
exactly zero."""
import numpy as np
import pytest

from bf16_attention_forward_amd import workloads as wl
from tests.helpers import assert_gates, check, run_hip, run_hip_gqa, say

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")


def assert_gate(st):
    assert_gates(st)


# every row checked; shapes span several query and key tiles with ragged
# tails, the diagonal crossing tiles, and the three Sq / Skv orders
CASES = [
    # layout, B, Hq, Hkv, Sq, Skv, causal
    ("bhsd", 1, 4, 2, 300, 300, True),     # square causal, diagonal inside tiles
    ("bshd", 2, 6, 3, 200, 333, True),     # Sq < Skv: queries are the last positions
    ("bhsd", 1, 2, 1, 333, 130, True),     # Sq > Skv: leading rows see no key
    ("bshd", 1, 2, 2, 600, 100, True),     # a whole query tile sees no key
    ("bhsd", 1, 3, 1, 1, 1, True),         # single query, single key
    ("bhsd", 2, 8, 2, 257, 257, False),    # grouped heads, no mask
    ("bshd", 1, 4, 4, 1000, 77, False),    # plain heads through the grouped entry
    ("bshd", 1, 4, 2, 300, 2000, False),   # grouped heads, keys past 16 tiles: 8-wave work-groups
    ("bshd", 1, 4, 1, 64, 4096, True),     # short query block at the end of a long key range
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}Hq{c[2]}Hkv{c[3]}_{c[4]}x{c[5]}_{'causal' if c[6] else 'full'}")
@pytest.mark.parametrize("mode", MODES)
def test_small_shapes_all_rows(case, mode):
    layout, B, Hq, Hkv, Sq, Skv, causal = case
    say(f"[case] gqa {case} {mode}")
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 200 + Sq + Skv, 1.0, 2.0, 1.0, Hkv=Hkv)
    o = run_hip_gqa(q, k, v, layout, mode, causal=causal)
    st, _ = check(o, q, k, v, layout, mode, label=str(case), causal=causal)
    assert_gate(st)


def test_rows_without_keys_are_exact_zeros():
    layout, B, Hq, Hkv, Sq, Skv = "bshd", 1, 2, 1, 700, 90
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 61, Hkv=Hkv)
    o = run_hip_gqa(q, k, v, layout, "rtne", causal=True).reshape(B, Sq, Hq, 128)
    n_empty = Sq - Skv
    assert np.all(o[:, :n_empty] == 0)
    assert np.all(np.any(o[:, n_empty:] != 0, axis=-1))


def test_grouped_equals_repeated_heads_bitwise():
    """GQA through the kernel equals plain attention on repeated K/V heads."""
    layout, B, Hq, Hkv, S = "bhsd", 1, 8, 2, 320
    q, k, v = wl.random_qkv(layout, B, Hq, S, S, 62, Hkv=Hkv)
    a = run_hip_gqa(q, k, v, layout, "rtne", causal=False)
    rep = lambda t: t.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    b = run_hip(q, rep(k), rep(v), layout, "rtne")    # same planner decision (key split) as a
    assert np.array_equal(a, b)


def test_causal_last_row_equals_unmasked_last_row():
    layout, B, Hq, S = "bshd", 1, 2, 500
    q, k, v = wl.random_qkv(layout, B, Hq, S, S, 63)
    a = run_hip_gqa(q, k, v, layout, "rtne", causal=True).reshape(B, S, Hq, 128)
    b = run_hip(q, k, v, layout, "rtne", kv_splits=1).reshape(B, S, Hq, 128)
    assert np.array_equal(a[:, -1], b[:, -1])


def test_deterministic():
    q, k, v = wl.random_qkv("bshd", 1, 8, 777, 777, 64, Hkv=2)
    outs = [run_hip_gqa(q, k, v, "bshd", "rtne", causal=True) for _ in range(3)]
    assert all(np.array_equal(outs[0], x) for x in outs[1:])


@pytest.mark.parametrize("number", [6, 7])
def test_full_size_causal_workloads_sampled(number):
    """The causal workloads at full size, gated on a seeded row sample that
    includes the first and last rows of every head (one key / all keys)."""
    w = wl.WORKLOADS[number]
    say(f"[case] full-size workload {w.name}")
    q, k, v = wl.make_inputs(w)
    rows = wl.sample_rows(w.B, w.H, w.Sq, n_per_head=4, seed=w.seed)
    res = None
    for mode in w.modes:
        o = run_hip_gqa(q, k, v, w.layout, mode, causal=w.causal)
        st, res = check(o, q, k, v, w.layout, mode, rows=rows, label=w.name, oracle_res=res, causal=w.causal)
        assert_gate(st)


LSE_CASES = [
    # layout, B, Hq, Hkv, Sq, Skv, causal
    ("bhsd", 1, 4, 2, 300, 300, True),
    ("bshd", 1, 2, 1, 333, 130, True),     # leading rows see no key: -inf
    ("bhsd", 1, 2, 2, 300, 1000, False),   # few work items: the planner splits the keys (4-wave groups)
    ("bhsd", 1, 2, 2, 300, 1500, False),   # the same on 8-wave groups (more than 16 key tiles)
    ("bshd", 2, 8, 2, 257, 513, False),
]


@pytest.mark.parametrize("case", LSE_CASES, ids=lambda c: f"{c[0]}_Hq{c[2]}Hkv{c[3]}_{c[4]}x{c[5]}_{'causal' if c[6] else 'full'}")
def test_lse_matches_oracle(case):
    """The log-sum-exp side output against the oracle's fp64 value.  The
    kernel forms it from the bf16-rounded weights (relative error of the
    row sum below 2^-8), so the bound is 2^-8 absolute plus fp32 rounding
    of the result."""
    import torch
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa
    import oracle
    layout, B, Hq, Hkv, Sq, Skv, causal = case
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 300 + Sq, 1.0, 2.0, 1.0, Hkv=Hkv)
    o, lse = attn_fwd_bf16_gqa(q.cuda(), k.cuda(), v.cuda(), layout=layout, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    got = lse.cpu().numpy().reshape(-1).astype(np.float64)
    res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=layout, scale=wl.DEFAULT_SCALE,
                           method=False, causal=causal)
    ref = res.lse
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = np.abs(got[fin] - ref[fin])
    say(f"[lse] {case} max err {err.max():.3e}")
    assert np.all(err <= 2.0 ** -8 + 2.0 ** -20 * np.abs(ref[fin]))
    # the output is unchanged by asking for the statistic
    st, _ = check(wl.bits(o.cpu()), q, k, v, layout, "rtne", label=f"lse {case}", causal=causal)
    assert_gate(st)


def test_causal_nonfinite_values_documented_pattern():
    """Under the causal mask a query tile of 256 rows runs every key below its
    last row's diagonal through the P.V product, with the weights of keys a
    row does not see set to 0.  A non-finite V[j, d] therefore reaches, as
    0 * Inf = NaN, column d of the rows of such a tile that do not see key j
    (the documented limitation; finite inputs are unaffected).  Pinned
    exactly: rows that see j follow the definition's closed form, rows of a
    tile that holds a row seeing j but that do not see it themselves are NaN
    in column d, rows of tiles whose key range ends before j are untouched,
    and everything finite passes the gates."""
    import torch
    layout, B, H, S = "bhsd", 1, 2, 600
    q, k, v = wl.random_qkv(layout, B, H, S, S, 811)
    sites = [(0, 300, 5, float("inf")), (0, 100, 7, float("nan")), (1, 550, 9, float("-inf")),
             (1, 20, 3, float("inf")), (1, 21, 3, float("-inf"))]
    for h, j, d, val in sites:
        v[0, h, j, d] = val
    o = run_hip_gqa(q, k, v, layout, "rtne", causal=True).reshape(B, H, S, 128)
    vals = (o.astype(np.uint32) << 16).view(np.float32)
    off = 0                                    # Skv - Sq
    want = np.zeros((H, S, 128), np.int8)     # 0 finite, 1 NaN, 2 +Inf, 3 -Inf
    for h in range(H):
        for d in range(128):
            col = [(j, val) for (hh, j, dd, val) in sites if hh == h and dd == d]
            if not col:
                continue
            for i in range(S):
                seen = [val for (j, val) in col if j <= i + off]
                tile_end = min(S, (i // 256) * 256 + 256 + off)      # the tile's key range end
                reached = [val for (j, val) in col if j < tile_end and j > i + off]
                if any(np.isnan(x) for x in seen) or (np.inf in seen and -np.inf in seen) or reached:
                    want[h, i, d] = 1
                elif np.inf in seen:
                    want[h, i, d] = 2
                elif -np.inf in seen:
                    want[h, i, d] = 3
    got = np.where(np.isnan(vals), 1, np.where(np.isposinf(vals), 2, np.where(np.isneginf(vals), 3, 0)))[0]
    assert np.array_equal(got, want), f"pattern differs in {(got != want).sum()} places"
    assert (want == 1).sum() > 0 and ((want == 1) & (got == 1)).sum() == (want == 1).sum()
    # rows untouched by any non-finite value pass both gates
    clean = np.where(~np.any(want != 0, axis=2).reshape(-1))[0]
    st, _ = check(o.reshape(-1), q, k, v, layout, "rtne", rows=clean, label="causal nonfinite clean rows",
                  causal=True)
    assert_gate(st)


@pytest.mark.parametrize("layout,mode", [("bshd", "rtne"), ("bhsd", "rtz")])
@pytest.mark.parametrize("Sq,Skv", [(8192, 8192), (8192, 4096)])
def test_causal_persistent_grid_equals_per_entry_calls_bitwise(Sq, Skv, layout, mode):
    """Two batch entries of 6 query heads in 256-row tiles make 384 causal
    blocks, more than one 8-wave work-group per CU: they run on a persistent
    grid that walks the longest-first blocks back in every other round (with
    Sq > Skv the rows above the diagonal, placed last, take the no-key path
    inside the loop).  One entry alone is 192 blocks, one per work-group.
    Every row's arithmetic is the same either way, so the bits are too."""
    B, Hq, Hkv = 2, 6, 2
    say(f"[case] causal persistent {Sq}x{Skv} {layout} {mode}")
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 64, Hkv=Hkv)
    both = run_hip_gqa(q, k, v, layout, mode, causal=True)
    for b in range(B):
        one = run_hip_gqa(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(),
                          layout, mode, causal=True)
        assert np.array_equal(both[b:b + 1], one)
    if Sq > Skv:
        rows = both[:, :Sq - Skv] if layout == "bshd" else both[:, :, :Sq - Skv]
        assert np.all(rows == 0)
