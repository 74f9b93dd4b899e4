"""Pins for the oracle's fp64 -> bf16 rounding (all three modes).

The pages name the three output rounding modes (RTNE, RTNA, RTZ) without
defining them; the reading is the IEEE 754 one: ties-to-even, ties-away-from
zero, toward zero.  The oracle rounds by arithmetic on the exponent and the
scaled significand.  These tests check it against a different construction:
the full list of bf16 values enumerated from their bit patterns, a bracket
search on that list, and exact fp64 midpoints between neighbours.  torch's
float32 -> bfloat16 cast (round-to-nearest-even) is a library cross-check.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _grid():
    """All non-negative finite bf16 values in increasing order, then 2^128 as
    the overflow neighbour (its pattern 0x7F80 has an even last bit)."""
    pats = np.arange(0x0000, 0x7F80, dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(pats)
    assert np.all(np.diff(vals) > 0)
    return np.append(vals, 2.0 ** 128), np.append(pats, np.uint16(0x7F80))


GRID, GRID_PATS = _grid()


def reference_round(x: np.ndarray, mode: str) -> np.ndarray:
    """Bracket-search rounding on the enumerated grid (independent of the oracle)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    sign = np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    a = np.abs(np.where(nan, 0.0, x))
    inf = np.isinf(a)
    a_clip = np.where(inf, 0.0, a)
    # lo = largest grid value <= a (grid[0] = 0 <= a always)
    idx = np.searchsorted(GRID, a_clip, side="right") - 1
    idx = np.minimum(idx, len(GRID) - 1)
    beyond = a_clip >= GRID[-1]          # >= 2^128
    idx_hi = np.minimum(idx + 1, len(GRID) - 1)
    lo, hi = GRID[idx], GRID[idx_hi]
    lo_p, hi_p = GRID_PATS[idx], GRID_PATS[idx_hi]
    exact = a_clip == lo
    mid = (lo + hi) / 2.0                # exact: neighbours have <= 9 significant bits
    if mode == "rtz":
        pick = lo_p.copy()
        pick = np.where(beyond | (lo_p == 0x7F80), np.uint16(0x7F7F), pick)
    elif mode == "rtne":
        up = (a_clip > mid) | ((a_clip == mid) & ((lo_p & 1) == 1))
        pick = np.where(exact, lo_p, np.where(up, hi_p, lo_p))
        pick = np.where(beyond, np.uint16(0x7F80), pick)
    elif mode == "rtna":
        up = a_clip >= mid
        pick = np.where(exact, lo_p, np.where(up, hi_p, lo_p))
        pick = np.where(beyond, np.uint16(0x7F80), pick)
    else:
        raise ValueError(mode)
    out = (pick | sign).astype(np.uint16)
    out = np.where(inf, (np.uint16(0x7F80) | sign).astype(np.uint16), out)
    out = np.where(nan, np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


def _test_values():
    fin = GRID[:-1]
    mids = (fin[:-1] + fin[1:]) / 2.0
    top_mid = (fin[-1] + 2.0 ** 128) / 2.0
    mids = np.append(mids, top_mid)
    up = np.nextafter(mids, np.inf)
    dn = np.nextafter(mids, -np.inf)
    rng = np.random.default_rng(7)
    rnd = rng.standard_normal(50000) * np.exp2(rng.integers(-140, 130, 50000))
    special = np.array([0.0, 2.0 ** -134, 2.0 ** -135, 3 * 2.0 ** -134, 2.0 ** -133, 2.0 ** -126,
                        2.0 ** -126 - 2.0 ** -134, 2.0 ** 128, 2.0 ** 129, 1e300, 5e-324,
                        np.inf, np.nan, fin[-1], top_mid, np.nextafter(top_mid, 0.0)])
    vals = np.concatenate([fin, mids, up, dn, rnd, special])
    return np.concatenate([vals, -vals])


@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
def test_round_matches_grid_search(mode):
    x = _test_values()
    got = oracle.round_bf16(x, mode)
    ref = reference_round(x, mode)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{mode}: {bad.size} mismatches, first x={x[bad[:5]]} got={got[bad[:5]]} ref={ref[bad[:5]]}"


@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
def test_every_bf16_value_is_fixed_point(mode):
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f64(pats)
    keep = ~np.isnan(vals)
    got = oracle.round_bf16(vals[keep], mode)
    assert np.array_equal(got, pats[keep])


def test_rtne_matches_torch_for_float32_inputs():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(f32.astype(np.float64), "rtne")
    assert np.array_equal(got, ref)


def test_tie_cases_distinguish_modes():
    # 1 + 2^-8 lies halfway between bf16 1.0 (0x3F80) and 1.0078125 (0x3F81)
    x = 1.0 + 2.0 ** -8
    assert oracle.round_bf16([x], "rtne")[0] == 0x3F80
    assert oracle.round_bf16([x], "rtna")[0] == 0x3F81
    assert oracle.round_bf16([x], "rtz")[0] == 0x3F80
    assert oracle.round_bf16([-x], "rtna")[0] == 0xBF81
    # just below the tie: all nearest modes go down; just above: up (RTZ always down)
    assert oracle.round_bf16([np.nextafter(x, 0)], "rtna")[0] == 0x3F80
    assert oracle.round_bf16([np.nextafter(x, 2)], "rtne")[0] == 0x3F81
    assert oracle.round_bf16([np.nextafter(x, 2)], "rtz")[0] == 0x3F80


def test_overflow_and_nonfinite():
    big = 2.0 ** 128
    mx = float(oracle.bf16_bits_to_f64([0x7F7F])[0])
    assert oracle.round_bf16([big], "rtz")[0] == 0x7F7F
    assert oracle.round_bf16([big], "rtne")[0] == 0x7F80
    assert oracle.round_bf16([-big], "rtna")[0] == 0xFF80
    halfway = (mx + big) / 2
    assert oracle.round_bf16([halfway], "rtne")[0] == 0x7F80
    assert oracle.round_bf16([np.nextafter(halfway, 0)], "rtne")[0] == 0x7F7F
    assert oracle.round_bf16([np.inf], "rtz")[0] == 0x7F80
    assert oracle.round_bf16([-np.inf], "rtz")[0] == 0xFF80
    assert oracle.round_bf16([np.nan], "rtne")[0] == 0x7FC0
    assert oracle.round_bf16([-0.0], "rtne")[0] == 0x8000
