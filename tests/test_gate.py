"""The accuracy gate's documented reading, pinned on the oracle alone.

oracle/gate.py states how often the ULP floor of the definition gate
governs (the floor is max(|o|, 2 sigma)) and by how much it widens the ULP
unit on the workloads' input recipes.  These tests recompute those shares
so the description cannot drift from what the gate does.  They also check
the gate's arithmetic on constructed cases.
"""
import numpy as np
import pytest

import oracle
from oracle import gate
from bf16_attention_forward_amd import workloads as wl


@pytest.mark.parametrize("number,sq,skv", [(1, 128, 128), (2, 256, 1024), (3, 256, 1024)])
def test_floor_share_matches_the_documented_reading(number, sq, skv):
    w = wl.WORKLOADS[number]
    q, k, v = wl.make_inputs(w, B=1, H=min(w.H, 2), Sq=sq, Skv=skv)
    res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout=w.layout, scale=wl.DEFAULT_SCALE,
                           method=True, l_from_rounded=True)
    o, s = res.o_exact, res.sigma
    share = float(np.mean(2 * s > np.abs(o)))
    widen = gate.ulp_bf16(np.maximum(np.abs(o), 2 * s)) / gate.ulp_bf16(o)
    assert 0.94 <= share <= 0.98, share
    assert 2.0 <= float(np.median(widen)) <= 4.0
    # the method gate's floor (1 x the companion's sigma) governs about two thirds
    share_m = float(np.mean(res.sigma_method > np.abs(res.o_method)))
    assert 0.55 <= share_m <= 0.8, share_m


def test_literal_elements_use_their_own_ulp():
    """Where |o| >= f sigma the gate is the literal ULP distance: one bf16 step
    of 1.5 is 2^-7, and a result one step away reads D = 1."""
    o = np.array([[1.5, -3.0, 0.0078125]])
    sig = np.zeros_like(o)
    exact_bits = oracle.round_bf16(o, "rtne")
    st = gate.compare(exact_bits, o, sig, "rtne")
    assert st["max_D"] == 0 and st["passed"]
    off = exact_bits.copy()
    off[0, 0] += 1                      # 1.5 -> 1.5078125
    st = gate.compare(off, o, sig, "rtne")
    assert st["max_D"] == 1.0 and st["literal_max_steps"] == 1
    off[0, 1] += 3                      # three steps away
    st = gate.compare(off, o, sig, "rtne")
    assert st["max_D"] == 3.0 and not st["passed"]


def test_floor_widens_the_unit_near_zero():
    """An exact output of 1e-4 with sigma 0.5: the unit is ulp(1.0) = 2^-7, so
    a result of 0 (about 1e-4 off, hundreds of literal steps) reads D < 1."""
    o = np.array([[1e-4]])
    st = gate.compare(np.zeros((1, 1), np.uint16), o, np.array([[0.5]]), "rtne")
    assert st["max_D"] < 0.02 and st["literal_max_steps"] > 100
    st1 = gate.compare(np.zeros((1, 1), np.uint16), o, np.array([[0.0]]), "rtne")
    assert st1["max_D"] > 100


def test_nonfinite_positions_must_match():
    o = np.array([[np.nan, np.inf, -np.inf, 1.0]])
    bits = oracle.round_bf16(o, "rtne")
    assert gate.compare(bits, o, np.zeros_like(o), "rtne")["nonfinite_match"]
    swapped = bits.copy()
    swapped[0, 1], swapped[0, 2] = bits[0, 2], bits[0, 1]
    st = gate.compare(swapped, o, np.zeros_like(o), "rtne")
    assert not st["nonfinite_match"] and not st["passed"]
