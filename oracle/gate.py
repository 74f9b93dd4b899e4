"""Accuracy gate between a bf16 result and the fp64 oracle -- TEST INFRASTRUCTURE.

The stated bound is "within 2 bf16 ULP of the fp64 oracle for every finite
element, within 1 ULP for at least 99.9% of them, NaN/Inf positions
identical".  Read literally (ULP of each exact output value) it cannot be
met by any kernel that feeds bf16 probabilities into the p.V product:
outputs that cancel to near zero have a tiny ULP while the bf16 rounding of
the weights perturbs them by about 2^-9 of the terms being summed.  The
reading used here takes the ULP at the larger of |o| and a multiple f of the
RMS size sigma of those terms:

    D = |g - round(o)| / ulp_bf16(max(|o|, f sigma))

with ulp_bf16(x) = 2^(max(floor(log2 x), -126) - 7).  This floor is not a
rare correction.  An attention output is a weighted mean of many values of
both signs, so |o| is typically of the order of sigma.  Measured with the
oracle on the workloads' input recipes (N(0,1)-type Q, K, V; 128 to 4096
keys), the definition gate's floor (f = 2) governs 95-97% of the elements.
It widens the median element's ULP unit 2-4 times over the literal one
(16 times at the 90th percentile).  On those elements the gate reads as an
absolute bound of 1-2 ULP of 2 sigma, not as a relative one.  Where
|o| >= 2 sigma (3-5% of elements) D is the literal ULP distance.  The
tests pin these shares (tests/test_gate.py).

So every forward parity test also applies a second, tighter gate.  It
compares against the oracle's method companion: the same operation with
the weights rounded to bf16 the way the kernel rounds them, normalised by
the sum of those rounded weights.  Its floor is f = 1 times that
companion's sigma, and it governs about two thirds of the elements.  What
separates the kernel from the companion is fp32 accumulation order and rare
weights whose fp32 exponential rounds to the other bf16 neighbour, so that
gate also holds it to D <= 2 everywhere and D <= 1 for >= 99.9%.  The
literal distance in bf16 steps is reported as well.
"""
from __future__ import annotations

import numpy as np

from . import bf16_bits_to_f64, round_bf16


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 values in the binade of |x| (subnormal spacing below 2^-126)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(np.maximum(e, -126.0) - 7.0)


def ordinal(bits) -> np.ndarray:
    """Monotone integer ordering of bf16 bit patterns (+0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def compare(gpu_bits, o_exact, sigma, mode: str, floor_factor: float = 2.0) -> dict:
    """Gate statistics for one output tensor.

    gpu_bits: uint16 [n, D] bf16 patterns from the device.
    o_exact, sigma: float64 [n, D] from the oracle (same rows).
    """
    g_bits = np.asarray(gpu_bits, dtype=np.uint16)
    g = bf16_bits_to_f64(g_bits)
    o = np.asarray(o_exact, dtype=np.float64)
    s = np.asarray(sigma, dtype=np.float64)
    r_bits = round_bf16(o, mode)
    r = bf16_bits_to_f64(r_bits)

    g_nan, r_nan = np.isnan(g), np.isnan(r)
    g_pinf, r_pinf = np.isposinf(g), np.isposinf(r)
    g_ninf, r_ninf = np.isneginf(g), np.isneginf(r)
    nonfinite_match = bool(np.array_equal(g_nan, r_nan) and np.array_equal(g_pinf, r_pinf)
                           and np.array_equal(g_ninf, r_ninf))
    fin = np.isfinite(g) & np.isfinite(r)
    out = {"n": int(g.size), "n_finite": int(fin.sum()), "nonfinite_match": nonfinite_match,
           "n_nan": int(r_nan.sum()), "n_inf": int((r_pinf | r_ninf).sum())}
    if fin.any():
        denom = ulp_bf16(np.maximum(np.abs(o[fin]), floor_factor * np.where(np.isfinite(s[fin]), s[fin], 0.0)))
        D = np.abs(g[fin] - r[fin]) / denom
        lit = np.abs(ordinal(g_bits[fin]) - ordinal(r_bits[fin]))
        out.update({
            "max_D": float(D.max()),
            "frac_D_gt1": float(np.mean(D > 1.0)),
            "frac_D_gt2": float(np.mean(D > 2.0)),
            "literal_max_steps": int(lit.max()),
            "literal_frac_gt1": float(np.mean(lit > 1)),
        })
    else:
        out.update({"max_D": 0.0, "frac_D_gt1": 0.0, "frac_D_gt2": 0.0,
                    "literal_max_steps": 0, "literal_frac_gt1": 0.0})
    out["passed"] = bool(nonfinite_match and out["max_D"] <= 2.0 and out["frac_D_gt1"] <= 1e-3)
    return out
