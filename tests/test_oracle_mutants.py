"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a textual edit of oracle/attn_oracle.c (a dropped term, a
wrong sign, a wrong index or operand, a layout or tie-rule slip), compiled
into a temporary library on the CPU and swapped in for the duration of the
check.  The real oracle source is never modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_attention as A
from tests import test_oracle_round as R

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "qk_index_shift": ("acc += qq[d] * kk[d];", "acc += qq[d] * kk[(d + 1) % D];"),
    "exp_sign": ("double p = exp(s[j] - m);", "double p = exp(m - s[j]);"),
    "no_normalise": ("oe[d] = num[d] / l;", "oe[d] = num[d];"),
    "no_scale": ("s[j] = sc * acc;", "s[j] = acc;"),
    "bshd_offset": ("if (layout == OR_LAYOUT_BSHD) return ((b * S + i) * H + h) * D;",
                    "if (layout == OR_LAYOUT_BSHD) return ((b * H + h) * S + i) * D;"),
    "bwd_no_delta": ("dr[j] = pr[j] * (dp - delta);", "dr[j] = pr[j] * dp;"),
    "bwd_dv_from_ds": ("const double tv = pw * bf16_to_double(gp[d]);", "const double tv = w * bf16_to_double(gp[d]);"),
    "row_stride_128": ("    return ((b * H + h) * S + i) * D;", "    return ((b * H + h) * S + i) * 128;"),
    "value_from_key": ("const uint16_t* vp = v + row_offset(layout, b, hk, j, Hkv, Skv, D);",
                       "const uint16_t* vp = k + row_offset(layout, b, hk, j, Hkv, Skv, D);"),
    "sigma_not_squared": ("sq[d] += (p * vv) * (p * vv);", "sq[d] += (p * vv);"),
    "rtne_tie_up": ("if (fr > 0.5) m = fl + 1.0;", "if (fr >= 0.5) m = fl + 1.0;"),
    "rtna_tie_down": ("if (fr >= 0.5) m = fl + 1.0;\n    } /* OR_RTZ", "if (fr > 0.5) m = fl + 1.0;\n    } /* OR_RTZ"),
    "rtz_overflow_inf": ("return (mode == OR_RTZ) ? (uint16_t)(sign | 0x7F7F)", "return (mode == OR_RTZ) ? (uint16_t)(sign | 0x7F80)"),
    "subnormal_flush": ("if (e < -126) e = -126;", "if (e < -126) return sign;"),
    "max_skips_last_key": ("for (int64_t j = 0; j < n_keys; j++) {\n                const uint16_t* kp",
                           "for (int64_t j = 0; j < n_keys; j++) {\n                if (j == n_keys - 1 && n_keys > 1) { s[j] = -INFINITY; continue; }\n                const uint16_t* kp"),
    "gqa_head_modulo": ("int64_t hk = h / group;", "int64_t hk = h % Hkv;"),
    "causal_off_by_one": ("\n                n_keys = i + (Skv - Sq) + 1;", "\n                n_keys = i + (Skv - Sq);"),
    "causal_top_left": ("\n                n_keys = i + (Skv - Sq) + 1;", "\n                n_keys = i + 1;"),
    "bwd_gqa_head_modulo": ("const int64_t kvh = h / group;", "const int64_t kvh = h % Hkv;"),
    "bwd_causal_off_by_one": ("\n                    n_keys = i + (Skv - Sq) + 1;", "\n                    n_keys = i + (Skv - Sq);"),
    "empty_rows_not_zero": ("if (n_keys <= 0) {", "if (n_keys < 0) {"),
    "lse_drops_max": ("if (lse) lse[t] = m + log(l);", "if (lse) lse[t] = log(l);"),
    "weights_mode_ignored": ("pt = round_trip_bf16(pm, p_round);", "pt = round_trip_bf16(pm, OR_RTNE);"),
    # the sigmas that set the gates' ULP floors
    "bwd_sdk_unsquared": ("gk[d] += tk; sk[d] += tk * tk;", "gk[d] += tk; sk[d] += tk;"),
    "bwd_sdq_no_scale": ("sg[d] += t * t;", "sg[d] += (t / sc) * (t / sc);"),
    "bwd_sdv_from_ds": ("gv[d] += tv; sv[d] += tv * tv;", "gv[d] += tv; sv[d] += tk * tk;"),
    "sigma_method_from_unrounded": ("sqm[d] += (pt * vv) * (pt * vv);", "sqm[d] += (pm * vv) * (pm * vv);"),
    "sigma_method_unnormalised": ("if (sm) sm[d] = sqrt(sqm[d]) / L;", "if (sm) sm[d] = sqrt(sqm[d]);"),
}


def pins():
    """(name, callable) for every pin; each raises AssertionError on failure."""
    out = []
    for mode in ("rtne", "rtna", "rtz"):
        out.append((f"round_grid_{mode}", lambda m=mode: R.test_round_matches_grid_search(m)))
    out.append(("round_torch", R.test_rtne_matches_torch_for_float32_inputs))
    out.append(("round_ties", R.test_tie_cases_distinguish_modes))
    out.append(("round_overflow", R.test_overflow_and_nonfinite))
    for skv in (1, 3):
        out.append((f"brute_{skv}", lambda s=skv: A.test_bruteforce_decimal(s, 1)))
    for lay in ("bshd", "bhsd"):
        out.append((f"sdpa_{lay}", lambda l=lay: A.test_matches_torch_sdpa_float64(l)))
    out.append(("single_key", A.test_single_key_returns_value_row))
    out.append(("equal_scores", lambda: A.test_equal_scores_return_exact_mean("zero_q")))
    out.append(("one_hot", lambda: A.test_one_hot_dominant_score_selects_row(40)))
    out.append(("identity", A.test_identity_values_give_softmax_weights))
    out.append(("permutation", A.test_joint_key_value_permutation_invariance))
    out.append(("layouts", A.test_layouts_agree_bitwise))
    for lay in ("bhsd", "bshd"):
        out.append((f"nonfinite_{lay}", lambda l=lay: A.test_nonfinite_positions_closed_form(l)))
    out.append(("gqa_repeat", lambda: A.test_gqa_equals_mha_on_repeated_heads("bshd", 6, 2)))
    for sq, skv in ((37, 37), (20, 53), (53, 20)):
        out.append((f"causal_sdpa_{sq}x{skv}", lambda a=sq, b=skv: A.test_causal_matches_torch_sdpa_float64(a, b)))
    out.append(("causal_brute", lambda: A.test_causal_bruteforce_decimal(4, 3)))
    out.append(("causal_first_row", A.test_causal_first_query_sees_only_first_key))
    out.append(("lse_torch", lambda: A.test_lse_matches_torch_logsumexp(True)))
    out.append(("lse_closed", A.test_lse_closed_forms))
    for mode in ("rtna", "rtz"):
        out.append((f"weights_{mode}", lambda m=mode: A.test_method_weights_rounded_in_mode(m)))
    out.append(("d64_sdpa", lambda: A.test_d64_matches_torch_sdpa_float64("bhsd", False, 3)))
    out.append(("d64_brute", lambda: A.test_d64_bruteforce_decimal(3)))
    out.append(("d64_pad", A.test_d64_equals_d128_zero_padded))
    from tests import test_oracle_backward as BW
    out.append(("bwd_autograd", lambda: BW.test_matches_torch_autograd_float64("bhsd", False, 23, 41)))
    out.append(("bwd_single_key", BW.test_single_key_closed_form))
    out.append(("bwd_causal", lambda: BW.test_matches_torch_autograd_float64("bshd", True, 37, 37)))
    out.append(("bwd_gqa", lambda: BW.test_grouped_heads_match_torch_autograd_float64("bshd", 2, True)))
    out.append(("bwd_sigmas", lambda: BW.test_gradient_sigmas_match_float64_products("bshd", 6, 2, True, 29, 35)))
    out.append(("bwd_brute", lambda: BW.test_gradients_and_sigmas_bruteforce_decimal(2, 3)))
    out.append(("sigma_method", lambda: A.test_method_companion_and_its_sigma_rebuilt("rtne", True)))
    out.append(("sigma_bounds", A.test_sigma_bounds_the_output))
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    str(mpath), "-o", str(so), "-lm"], check=True)
    lib = oracle.configure(ctypes.CDLL(str(so)))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = []
    for pin_name, fn in pins():
        try:
            with np.errstate(all="ignore"):
                fn()
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin_name)
    assert caught, f"mutant {name} passed every pin"
