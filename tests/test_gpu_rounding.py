"""GPU check of the output rounding (RTNE, RTNA, RTZ) bit for bit, on outputs
whose exact value the kernel's fp32 arithmetic reaches exactly.

The MoonMath article's numerics paragraph names three output rounding
modes.  The ULP gates elsewhere allow one step, so they cannot see a mode
that rounds the wrong way on ties or truncates where it should round; this
test can.  With Q = 0 every score is 0, so every weight is 2^0 = 1 exactly,
the row sum is Skv and the output is the plain mean of a V column.  V is
drawn from one binade with bf16's 8 significant bits and Skv = 2^k keys
(k <= 16), so every partial sum is a multiple of the binade's bf16 step
below 2^(k+8) of them: exact in fp32 in any order, and the division by
2^k is exact too.  The kernel's fp32 result is therefore the exact mean,
and its bf16 output must equal the oracle's rounding of the exact mean in
the requested mode, bit for bit.  With 2 keys every mean is either a bf16
value or an exact tie; with 4 and more keys ties, near-ties and plain
values mix.  Both signs and several binades are covered, and both
work-group sizes and the split path are exercised.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from bf16_attention_forward_amd import workloads as wl
from tests.helpers import say, to_dev

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")


def one_binade_values(rng, shape, exps):
    """bf16 values m * 2^(e-7), m in [128, 255], one exponent e (drawn from
    `exps`) per column.  Signs: one per column in even heads (means stay in
    the binade, so with two keys half of them are ties), one per element in
    odd heads (cancellation reaches lower binades)."""
    m = rng.integers(128, 256, size=shape).astype(np.float64)
    e = rng.choice(np.asarray(exps), size=shape[:-2] + (1, shape[-1]))
    col = rng.choice([-1.0, 1.0], size=shape[:-2] + (1, shape[-1]))
    elem = rng.choice([-1.0, 1.0], size=shape)
    odd = (np.arange(shape[1]) % 2 == 1)[None, :, None, None]
    return np.where(odd, elem, col) * m * np.exp2(e - 7.0)


def bf16_tensor(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy().astype(np.float64), np.asarray(x)), "values must be bf16"
    return t


@pytest.mark.parametrize("skv,kw", [(2, {}), (4, {}), (8, {"waves": 8}), (64, {}), (1024, {"kv_splits": 4}),
                                    (256, {"waves": 4})])
def test_exact_means_round_bit_for_bit(skv, kw):
    from bf16_attention_forward_amd import attn_fwd_bf16
    B, H, Sq = 4, 256, 3
    rng = np.random.default_rng(skv)
    v64 = one_binade_values(rng, (B, H, skv, 128), exps=[-20, -3, 0, 1, 7, 30])
    v = bf16_tensor(v64)
    q = torch.zeros((B, H, Sq, 128), dtype=torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, H, skv, 128)).astype(np.float32)).to(torch.bfloat16)
    mean = v64.mean(axis=2)                                    # exact: power-of-two count, bounded bits
    q_d, k_d, v_d = to_dev(q), to_dev(k), to_dev(v)
    ties = 0
    for mode in MODES:
        say(f"[case] exact means skv={skv} {kw} {mode}")
        o = attn_fwd_bf16(q_d, k_d, v_d, layout="bhsd", round_mode=mode, **kw)
        torch.cuda.synchronize()
        g = wl.bits(o.cpu()).reshape(B, H, Sq, 128)
        want = oracle.round_bf16(mean, mode)                    # [B, H, 128]
        bad = g != want[:, :, None, :]
        assert not bad.any(), f"{mode}: {int(bad.sum())} of {bad.size} outputs differ"
        # the oracle's own path agrees with the plain mean (a check of the setup)
        res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=wl.DEFAULT_SCALE,
                               rows=np.arange(0, B * H * Sq, Sq * 37), method=False)
        assert np.array_equal(res.o_exact, mean.reshape(B * H, 128)[::37])
        if mode == "rtne":
            r_up = oracle.bf16_bits_to_f64(oracle.round_bf16(mean, "rtna"))
            r_dn = oracle.bf16_bits_to_f64(oracle.round_bf16(mean, "rtz"))
            lo, hi = np.minimum(r_up, r_dn), np.maximum(r_up, r_dn)
            ties = int(np.sum((hi != lo) & (mean - lo == hi - mean)))
    n = mean.size
    say(f"[rounding] skv={skv}: {n} distinct outputs per mode, {ties} exact ties")
    assert n >= 100_000
    if skv == 2:
        assert ties > 0.3 * n
    elif skv <= 64:
        assert ties > 0.01 * n


def test_plain_c_entry_point_matches_the_extended_one():
    """The exported attn_fwd_bf16 symbol, called straight through ctypes with
    raw device pointers, gives the same bits as attn_fwd_bf16_ex with the
    planner's choices, in every mode (unsplit and planner-split shapes)."""
    from bf16_attention_forward_amd import load_library
    lib = load_library()
    for (B, H, Sq, Skv, layout) in ((1, 3, 300, 1000, 1), (2, 16, 4096, 4096, 1), (1, 2, 129, 63, 0)):
        q, k, v = wl.random_qkv("bhsd" if layout else "bshd", B, H, Sq, Skv, 21 + Sq, 1.0, 2.0, 1.0)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        oa, ob = torch.empty_like(qd), torch.empty_like(qd)
        stream = torch.cuda.current_stream().cuda_stream
        for m in range(3):
            fn = lib.attn_fwd_bf16
            rc = fn(ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kd.data_ptr()), ctypes.c_void_p(vd.data_ptr()),
                    ctypes.c_void_p(oa.data_ptr()), layout, B, H, Sq, Skv, ctypes.c_float(wl.DEFAULT_SCALE), m,
                    ctypes.c_void_p(stream))
            assert rc == 0, rc
            rc = lib.attn_fwd_bf16_ex(ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kd.data_ptr()),
                                      ctypes.c_void_p(vd.data_ptr()), ctypes.c_void_p(ob.data_ptr()), layout, B, H,
                                      Sq, Skv, ctypes.c_float(wl.DEFAULT_SCALE), m, ctypes.c_void_p(stream), 0, 0, 0, 0)
            assert rc == 0, rc
            torch.cuda.synchronize()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), (B, H, Sq, Skv, m)
