"""GPU parity of attn_fwd_bf16_varlen: packed sequences of different lengths
(queries and keys), each gated against the fp64 oracle run on that
sequence alone, through the C ABI.  Same bar as the dense path (both gates);
a sequence with no keys gives zero rows and lse -inf; a single sequence
gives the dense call's bits."""
import numpy as np
import pytest
import torch

from bf16_attention_forward_amd import workloads as wl
from tests.helpers import assert_gates, check, say, to_dev

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")


def run_varlen(pk, mode="rtne", causal=False, scale=None, lse=False, max_q=None, max_k=None, cu_q=None, cu_k=None):
    from bf16_attention_forward_amd import attn_fwd_bf16_varlen
    lq = (pk.cu_q[1:] - pk.cu_q[:-1]).tolist()
    lk = (pk.cu_k[1:] - pk.cu_k[:-1]).tolist()
    out = attn_fwd_bf16_varlen(to_dev(pk.q), to_dev(pk.k), to_dev(pk.v),
                               to_dev(pk.cu_q if cu_q is None else cu_q), to_dev(pk.cu_k if cu_k is None else cu_k),
                               max_seqlen_q=max_q or max(max(lq), 1), max_seqlen_k=max_k or max(max(lk), 1),
                               round_mode=mode, causal=causal, scale=scale, return_lse=lse)
    torch.cuda.synchronize()
    if lse:
        return wl.bits(out[0].cpu()), out[1].cpu().numpy()
    return wl.bits(out.cpu())


def gate_sequences(o_bits, pk, mode, causal, scale, label):
    for b in range(len(pk.cu_q) - 1):
        q0, q1 = int(pk.cu_q[b]), int(pk.cu_q[b + 1])
        if q1 == q0:
            continue
        qs, ks, vs = pk.seq(b)
        ob = o_bits[q0:q1][None]
        if ks.shape[1] == 0:
            assert np.all(ob == 0), (label, b)
            continue
        st, _ = check(ob, qs, ks, vs, "bshd", mode, scale=scale, label=f"{label} seq {b}", causal=causal)
        assert_gates(st)


# Hq, Hkv, lens_q, lens_k, causal, D
CASES = [
    (4, 2, (300, 1, 65, 700), (333, 64, 1000, 700), False, 128),     # ragged lengths, GQA
    (2, 2, (257, 130, 64), (257, 300, 64), True, 128),                 # causal per sequence, Sq != Skv
    (4, 4, (0, 90, 129, 0), (50, 0, 129, 70), False, 128),             # empty query and key sequences
    (4, 1, (300, 2000), (120, 2000), True, 64),                        # head dimension 64, Sq > Skv
    (6, 3, (40, 1500, 513), (4097, 20, 513), False, 64),               # long keys, short queries
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Hq{c[0]}Hkv{c[1]}_q{'-'.join(map(str, c[2]))}_k{'-'.join(map(str, c[3]))}_{'causal' if c[4] else 'full'}_d{c[5]}")
@pytest.mark.parametrize("mode", MODES)
def test_varlen_matches_oracle(case, mode):
    Hq, Hkv, lq, lk, causal, D = case
    say(f"[case] varlen {case} {mode}")
    pk = wl.make_packed(Hq, Hkv, lq, lk, seed=400 + sum(lq), D=D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o = run_varlen(pk, mode, causal, scale=scale)
    gate_sequences(o, pk, mode, causal, scale, str(case))


def test_single_sequence_equals_dense_bitwise():
    """One sequence of the whole tensor gives the dense call's bits under the
    causal mask (the same kernel code on the same rows, keys unsplit; without
    the mask the dense kernel at head dimension 128 sums the weights on the
    matrix core and the per-sequence one with VALU adds)."""
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa
    S, Skv, H = 700, 900, 4
    pk = wl.make_packed(H, H, (S,), (Skv,), seed=81)
    a = run_varlen(pk, causal=True, scale=wl.DEFAULT_SCALE)
    bd = attn_fwd_bf16_gqa(to_dev(pk.q[None]), to_dev(pk.k[None]), to_dev(pk.v[None]), layout="bshd",
                           scale=wl.DEFAULT_SCALE, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(a, wl.bits(bd.cpu()[0]))


def test_lse_layout_and_empty_sequences():
    """lse is [Hq, total_q]: each row's natural-log log-sum-exp (the oracle's,
    within the lse gate); a sequence with no keys has zero rows and lse -inf."""
    import oracle
    pk = wl.make_packed(2, 2, (90, 40, 70), (150, 0, 64), seed=82)
    o, lse = run_varlen(pk, scale=wl.DEFAULT_SCALE, lse=True)
    assert lse.shape == (2, 200)
    assert np.all(o[90:130] == 0) and np.all(np.isneginf(lse[:, 90:130]))
    for b, (q0, q1) in enumerate(((0, 90), (130, 200))):
        qs, ks, vs = pk.seq(0 if b == 0 else 2)
        res = oracle.attention(wl.bits(qs), wl.bits(ks), wl.bits(vs), layout="bshd", scale=wl.DEFAULT_SCALE,
                               method=False)
        ref = res.lse.reshape(1, 2, q1 - q0)[0]
        assert np.all(np.abs(lse[:, q0:q1] - ref) <= 2.0 ** -8 + 2.0 ** -20 * np.abs(ref))


def test_many_sequences_unsorted():
    """70 sequences (more than one wave ranks: index order) and 9 (ranked
    longest first) of seeded lengths, some empty."""
    rng = np.random.default_rng(83)
    for B in (70, 9):
        lq = [int(x) for x in rng.integers(0, 200, size=B)]
        lk = [int(x) for x in rng.integers(0, 300, size=B)]
        lq[2], lk[5] = 0, 0
        say(f"[case] varlen many sequences B={B}")
        pk = wl.make_packed(2, 1, lq, lk, seed=84 + B)
        o = run_varlen(pk, scale=wl.DEFAULT_SCALE)
        gate_sequences(o, pk, "rtne", False, wl.DEFAULT_SCALE, f"B={B}")


def test_prefix_sums_are_clamped():
    """Prefix sums past the packed tensors, or lengths past max_seqlen, are
    cut to fit: here the last sequence's key range ends at the tensor's last
    row and its queries at max_seqlen_q, and the result is that of the cut
    sequence (rows past it untouched)."""
    pk = wl.make_packed(2, 2, (100, 80), (120, 90), seed=85)
    cu_k = pk.cu_k.clone()
    cu_k[2] = 10 ** 6                                  # past total_k = 210: clamped to 210
    from bf16_attention_forward_amd import attn_fwd_bf16_varlen
    o = torch.full_like(to_dev(pk.q), 7.0)
    attn_fwd_bf16_varlen(to_dev(pk.q), to_dev(pk.k), to_dev(pk.v), to_dev(pk.cu_q), to_dev(cu_k), o,
                         max_seqlen_q=60, max_seqlen_k=200, scale=wl.DEFAULT_SCALE)
    torch.cuda.synchronize()
    ob = wl.bits(o.cpu())
    seven = wl.bits(torch.full((1,), 7.0, dtype=torch.bfloat16))[0]
    for b, (q0, n) in enumerate(((0, 60), (100, 60))):  # both sequences cut to 60 query rows
        qs, ks, vs = pk.seq(b)
        st, _ = check(ob[q0:q0 + n][None], qs[:, :n], ks, vs, "bshd", "rtne", label=f"clamped seq {b}")
        assert_gates(st)
    assert np.all(ob[60:100] == seven) and np.all(ob[160:180] == seven)


def test_deterministic():
    pk = wl.make_packed(4, 2, (333, 700, 64), (500, 64, 900), seed=86)
    outs = [run_varlen(pk, causal=True, scale=wl.DEFAULT_SCALE) for _ in range(3)]
    assert all(np.array_equal(outs[0], x) for x in outs[1:])
