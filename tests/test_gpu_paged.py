"""GPU parity of attn_fwd_bf16_paged: keys and values in a paged cache with a
key count per batch entry, against the fp64 oracle run on each entry's
keys and values laid out densely (the test gathers them from the cache by
the block table), through the C ABI.  Same bar as the dense path (both
gates); entries with no keys give zero rows and lse -inf."""
import numpy as np
import pytest
import torch

from bf16_attention_forward_amd import workloads as wl
from tests.helpers import assert_gates, check, say, to_dev

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")


def dense_kv(pk: wl.PagedKV, b: int):
    """Entry b's keys and values as [1, kv_len, Hkv, D] (bshd), gathered on the CPU."""
    n = int(pk.kv_lens[b])
    idx = torch.arange(n)
    pages = pk.block_table[b, (idx // pk.page_size)].long()
    rows = idx % pk.page_size
    return pk.k_cache[pages, rows].unsqueeze(0), pk.v_cache[pages, rows].unsqueeze(0)


def to_layout(t_bshd, layout):
    return t_bshd if layout == "bshd" else t_bshd.permute(0, 2, 1, 3).contiguous()


def run_paged(q, pk, layout, mode, causal, scale=None, lse=False):
    from bf16_attention_forward_amd import attn_fwd_bf16_paged
    out = attn_fwd_bf16_paged(to_dev(q), to_dev(pk.k_cache), to_dev(pk.v_cache), to_dev(pk.block_table),
                              to_dev(pk.kv_lens), max_kv_len=pk.max_kv_len, layout=layout, round_mode=mode,
                              causal=causal, scale=scale, return_lse=lse)
    torch.cuda.synchronize()
    if lse:
        return wl.bits(out[0].cpu()), out[1].cpu().numpy()
    return wl.bits(out.cpu())


def gate_entries(o_bits, q, pk, layout, mode, causal, D, scale, label):
    B = q.shape[0]
    for b in range(B):
        n = int(pk.kv_lens[b])
        ob = o_bits[b:b + 1]
        if n == 0:
            assert np.all(ob == 0), (label, b)
            continue
        kb, vb = dense_kv(pk, b)
        st, _ = check(ob, q[b:b + 1], to_layout(kb, layout), to_layout(vb, layout), layout, mode,
                      scale=scale, label=f"{label} entry {b} kv {n}", causal=causal)
        assert_gates(st)


# layout, B, Hq, Hkv, Sq, kv_lens, page_size, causal, D
CASES = [
    ("bshd", 3, 4, 2, 200, (333, 64, 1000), 64, False, 128),      # ragged lengths, page = key tile
    ("bhsd", 2, 2, 2, 130, (257, 130), 16, True, 128),            # small pages, causal per entry
    ("bshd", 4, 6, 3, 70, (0, 1, 63, 700), 128, False, 128),      # an empty entry, single key, tile edge
    ("bhsd", 2, 4, 1, 300, (120, 2000), 256, True, 64),           # head dimension 64, Sq > kv_len in entry 0
    ("bshd", 2, 2, 2, 64, (4097, 50), 100, False, 64),            # page size not a power of two
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}Hq{c[2]}Hkv{c[3]}_sq{c[4]}_kv{'-'.join(map(str, c[5]))}_p{c[6]}_{'causal' if c[7] else 'full'}_d{c[8]}")
@pytest.mark.parametrize("mode", MODES)
def test_paged_matches_oracle(case, mode):
    layout, B, Hq, Hkv, Sq, kv_lens, ps, causal, D = case
    say(f"[case] paged {case} {mode}")
    pk = wl.make_paged_kv(B, Hkv, kv_lens, ps, seed=300 + Sq, D=D, share_first_page=True)
    q = wl.random_qkv(layout, B, Hq, Sq, 1, 300 + Sq, D=D)[0]
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o = run_paged(q, pk, layout, mode, causal, scale=scale)
    gate_entries(o, q, pk, layout, mode, causal, D, scale, str(case))


def test_paged_identity_table_equals_dense_bitwise():
    """Pages laid out in order (block table = identity, every entry full)
    give the dense kernel's bits under the causal mask: the same kernel code
    runs on the same rows.  (Without the mask the dense kernel at head
    dimension 128 sums the weights on the matrix core and the per-entry one
    with VALU adds, so the two agree within the gates, not bit for bit.)"""
    from bf16_attention_forward_amd import attn_fwd_bf16_gqa
    B, H, Sq, Skv, ps = 2, 4, 300, 640, 64
    q, k, v = wl.random_qkv("bshd", B, H, Sq, Skv, 71)
    pages = Skv // ps
    kc = k.reshape(B * pages, ps, H, 128).contiguous()
    vc = v.reshape(B * pages, ps, H, 128).contiguous()
    table = torch.arange(B * pages, dtype=torch.int32).reshape(B, pages)
    pk = wl.PagedKV(kc, vc, table, torch.full((B,), Skv, dtype=torch.int32), ps, Skv)
    a = run_paged(q, pk, "bshd", "rtne", True, scale=wl.DEFAULT_SCALE)
    bd = attn_fwd_bf16_gqa(to_dev(q), to_dev(k), to_dev(v), layout="bshd", scale=wl.DEFAULT_SCALE, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(a, wl.bits(bd.cpu()))


def test_empty_entries_and_lse():
    """Entries with no keys: zero rows and lse -inf; the other entries' lse
    matches the dense path's definition within the lse gate."""
    import oracle
    layout, B, H, Sq = "bshd", 3, 2, 90
    pk = wl.make_paged_kv(B, H, (0, 150, 0), 64, seed=72)
    q = wl.random_qkv(layout, B, H, Sq, 1, 72)[0]
    o, lse = run_paged(q, pk, layout, "rtne", False, scale=wl.DEFAULT_SCALE, lse=True)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    kb, vb = dense_kv(pk, 1)
    res = oracle.attention(wl.bits(q[1:2]), wl.bits(kb), wl.bits(vb), layout=layout, scale=wl.DEFAULT_SCALE,
                           method=False)
    ref = res.lse.reshape(1, H, Sq)
    assert np.all(np.abs(lse[1] - ref[0]) <= 2.0 ** -8 + 2.0 ** -20 * np.abs(ref[0]))


def test_out_of_range_table_entries_read_as_zero_rows():
    """A block-table entry outside [0, num_pages) reads as zero rows: the
    result equals the dense attention over keys whose rows are zero there."""
    layout, B, H, Sq, ps = "bshd", 1, 2, 64, 64
    pk = wl.make_paged_kv(B, H, (192,), ps, seed=73)
    bad = pk.block_table.clone()
    bad[0, 1] = 10 ** 6
    pk_bad = wl.PagedKV(pk.k_cache, pk.v_cache, bad, pk.kv_lens, ps, pk.max_kv_len)
    q = wl.random_qkv(layout, B, H, Sq, 1, 73)[0]
    o = run_paged(q, pk_bad, layout, "rtne", False, scale=wl.DEFAULT_SCALE)
    kb, vb = dense_kv(pk, 0)
    kb[:, ps:2 * ps] = 0
    vb[:, ps:2 * ps] = 0
    st, _ = check(o, q, kb, vb, layout, "rtne", label="zero page")
    assert_gates(st)


def test_deterministic():
    pk = wl.make_paged_kv(2, 2, (700, 333), 64, seed=74)
    q = wl.random_qkv("bshd", 2, 4, 257, 1, 74)[0]
    outs = [run_paged(q, pk, "bshd", "rtne", True, scale=wl.DEFAULT_SCALE) for _ in range(3)]
    assert all(np.array_equal(outs[0], x) for x in outs[1:])


def test_many_entries_unsorted_lengths():
    """70 entries (more than one wave can rank: index order) and 9 entries
    (ranked longest first) with seeded unsorted lengths, some empty."""
    rng = np.random.default_rng(75)
    for B in (70, 9):
        lens = [int(v) for v in rng.integers(0, 300, size=B)]
        lens[3] = 0
        say(f"[case] paged many entries B={B}")
        pk = wl.make_paged_kv(B, 1, lens, 32, seed=75 + B)
        q = wl.random_qkv("bshd", B, 2, 40, 1, 75 + B)[0]
        o = run_paged(q, pk, "bshd", "rtne", False, scale=wl.DEFAULT_SCALE)
        gate_entries(o, q, pk, "bshd", "rtne", False, 128, wl.DEFAULT_SCALE, f"B={B}")


def test_in_place_and_copy_paths_agree_bitwise():
    """Pages of 128 rows (read in place) and of 96 rows (copied first) holding
    the same logical rows give the same bits, causal and not."""
    B, H, Sq = 3, 4, 200
    pk = wl.make_paged_kv(B, 2, (700, 129, 400), 128, seed=76)
    q = wl.random_qkv("bshd", B, H, Sq, 1, 76)[0]
    ps2 = 96
    pages = [(int(pk.kv_lens[b]) + ps2 - 1) // ps2 for b in range(B)]
    kc = torch.zeros((sum(pages) + 1, ps2, 2, 128), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    table = torch.full((B, max(pages)), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        kb, vb = dense_kv(pk, b)
        n = kb.shape[1]
        for i in range(pages[b]):
            rows = slice(i * ps2, min(n, (i + 1) * ps2))
            m = rows.stop - rows.start
            kc[nxt, :m] = kb[0, rows]
            vc[nxt, :m] = vb[0, rows]
            table[b, i] = nxt
            nxt += 1
    pk2 = wl.PagedKV(kc, vc, table, pk.kv_lens, ps2, pk.max_kv_len)
    for causal in (False, True):
        a = run_paged(q, pk, "bshd", "rtne", causal, scale=wl.DEFAULT_SCALE)
        b2 = run_paged(q, pk2, "bshd", "rtne", causal, scale=wl.DEFAULT_SCALE)
        assert np.array_equal(a, b2), causal
