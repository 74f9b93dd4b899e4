"""CPU model of the kernels' LDS tile layouts (no GPU).

The kernels move K/V (forward) and K/V, Q/dO (backward) tiles from HBM into
LDS with buffer_load ... lds, where lane l of an instruction writes 16 bytes
at LDS base + 16 l, and put the bank swizzle into each lane's source
address.  The MFMA operands are then read back with ds_read_b128 (straight:
8 consecutive dims of one row per lane) and ds_read_b64_tr_b16 (transposed:
within each 16-lane group, output lane j element e is element j % 4 of the
4 bf16 addressed by source lane 4 e + j / 4 -- the lane map probed on the
GPU).  This model replays the index arithmetic of the kernels on symbolic
tiles (each element tagged with its (row, dim)) and checks:

  * placement: every (row, 16-byte chunk) of a tile lands exactly once, at
    the position the readers assume;
  * operands: every lane reads exactly the (row, dim) the MFMA operand
    layout needs (16x16x32 bf16: A lane (g, j) holds row j, k = 8 g .. 8 g +
    7; the score fragment's keys 16 kb + 4 g + r fix the k order of the
    weights, which the transposed V reads must match);
  * banks, transposed reads: the 32 lanes of a half-wave, which one
    ds_read_b64_tr_b16 serves together, read 32 distinct 8-byte slots of a
    256-byte bank pass (this rule matched every swizzle measured with the
    SQ_LDS_BANK_CONFLICT counter);
  * banks, straight reads: no simple lane-grouping rule matched the
    ds_read_b128 conflicts measured for five candidate swizzles (a layout
    whose 16 rows take 16 distinct 16-byte slots conflicted, one with 8
    did not), so the straight-read layouts are pinned to the swizzles
    measured conflict-free, and the kernels' own counters confirm it.

The formulas restate the kernels' (attn_fwd_kernel.hip, attn_bwd_kernel.hip);
the invariants they must satisfy come from the operand layouts.
"""
import pytest

TILE_ROWS = 64


# Chunk swizzles whose straight ds_read_b128 fragment reads (lane (g, j):
# row j, 16-byte chunk 4 kk + g) showed zero SQ_LDS_BANK_CONFLICT cycles on
# gfx950, by head dimension, over rows 0..15.  Measured and found
# conflicting: 2 (r & 7) + ((r >> 3) & 1) at 128 (2.7 conflict cycles per
# read) and 2 ((r >> 1) & 3) + ((r >> 3) & 1) at 64 (2.0).
STRAIGHT_CONFLICT_FREE = {
    128: [[r & 15 for r in range(16)], [(r & 7) << 1 for r in range(16)]],
    64: [[(r >> 1) & 7 for r in range(16)], [((r >> 1) & 3) << 1 for r in range(16)]],
}


# ---------------------------------------------------------------- forward
def swz_k(hd, row):
    return (row & 15) if hd == 128 else ((row >> 1) & 7)


def swz_v(hd, row):
    return ((row & 7) << 1) if hd == 128 else (((row >> 1) & 3) << 1)


def fwd_dma_image(hd, swz):
    """LDS image of a 64-row tile after the forward's DMA: {byte offset of a
    16-byte slot: (row, logical chunk)}."""
    row_bytes = hd * 2
    cpr = row_bytes // 16            # chunks per row
    rpw = 64 // cpr                  # rows per wave and round
    rpr = 4 * rpw                    # rows per round (4 issuing waves)
    image = {}
    for r in range(TILE_ROWS // rpr):
        for w in range(4):
            for lane in range(64):
                dma_row = w * rpw + lane // cpr
                chunk = lane % cpr
                src_row = rpr * r + dma_row
                src_chunk = chunk ^ swz(hd, dma_row)           # the swizzle is on the source side
                lds = ((r * 4 + w) * 64 + lane) * 16
                assert lds not in image
                image[lds] = (src_row, src_chunk)
    return image


def element(image, byte):
    """(row, dim) of the bf16 at LDS byte offset `byte`."""
    row, chunk = image[byte - byte % 16]
    return row, chunk * 8 + (byte % 16) // 2


@pytest.mark.parametrize("hd", [128, 64])
@pytest.mark.parametrize("which", ["k", "v"])
def test_forward_dma_places_every_chunk_once(hd, which):
    swz = swz_k if which == "k" else swz_v
    image = fwd_dma_image(hd, swz)
    row_bytes = hd * 2
    assert sorted(image.values()) == [(r, c) for r in range(TILE_ROWS) for c in range(row_bytes // 16)]
    for lds, (row, chunk) in image.items():
        assert lds == row * row_bytes + ((chunk ^ swz(hd, row)) << 4)


@pytest.mark.parametrize("hd", [128, 64])
def test_forward_k_fragments(hd):
    """S^T = K Q^T, K as operand A: lane (g, j) of step (ks, kb) must read
    key 16 kb + j, dims 32 ks + 8 g .. + 7, through a swizzle measured
    conflict-free for these reads."""
    image = fwd_dma_image(hd, swz_k)
    row_bytes = hd * 2
    assert [swz_k(hd, r) for r in range(16)] in STRAIGHT_CONFLICT_FREE[hd]
    for ks in range(hd // 32):
        for kb in range(4):
            for g in range(4):
                for j in range(16):
                    k_addr = j * row_bytes + (((4 * ks + g) ^ swz_k(hd, j)) << 4)
                    addr = k_addr + kb * 16 * row_bytes
                    got = [element(image, addr + 2 * e) for e in range(8)]
                    assert got == [(16 * kb + j, 32 * ks + 8 * g + e) for e in range(8)]


def tr16(addrs, image):
    """ds_read_b64_tr_b16 on one 16-lane group: source lane s addresses 4
    bf16; output lane j element e is element j % 4 of source lane 4 e + j / 4."""
    out = []
    for j in range(16):
        s_lane = [4 * e + j // 4 for e in range(4)]
        out.append([element(image, addrs[s] + 2 * (j % 4)) for s in s_lane])
    return out


@pytest.mark.parametrize("hd", [128, 64])
def test_forward_v_fragments_match_the_weights(hd):
    """O^T += V^T P^T, V^T as operand A read transposed: lane (g, j),
    element 4 hf + e, must hold V[key][dim 16 db + j] for the key of the
    weight in element 4 hf + e of the P fragment: 32 ks + 16 hf + 4 g + e.
    A half-wave (32 lanes, 8 bytes each) reads 32 distinct 8-byte slots."""
    image = fwd_dma_image(hd, swz_v)
    row_bytes = hd * 2
    for ks in range(2):
        for db in range(hd // 16):
            for hf in range(2):
                lane_addr = {}
                for g in range(4):
                    for j in range(16):
                        row = 4 * g + (j >> 2)
                        chunk = (2 * db + ((j & 3) >> 1)) ^ swz_v(hd, row)
                        v_addr = row * row_bytes + (chunk << 4) + ((j & 1) << 3)
                        lane_addr[(g, j)] = v_addr + (32 * ks + 16 * hf) * row_bytes
                for g in range(4):
                    out = tr16([lane_addr[(g, s)] for s in range(16)], image)
                    for j in range(16):
                        assert out[j] == [(32 * ks + 16 * hf + 4 * g + e, 16 * db + j) for e in range(4)]
                for half in range(2):
                    slots = {(lane_addr[(g, j)] % 256) // 8 for g in (2 * half, 2 * half + 1) for j in range(16)}
                    assert len(slots) == 32, (hd, ks, db, hf, half)


def test_forward_weight_key_order():
    """The P fragment (operand B) element e of lane (g, j) in k-step ks holds
    the weight of key 32 ks + 16 (e >> 2) + 4 g + (e & 3): score fragment kb =
    2 ks + (e >> 2), register e & 3 (lane (g, j) holds keys 16 kb + 4 g + r),
    packed pairwise in that order."""
    for ks in range(2):
        for g in range(4):
            keys = []
            for i in range(4):                        # the four bf16 pairs, low then high
                kb = 2 * ks + (i >> 1)
                keys += [16 * kb + 4 * g + 2 * (i & 1), 16 * kb + 4 * g + 2 * (i & 1) + 1]
            assert keys == [32 * ks + 16 * (e >> 2) + 4 * g + (e & 3) for e in range(8)]


# ---------------------------------------------------------------- backward
def swz_b(hd, row):
    """256-byte rows: 2 (r & 7); 128-byte rows (two rows per 256-byte bank
    pass): 2 ((r >> 1) & 3) -- the forward's V layouts, which serve both
    read kinds without conflicts."""
    if hd == 128:
        return (row & 7) << 1
    return ((row >> 1) & 3) << 1


def bwd_dma_image(hd, nwk):
    """The backward's issue_tile_n: NWK waves move a 64-row tile in rounds of
    64 NWK / CPR rows (CPR = 16-byte chunks per row); lane l of wave w in
    round i writes row (64 / CPR) (NWK i + w) + l / CPR, chunk position
    l % CPR, holding source chunk (l % CPR) ^ swz(row)."""
    cpr = hd // 8
    rpw = 64 // cpr                  # rows per wave and round
    image = {}
    for i in range(TILE_ROWS // (rpw * nwk)):
        for w in range(nwk):
            for lane in range(64):
                row = rpw * w + lane // cpr
                pos = lane % cpr
                src_row = rpw * nwk * i + row
                lds = ((i * nwk + w) * 64 + lane) * 16
                assert lds not in image
                image[lds] = (src_row, pos ^ swz_b(hd, row))
    return image


@pytest.mark.parametrize("hd", [128, 64])
@pytest.mark.parametrize("nwk", [8, 4])
def test_backward_dma_places_every_chunk_once(hd, nwk):
    image = bwd_dma_image(hd, nwk)
    row_bytes = 2 * hd
    assert sorted(image.values()) == [(r, c) for r in range(TILE_ROWS) for c in range(hd // 8)]
    for lds, (row, chunk) in image.items():
        assert lds == row * row_bytes + ((chunk ^ swz_b(hd, row)) << 4)


@pytest.mark.parametrize("hd", [128, 64])
def test_backward_straight_and_transposed_reads(hd):
    """One layout serves both reads of every backward tile: read_rows (lane
    (g, j) of step (kk, rb): row 16 rb + j, dims 32 kk + 8 g .. + 7) and
    read_cols (lane (g, j), element 4 hf + e: row 32 ks + 16 hf + 4 g + e,
    dim 16 db + j); the straight reads through a swizzle measured
    conflict-free, the transposed ones on 32 distinct slots per half-wave."""
    image = bwd_dma_image(hd, 8)
    rb_ = 2 * hd
    assert [swz_b(hd, r) for r in range(16)] in STRAIGHT_CONFLICT_FREE[hd]
    for kk in range(hd // 32):
        for rb in range(4):
            for g in range(4):
                for j in range(16):
                    addr = j * rb_ + (((4 * kk + g) ^ swz_b(hd, j)) << 4) + rb * 16 * rb_
                    assert [element(image, addr + 2 * e) for e in range(8)] == \
                        [(16 * rb + j, 32 * kk + 8 * g + e) for e in range(8)]
    for ks in range(2):
        for db in range(hd // 16):
            for hf in range(2):
                lane_addr = {}
                for g in range(4):
                    for j in range(16):
                        row = 4 * g + (j >> 2)
                        a_col = row * rb_ + (((2 * db + ((j & 3) >> 1)) ^ swz_b(hd, row)) << 4) + ((j & 1) << 3)
                        lane_addr[(g, j)] = a_col + (32 * ks + 16 * hf) * rb_
                for g in range(4):
                    out = tr16([lane_addr[(g, s)] for s in range(16)], image)
                    for j in range(16):
                        assert out[j] == [(32 * ks + 16 * hf + 4 * g + e, 16 * db + j) for e in range(4)]
                for half in range(2):
                    slots = {(lane_addr[(g, j)] % 256) // 8 for g in (2 * half, 2 * half + 1) for j in range(16)}
                    assert len(slots) == 32
