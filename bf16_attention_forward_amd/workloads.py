"""Seeded synthetic workloads for bf16 attention forward.

This module only draws inputs; it holds none of the attention arithmetic, so
both the HIP path and the fp64 oracle can be fed from it.

The shapes stand in for the workloads the pages measure: plain N(0,1)
attention inputs (HipKittens summary, experiments section), video-diffusion
self-attention over a latent token grid and cross-attention from video
tokens to a short text sequence (MoonMath AI MI300X attention article, use
case section: Wan2.1 text-to-video with BSHD tensors and arbitrary KV
lengths).  No dataset or trained weights are involved: every tensor is
drawn from a seeded generator.

Recipe: torch CPU generator seeded per tensor, float32 normal draws, times
the workload's scale factor (a power of two, so exact), rounded to bf16 by
torch (round-to-nearest-even), created directly in the workload's layout.
Seeds: s = 1000 + workload number; q, k, v and the non-finite injection
sites use streams 4s, 4s+1, 4s+2, 4s+3.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
DEFAULT_SCALE = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    layout: str          # "bshd" or "bhsd"
    B: int
    H: int
    Sq: int
    Skv: int
    q_factor: float = 1.0
    k_factor: float = 1.0
    v_factor: float = 1.0
    modes: tuple = ("rtne", "rtna", "rtz")
    nonfinite_instance: bool = False
    note: str = ""
    Hkv: int = 0          # key/value heads (grouped-query attention); 0 = H
    causal: bool = False  # bottom-right aligned causal mask
    D: int = HEAD_DIM     # head dimension (128, or 64)

    @property
    def scale(self) -> float:
        """fp32(1/sqrt(D)), the usual softmax scale."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def pairs(self) -> int:
        """Attended (query, key) pairs per (batch, query head)."""
        return attended_pairs(self.Sq, self.Skv, self.causal)

    @property
    def flops(self) -> int:
        return 4 * self.B * self.H * self.pairs * self.D

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once and O written once, bf16."""
        return 2 * self.D * self.B * (2 * self.H * self.Sq + 2 * self.kv_heads * self.Skv)

    def describe(self) -> dict:
        d = {"workload": self.name, "layout": self.layout, "B": self.B, "H": self.H,
             "Sq": self.Sq, "Skv": self.Skv, "head_dim": self.D}
        if self.Hkv:
            d["Hkv"] = self.Hkv
        if self.causal:
            d["causal"] = True
        return d


def attended_pairs(Sq: int, Skv: int, causal: bool) -> int:
    """Number of (query, key) pairs per head: all of them, or under the
    bottom-right causal mask (query i sees keys j <= i + Skv - Sq)."""
    if not causal:
        return Sq * Skv
    i = np.arange(Sq, dtype=np.int64)
    return int(np.clip(i + (Skv - Sq) + 1, 0, Skv).sum())


WORKLOADS = {
    1: Workload(1, "tiny_self_attn_bshd_b1_h2_s128", "bshd", 1, 2, 128, 128,
                note="tiny self-attention"),
    2: Workload(2, "self_attn_bhsd_b2_h16_s4096_k2x", "bhsd", 2, 16, 4096, 4096, k_factor=2.0,
                nonfinite_instance=True, note="K scaled x2 to sharpen the softmax"),
    3: Workload(3, "video_self_attn_bshd_b1_h12_s32760", "bshd", 1, 12, 32760, 32760,
                q_factor=0.5, k_factor=0.5, v_factor=0.5, modes=("rtne",),
                note="21x30x52 latent tokens"),
    4: Workload(4, "video_text_cross_attn_bshd_b1_h12_sq32760_skv512", "bshd", 1, 12, 32760, 512,
                k_factor=0.5, v_factor=0.5, note="32760 video tokens attend to 512 text tokens"),
    5: Workload(5, "long_self_attn_bhsd_b1_h32_s16384", "bhsd", 1, 32, 16384, 16384,
                modes=("rtz", "rtne"), note="long sequence"),
    6: Workload(6, "causal_gqa_bhsd_b1_hq32_hkv8_s16384", "bhsd", 1, 32, 16384, 16384,
                Hkv=8, causal=True, modes=("rtne",),
                note="causal grouped-query attention, 4 query heads per key/value head"),
    7: Workload(7, "causal_self_attn_bshd_b2_h16_s4096", "bshd", 2, 16, 4096, 4096,
                causal=True, modes=("rtne", "rtz"), note="causal self-attention"),
    8: Workload(8, "self_attn_bhsd_b4_h16_s4096_d64", "bhsd", 4, 16, 4096, 4096, D=64,
                modes=("rtne",), note="head dimension 64, same FLOPs as the 4096^2 d=128 workload"),
    9: Workload(9, "video_self_attn_bshd_b1_h24_s32760_d64", "bshd", 1, 24, 32760, 32760, D=64,
                q_factor=0.5, k_factor=0.5, v_factor=0.5, modes=("rtne",),
                note="the video self-attention split into twice the heads of dimension 64"),
}


# The paged-cache workload: the video self-attention's per-head size with its
# keys and values in 256-token pages of a shared pool, four batch entries
# with a mix of cached lengths (the longest the full 32760-token latent) and
# 4096 new query tokens each, BSHD, no mask.
PAGED = dict(name="paged_kv_bshd_b4_h12_sq4096_kvmix_page256", B=4, H=12, Sq=4096,
             kv_lens=(32760, 20480, 12000, 4100), page_size=256, seed=1010,
             note="keys and values in a paged cache, per-entry lengths")


def paged_flops(H: int, Sq: int, kv_lens, D: int = HEAD_DIM) -> int:
    """Algorithmic FLOPs of the paged workload: 4 * H * Sq * kv_len * D per entry."""
    return sum(4 * H * Sq * int(n) * D for n in kv_lens)


def shape(layout: str, B: int, H: int, S: int, D: int = HEAD_DIM) -> tuple:
    if layout == "bshd":
        return (B, S, H, D)
    if layout == "bhsd":
        return (B, H, S, D)
    raise ValueError(layout)


def _draw(shape_, seed: int, factor: float) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    t = torch.randn(shape_, generator=g, dtype=torch.float32)
    if factor != 1.0:
        t = t * factor
    return t.to(torch.bfloat16)


def random_qkv(layout: str, B: int, H: int, Sq: int, Skv: int, seed: int,
               q_factor: float = 1.0, k_factor: float = 1.0, v_factor: float = 1.0,
               Hkv: int | None = None, D: int = HEAD_DIM):
    """Return (q, k, v) as bf16 CPU tensors in the given layout; k and v have
    Hkv heads (default H); D is the head dimension."""
    q = _draw(shape(layout, B, H, Sq, D), 4 * seed + 0, q_factor)
    k = _draw(shape(layout, B, Hkv or H, Skv, D), 4 * seed + 1, k_factor)
    v = _draw(shape(layout, B, Hkv or H, Skv, D), 4 * seed + 2, v_factor)
    return q, k, v


def make_inputs(w: Workload, *, Sq: int | None = None, Skv: int | None = None,
                B: int | None = None, H: int | None = None, seed: int | None = None):
    """Draw the workload's q, k, v (bf16 CPU tensors); sizes may be overridden."""
    return random_qkv(w.layout, B or w.B, H or w.H, Sq or w.Sq, Skv or w.Skv,
                      w.seed if seed is None else seed, w.q_factor, w.k_factor, w.v_factor,
                      Hkv=w.Hkv or None, D=w.D)


@dataclass
class PagedKV:
    """A paged key/value cache and its index tables (CPU tensors).

    k_cache, v_cache: bf16 [num_pages, page_size, Hkv, D]; block_table: int32
    [B, pages_per_seq]; kv_lens: int32 [B].  Row i < kv_lens[b] of batch
    entry b is row i % page_size of page block_table[b, i // page_size]."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    kv_lens: torch.Tensor
    page_size: int
    max_kv_len: int


def make_paged_kv(B: int, Hkv: int, kv_lens, page_size: int, seed: int, D: int = HEAD_DIM,
                  k_factor: float = 1.0, v_factor: float = 1.0, spare_pages: int = 3,
                  share_first_page: bool = False) -> PagedKV:
    """Seeded paged cache: every batch entry's pages are drawn from one pool
    in a seeded random order (so logical order never matches physical order),
    with `spare_pages` pages that no entry uses; with share_first_page,
    entries 0 and 1 share their first page (a common prefix).  Table slots
    past an entry's length hold -1 (never read)."""
    kv_lens = [int(x) for x in kv_lens]
    max_kv = max(max(kv_lens), 1)
    pps = (max_kv + page_size - 1) // page_size
    need = [(n + page_size - 1) // page_size for n in kv_lens]
    num_pages = sum(need) + spare_pages
    g = torch.Generator(device="cpu")
    g.manual_seed(4 * seed + 3)
    order = torch.randperm(num_pages, generator=g)
    table = torch.full((B, pps), -1, dtype=torch.int32)
    pos = 0
    for b in range(B):
        for i in range(need[b]):
            table[b, i] = int(order[pos])
            pos += 1
    if share_first_page and B >= 2 and need[0] > 0 and need[1] > 0:
        table[1, 0] = table[0, 0]
    k_cache = _draw((num_pages, page_size, Hkv, D), 4 * seed + 1, k_factor)
    v_cache = _draw((num_pages, page_size, Hkv, D), 4 * seed + 2, v_factor)
    return PagedKV(k_cache, v_cache, table, torch.tensor(kv_lens, dtype=torch.int32), page_size, max_kv)


@dataclass
class Packed:
    """A batch of packed sequences (CPU tensors): q [total_q, H, D], k, v
    [total_k, Hkv, D] bf16 hold the rows of all sequences; cu_q, cu_k int32
    [B + 1] are the prefix sums of their row counts."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_q: torch.Tensor
    cu_k: torch.Tensor

    def seq(self, b: int):
        """Sequence b as BSHD tensors [1, len, heads, D] (q, k, v)."""
        q0, q1 = int(self.cu_q[b]), int(self.cu_q[b + 1])
        k0, k1 = int(self.cu_k[b]), int(self.cu_k[b + 1])
        return self.q[q0:q1].unsqueeze(0), self.k[k0:k1].unsqueeze(0), self.v[k0:k1].unsqueeze(0)


def make_packed(H: int, Hkv: int, lens_q, lens_k, seed: int, D: int = HEAD_DIM,
                q_factor: float = 1.0, k_factor: float = 1.0, v_factor: float = 1.0) -> Packed:
    """Seeded packed sequences of the given query and key row counts."""
    lq, lk = [int(x) for x in lens_q], [int(x) for x in lens_k]
    cu_q = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32)
    q = _draw((max(sum(lq), 1), H, D), 4 * seed + 0, q_factor)
    k = _draw((max(sum(lk), 1), Hkv, D), 4 * seed + 1, k_factor)
    v = _draw((max(sum(lk), 1), Hkv, D), 4 * seed + 2, v_factor)
    return Packed(q, k, v, cu_q, cu_k)


# Packed sequences: the video self-attention's 12 heads of 128 over eight
# clips of different lengths (30 x 52 latent tokens per frame, 21 frames
# down to 1 frame: 32760 down to 1560 tokens), self-attention within each
# clip, all clips in one tensor.
VARLEN = dict(name="varlen_self_attn_thd_h12_8clips", H=12,
              lens=(32760, 24960, 18720, 12480, 9360, 6240, 3120, 1560), seed=1011,
              note="packed sequences of different lengths")


def varlen_flops(H: int, lens_q, lens_k, D: int = HEAD_DIM) -> int:
    """Algorithmic FLOPs of packed non-causal attention: 4 * H * len_q * len_k * D per sequence."""
    return sum(4 * H * int(a) * int(b) * D for a, b in zip(lens_q, lens_k))


@dataclass
class Injection:
    """Non-finite values planted into q and v (positions as (b, h, s, d))."""
    q_sites: list = field(default_factory=list)   # (b, h, i, d, value)
    v_sites: list = field(default_factory=list)   # (b, h, j, d, value)


def inject_nonfinite(q: torch.Tensor, v: torch.Tensor, layout: str, seed: int,
                     n_q=(3, 2, 2), n_v=(2, 2, 2), mixed_inf_column: bool = True) -> Injection:
    """Plant NaN / +Inf / -Inf into q and v in place at seeded sites.

    n_q, n_v: counts of (NaN, +Inf, -Inf).  With mixed_inf_column, one more
    column of v (one head, one d) gets both a +Inf and a -Inf.
    """
    rng = np.random.default_rng(4 * seed + 3)
    if layout == "bshd":
        B, Sq, H, D = q.shape
        Skv = v.shape[1]
    else:
        B, H, Sq, D = q.shape
        Skv = v.shape[2]
    inj = Injection()

    def put(t, b, h, s, d, val):
        if layout == "bshd":
            t[b, s, h, d] = val
        else:
            t[b, h, s, d] = val

    vals = [float("nan"), float("inf"), float("-inf")]
    for kind, cnt in enumerate(n_q):
        for _ in range(cnt):
            b, h, i, d = (int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Sq)), int(rng.integers(D)))
            put(q, b, h, i, d, vals[kind])
            inj.q_sites.append((b, h, i, d, vals[kind]))
    for kind, cnt in enumerate(n_v):
        for _ in range(cnt):
            b, h, j, d = (int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Skv)), int(rng.integers(D)))
            put(v, b, h, j, d, vals[kind])
            inj.v_sites.append((b, h, j, d, vals[kind]))
    if mixed_inf_column and Skv >= 2:
        b, h, d = int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(D))
        j1, j2 = rng.choice(Skv, size=2, replace=False)
        put(v, b, h, int(j1), d, float("inf"))
        put(v, b, h, int(j2), d, float("-inf"))
        inj.v_sites.append((b, h, int(j1), d, float("inf")))
        inj.v_sites.append((b, h, int(j2), d, float("-inf")))
    return inj


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (a view of the same bytes)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def row_ids(layout: str, B: int, H: int, Sq: int, b, h, i) -> np.ndarray:
    """Flat query-row ids r = (b*H + h)*Sq + i (independent of layout)."""
    return (np.asarray(b) * H + np.asarray(h)) * Sq + np.asarray(i)


def gather_rows(o_bits: np.ndarray, layout: str, B: int, H: int, Sq: int, rows) -> np.ndarray:
    """Pick rows (flat ids) out of an output tensor's bf16 bits -> [n, D]."""
    rows = np.asarray(rows, dtype=np.int64)
    i = rows % Sq
    bh = rows // Sq
    h = bh % H
    b = bh // H
    if layout == "bshd":
        return o_bits.reshape(B, Sq, H, -1)[b, i, h]
    return o_bits.reshape(B, H, Sq, -1)[b, h, i]


def sample_rows(B: int, H: int, Sq: int, n_per_head: int, seed: int, tile: int = 256) -> np.ndarray:
    """Seeded row sample: per head the first and last rows, the last row of
    the first query tile, every row of the last query tile when it is ragged
    (Sq not a multiple of `tile`; otherwise its first row), and n_per_head
    random rows.  With tile = 256, the query tile of the 8-wave kernel, the
    ragged tail also holds the whole last tile of the 128-row kernel."""
    rng = np.random.default_rng(seed)
    out = []
    last0 = (Sq - 1) // tile * tile
    tail = set(range(last0, Sq)) if Sq % tile else {last0}
    for bh in range(B * H):
        base = bh * Sq
        fixed = {0, Sq - 1, min(Sq - 1, tile - 1)} | tail
        rnd = rng.integers(0, Sq, size=n_per_head)
        out.extend(base + np.array(sorted(fixed | set(int(x) for x in rnd))))
    return np.array(out, dtype=np.int64)
