// attn_fwd_kernel.hip -- gfx950 (MI355X, CDNA4) kernels for bf16 attention forward.
//
// Computes O = softmax(Q K^T * scale) V for head dimension 128 or 64 (the
// fused operation of "MoonMath AI open-sources a HIP attention kernel for AMD
// MI300X that beats AITER", opening paragraphs), streaming K/V tiles with an
// online softmax.  Design, per work-group (8 waves, 256 query rows of one
// (batch, head), one work-group per CU; for key ranges of at most 16 tiles a
// 4-wave variant with 128 rows, two work-groups per CU, so one's Q loads and
// O stores overlap the other's matrix work):
//
//  * Each wave owns 32 query rows; its Q fragments stay in VGPRs for the
//    whole key loop and O accumulates in registers (the MI300X article's data
//    placement section keeps Q and the accumulators in registers too).
//  * K and V tiles of 64 keys go HBM -> LDS with buffer_load ... lds (16 B per
//    lane, lane-contiguous in LDS), double-buffered and shared by all waves.
//    The bank swizzle is applied to the source address of each lane, not to
//    the LDS address (HipKittens summary, method section on global async
//    loads).  Rows past the key range read as zero through the buffer range
//    check.  The first four waves issue all of it, one instruction every few
//    MFMA steps: issued at once, the 32 KiB of a tile queue behind the CU's
//    address unit and stall the issuing waves for ~500 cycles.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16, K as operand A and Q as
//    operand B.  With that order each lane holds scores of ONE query for a
//    set of keys, which is the B-operand layout of the next product
//    O^T = V^T P^T, so P never leaves registers (the FlyDSL procedure article,
//    optimisation section, states the operand-order trick for gfx942; here it
//    is re-derived for the 16x16x32 shape).  The AITER docs index names the
//    same bf16 16x16x32 MFMA for both attention products on gfx950.
//  * V^T fragments come from the row-major V tile through ds_read_b64_tr_b16,
//    the gfx950 transposing LDS read (FlyDSL article: gfx950 adds
//    LDS-to-register transpose loads); its 4+4 source rows are chosen to match
//    the keys of P's elements, so V needs no shuffle.
//  * Online softmax with a power-of-two running offset: x = s * scale *
//    log2(e), p = 2^(x - M), M an integer set to ceil(max x) on the first
//    tile.  Later tiles compute no maximum at all: a weight can exceed 2^16
//    only if its lane's sum of the tile's weights does, and only then (the
//    row max moved far past M) is the tile redone with M = ceil(max x) and O
//    and the row sum rescaled by the exact power of two.  With a positive
//    scale the score MFMAs start from -M/c instead of zero, so the exponent
//    x - M is one multiply by c (which co-issues) rather than a multiply-add.
//    Row maxima and sums are reduced across the 4 lanes of a row with the
//    gfx950 v_permlane16/32_swap instructions.
//  * P enters the second product as bf16 rounded to nearest-even
//    (v_cvt_pk_bf16_f32); the row sum adds those same bf16 weights (as fp32,
//    by bit placement: v_dot2c_f32_bf16 would wait for the matrix core that
//    the other wave of the SIMD keeps busy), and the output is divided by it
//    and rounded to bf16 in the requested mode with integer bit arithmetic
//    after a NaN guard.
//  * One barrier per key tile, at a different place for the two waves of a
//    SIMD (the two-group schedule of the MI300X article's architecture
//    section and of the HipKittens 8-wave ping-pong).  Waves 0-3 run, between
//    barriers t and t+1, S_t = K_t Q^T interleaved with the fragment reads of
//    O += V_{t-1}^T P_{t-1}^T and then the softmax of S_t; waves 4-7 run the
//    softmax of S_{t-1} and then the same MFMA phase.  One wave of each SIMD
//    is thus in its softmax while the other feeds the matrix core (at raised
//    issue priority, s_setprio).  Both groups read K_t and V_{t-1} between
//    the same two barriers, so one double-buffered protocol serves both.
//  * Optional split of the key range (the flash-decoding style tail split of
//    the MI300X article, section on the two later improvements): each split
//    writes its unnormalised fp32 O, M and row sum; a combine kernel merges the
//    splits in a fixed order with exact power-of-two weights.
//  * The block id -> work item map groups consecutive query tiles of a head
//    onto one XCD (blocks are dealt to the 8 XCDs round-robin), so the K/V of
//    a head is fetched into one XCD's L2 (HipKittens summary, chiplet-aware
//    grid schedule).  With per-entry key counts every XCD takes an equal
//    share of each batch entry, longest entry first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "attn_fwd_internal.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int BN = 64;          // keys per K/V tile
constexpr int NQB = KERNEL_NQB; // 16-row query blocks per wave
constexpr float LN2 = 0.693147180559945309f;
constexpr float WEIGHT_LIMIT = 65536.0f;    // a lane's tile sum of weights above this triggers a new offset

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over lanes {l, l^16, l^32, l^48} (NaN-propagating)
__device__ __forceinline__ float rowmax4(float x) {
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __builtin_elementwise_maximum(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

// sum over lanes {l, l^16, l^32, l^48}, in a fixed pairing order
__device__ __forceinline__ float rowsum4(float x) {
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// fp32 -> bf16 in the requested mode as integer arithmetic on the bit
// pattern: add 0x7FFF plus the lowest kept bit (nearest-even), 0x8000 (ties
// away) or 0 (toward zero), keep the high half.  A NaN first becomes the
// canonical quiet NaN, whose sum keeps the high half 0x7FC0 in every mode;
// an infinity stays one, and the nearest modes overflow to it.  The mode's
// addend and the width of the lowest-bit field (1 or 0) are uniform, so a
// value costs a select, a bit-field extract and one three-way add, with no
// branch.
struct Bf16Round {
    uint32_t base, lsb_width;
};
__device__ __forceinline__ Bf16Round bf16_round(int mode) {
    return Bf16Round{mode == ROUND_RTNE ? 0x7fffu : (mode == ROUND_RTNA ? 0x8000u : 0u), mode == ROUND_RTNE ? 1u : 0u};
}
// the rounded value in the high half of the result (the low half is discarded)
__device__ __forceinline__ uint32_t bf16_round_hi(float f, Bf16Round m) {
    // an integer select: a floating-point select may pass any NaN through
    const uint32_t u = __builtin_isnan(f) ? 0x7fc00000u : __float_as_uint(f);
    return u + m.base + __builtin_amdgcn_ubfe(u, 16, m.lsb_width);
}
// a and b rounded, packed as bf16 (a in the low half)
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b, Bf16Round m) {
    return __builtin_amdgcn_perm(bf16_round_hi(b, m), bf16_round_hi(a, m), 0x07060302u);
}

// o / l with a reciprocal and one residual correction (q1 = q0 + (o - q0 l) r).
// When the true quotient is an fp32 value (e.g. o = l * v exactly) q1 is that
// value; non-finite q0 (Inf/NaN outputs) passes through unchanged.
__device__ __forceinline__ float div_corrected(float o, float l, float r) {
    const float q0 = o * r;
    const float e = __builtin_fmaf(-q0, l, o);
    const float q1 = __builtin_fmaf(e, r, q0);
    return (q1 == q1) ? q1 : q0;
}

// LDS layout of a K or V tile: 64 rows of HD*2 bytes (16-byte chunks), chunk
// positions XOR-swizzled per row so the reads below hit distinct banks (the
// LDS serves 256 bytes, 16 chunk positions, per pass).
// K is read with ds_read_b128: the 16 lanes of a lane group read 16
// consecutive rows at one logical chunk.  With 256-byte rows (HD = 128)
// chunk c of row r sits at c ^ (r & 15); with 128-byte rows (HD = 64) two
// rows share a pass, so c ^ ((r >> 1) & 7).
// V is read with ds_read_b64_tr_b16: per 16 lanes, 4 consecutive rows, 32
// bytes (a chunk pair) each.  With 256-byte rows the pair index moves with
// r & 7; with 128-byte rows (8 rows per 32 lanes, two per pass position)
// with (r >> 1) & 3.  Every swizzle depends only on bits of the row that are
// fixed per lane, which lets each fragment address be a per-lane base plus
// an immediate offset.
template <int HD> __device__ __forceinline__ int swz_k(int row) { return HD == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int HD> __device__ __forceinline__ int swz_v(int row) { return HD == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1); }

// The kernel's arguments in the kernel-argument segment, through a pointer
// the compiler cannot see through: values read from it are read again at
// each use site instead of being held in scalar registers from the kernel's
// entry, which keeps the item loop of a persistent work-group from holding
// every argument across its key loop.
typedef const __attribute__((address_space(4))) AttnParams KParams;
template <bool OPAQUE>
__device__ __forceinline__ KParams& kernel_params() {
    auto kp = __builtin_amdgcn_kernarg_segment_ptr();
    if (OPAQUE) __asm__ volatile("" : "+s"(kp));
    return *(KParams*)kp;
}

__device__ __forceinline__ int map_block(int bid, int n, int order) {
    if (order != ORDER_XCD) return bid;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Work item at position pos of the map above when every batch entry has its
// own key count (no mask).  All M = H * n_qtiles items of an entry cost the
// same, but entries differ, so numbering the items entry by entry would
// leave whole XCDs with the long entries.  Instead the positions are cut in
// 8 groups (the eighth of the positions each XCD receives); group x holds,
// for each entry, the items [x M / 8, (x + 1) M / 8) of that entry (runs of
// consecutive query tiles, so a head's tiles share one XCD's L2), entry
// after entry, the entry with the most keys first: a longest-first list
// schedule on every XCD.  The entries are ranked in-wave when there are at
// most 64 of them (ties by index); with more they run in index order.
// Called with all 64 lanes of the wave active.
// The query and key rows of batch entry b with per-entry counts: packed
// sequences (cu_q, cu_k: prefix sums of the rows, clamped so a row never
// falls outside the packed tensors or past the longest length the call
// names), or a common query count and a key count per entry (kv_lens).
template <class PT>
__device__ __forceinline__ int entry_keys(PT& p, int b, int* first = nullptr) {
    if (p.cu_k) {
        const int s = min(max(p.cu_k[b], 0), p.total_k);
        const int e = min(max(p.cu_k[b + 1], s), p.total_k);
        if (first) *first = s;
        return min(e - s, p.Skv);
    }
    if (first) *first = 0;
    return min(max(p.kv_lens[b], 0), p.Skv);
}
template <class PT>
__device__ __forceinline__ int entry_queries(PT& p, int b, int* first) {
    if (p.cu_q) {
        const int s = min(max(p.cu_q[b], 0), p.total_q);
        const int e = min(max(p.cu_q[b + 1], s), p.total_q);
        *first = s;
        return min(e - s, p.Sq);
    }
    *first = 0;
    return p.Sq;
}

template <class PT>
__device__ __forceinline__ void kvlen_item(int pos, PT& p, int& qt, int& bh) {
    const int64_t M = (int64_t)p.H * p.n_qtiles;
    int x = 0;
    int64_t base = 0;
    for (; x < 7; x++) {
        const int64_t c = ((x + 1) * M >> 3) - (x * M >> 3);
        if (pos < base + p.B * c) break;
        base += p.B * c;
    }
    // group x is never empty here: pos < B * M and group 7 holds M - 7M/8 >= 1 items per entry
    const int64_t c = ((x + 1) * M >> 3) - (x * M >> 3);
    const int64_t t = pos - base;
    const int r = (int)(t / c);                              // rank of the entry
    const int k = (int)((x * M >> 3) + t % c);               // item within the entry
    int b = r;
    if (p.B <= 64) {
        const int lane = threadIdx.x & 63;
        const int len = lane < p.B ? entry_keys(p, lane) : -1;
        int rank = 0;
        for (int u = 0; u < p.B; u++) {
            const int lu = __builtin_amdgcn_readlane(len, u);
            rank += (lu > len || (lu == len && u < lane)) ? 1 : 0;
        }
        const unsigned long long m = __ballot(lane < p.B && rank == r);
        b = __builtin_amdgcn_readfirstlane(__ffsll(m) - 1);
    }
    qt = k % p.n_qtiles;
    bh = b * p.H + k / p.n_qtiles;
}

// ------------------------------------------------------------ main kernel
// Workgroup barrier between key tiles.  Every wave waits for its own K/V DMA
// (vmcnt) explicitly before it, so the barrier itself only needs the LDS
// reads done (lgkmcnt); the "memory" clobber and the scheduling barriers
// keep the compiler from moving any instruction across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);   // no instruction may be scheduled across a phase boundary
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// NWT waves (8, or 4 for short key ranges), each owning 32 query rows of the
// work item; see the file header for the per-tile schedule.
template <int HD, bool CPOS, bool CAUSAL, bool KVL, int PMODE, int NWT>
__global__ __launch_bounds__(NWT * 64, 8 / NWT) void attn_fwd_main(const AttnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    static_assert(NWT == 8 || NWT == 4, "8 waves (one work-group per CU) or 4 (two)");
    constexpr int NW = NWT;                      // waves per work-group
    constexpr int BM = NW * 16 * NQB;            // query rows per work item
    static_assert(HD == 128 || HD == 64, "head dimension 128 or 64");
    constexpr int ROW_BYTES = HD * 2;
    constexpr int TILE_BYTES = BN * ROW_BYTES;   // 16 KiB (HD = 128) or 8 KiB
    constexpr int NKS = HD / 32;                 // k-steps of S^T = K Q^T
    constexpr int NDB = HD / 16;                 // 16-dim blocks of O
    constexpr int SS = 4 * NKS;                  // fragment steps of S^T (4 key blocks x NKS)
    constexpr int ST = SS + 2 * NDB;             // all steps of a tile (+ NDB x 2 k-steps of O^T)
    // Row sums of the weights on the matrix core (ones^T P^T, 2 MFMAs per
    // query block and tile) instead of VALU adds: the SIMD's VALU work, which
    // overlaps the matrix work only in part, shrinks by a third of the
    // softmax.  Always at HD = 64 (the softmax outweighs the MFMAs there); at
    // HD = 128 in the variants without the causal mask or per-entry key
    // counts, the ones whose registers take it (those two spill inside the
    // key loop with it).
    constexpr bool MFMA_SUM = HD == 64 || (!CAUSAL && !KVL);
    // Four distinct LDS objects (K and V, two buffers each): with the buffer
    // choice a compile-time constant the compiler can tell that a DMA into one
    // buffer does not alias reads of another and does not wait for it.
    __shared__ __attribute__((aligned(1024))) uint8_t sk0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sk1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sv0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sv1[TILE_BYTES];

    // ---- work items
    // Blocks [0, n_full) take the unsplit items (in XCD-aware order); the
    // remaining blocks take the key ranges of the split items.  Without the
    // causal mask or per-entry key counts every item costs the same, and an
    // 8-wave grid of G blocks at head dimension 128, fewer than the plan's,
    // is persistent: block i runs the plan's blocks i, i + G, i + 2G, ... (G
    // a multiple of 8, so each lands on the XCD it would have had) and
    // fetches the next one's Q and first K tile during the current item's
    // last iteration.  (Two 4-wave work-groups per CU already overlap one's
    // item boundary with the other's matrix work; kept persistent, they run
    // in step and their epilogues coincide, which measured slower.  At head
    // dimension 64 the item loop costs more registers than it saves time.)
    constexpr bool PERSIST = !KVL && NWT == 8 && HD == 128;
    // A persistent work-group's next Q tile, staged by DMA during the current
    // item's last iteration: per wave, its NQB x NKS fragments in operand
    // order (fragment n of lane l at byte 1024 n + 16 l), so that no register
    // holds it across the last iteration and the epilogue (held in registers,
    // the compiler spilled it, and the spill store waited for the load from
    // memory), and the next item reads each fragment with one conflict-free
    // ds_read_b128.  Its smaller alignment places it after the four tile
    // buffers, whose addresses then stay below 64 KiB and fold into the
    // 16-bit offset field of every fragment read (below them, each read
    // needed its own address add).
    constexpr int QSTAGE_WAVE = NQB * NKS * 1024;
    __shared__ __attribute__((aligned(16))) uint8_t sq_stage[PERSIST ? NW * QSTAGE_WAVE : 16];
    struct Loc {
        int item, split, nsplit, qt, b, h, hk, coff, kv_begin, kv_end;
        int sq;                          // query rows of the entry
        int64_t qoff, koff, lse_off;     // elements to the entry's row 0 of head h (q, o), hk (k, v); lse index
    };
    // The element offsets of an item's rows (per-entry counts: from the
    // locator; otherwise from b and h where they are used, as few values as
    // possible live across the key loop)
    auto q_off = [&](KParams& p, const Loc& L) __attribute__((always_inline)) -> int64_t {
        return KVL ? L.qoff : (int64_t)L.b * p.q_batch + (int64_t)L.h * p.q_head;
    };
    auto k_off = [&](KParams& p, const Loc& L) __attribute__((always_inline)) -> int64_t {
        return KVL ? L.koff : (int64_t)L.b * p.kv_batch + (int64_t)L.hk * p.kv_head;
    };
    auto lse_base = [&](KParams& p, const Loc& L) __attribute__((always_inline)) -> int64_t {
        return KVL ? L.lse_off : ((int64_t)L.b * p.H + L.h) * p.Sq;
    };
    auto locate = [&](KParams& p, int vb) __attribute__((always_inline)) -> Loc {
        Loc L;
        if (vb < p.n_full) {
            L.item = map_block(vb, p.n_full, p.block_order);
            L.split = 0;
            L.nsplit = 1;
        } else {
            const int tb = vb - p.n_full;
            L.item = p.n_full + tb / p.kv_splits;
            L.split = tb % p.kv_splits;
            L.nsplit = p.kv_splits;
        }
        int bh;
        if (CAUSAL) {
            // Causal items run longest first: items [0, BH) are the last query
            // tile of every head, then the second last, ...; the block order is
            // naive, so the XCD of item i is i mod 8 and each XCD gets an equal
            // share of every tile length.  Within a tile length, XCD x takes
            // heads [x*BH/8, (x+1)*BH/8), which share key/value heads under GQA.
            const int BH = p.B * p.H;
            const int slot = L.item % BH;
            L.qt = p.n_qtiles - 1 - L.item / BH;
            bh = (BH % 8 == 0) ? (slot % 8) * (BH / 8) + slot / 8 : slot;
        } else if (KVL) {
            kvlen_item(L.item, p, L.qt, bh);
        } else {
            L.qt = L.item % p.n_qtiles;
            bh = L.item / p.n_qtiles;
        }
        L.h = bh % p.H;
        L.b = bh / p.H;
        L.hk = L.h / p.group;                      // key/value head of query head h
        // keys and queries of this batch entry (per-entry lengths: never
        // split) and the causal offset that aligns its queries with the last
        // of its keys
        int q0 = 0, k0 = 0;
        const int kvl = KVL ? entry_keys(p, L.b, &k0) : p.Skv;
        L.sq = KVL ? entry_queries(p, L.b, &q0) : p.Sq;
        L.coff = KVL ? kvl - L.sq : p.causal_off;
        L.qoff = L.koff = L.lse_off = 0;
        if (KVL && p.cu_q) {
            // packed sequences: rows of all entries in one tensor, lse [H][total rows]
            L.qoff = (int64_t)q0 * p.q_row + (int64_t)L.h * p.q_head;
            L.koff = (int64_t)k0 * p.kv_row + (int64_t)L.hk * p.kv_head;
            L.lse_off = (int64_t)L.h * p.total_q + q0;
        } else if (KVL) {
            L.qoff = (int64_t)L.b * p.q_batch + (int64_t)L.h * p.q_head;
            L.koff = (int64_t)L.b * p.kv_batch + (int64_t)L.hk * p.kv_head;
            L.lse_off = ((int64_t)L.b * p.H + L.h) * p.Sq;
        }
        // split s covers key tiles [s*T/ns, (s+1)*T/ns) of the T tiles: never empty for ns <= T
        L.kv_begin = (int)(((int64_t)L.split * p.n_kv_tiles) / L.nsplit) * BN;
        L.kv_end = min(kvl, (int)(((int64_t)(L.split + 1) * p.n_kv_tiles) / L.nsplit) * BN);
        if (CAUSAL) {
            // keys up to the diagonal of the tile's last row (never split)
            const int last_row = min(L.sq, (L.qt + 1) * BM) - 1;
            L.kv_end = min(L.kv_end, last_row + L.coff + 1);
        }
        return L;
    };
    // Buffer descriptor of a head's K or V rows [0, kv_end) (rows of
    // kv_row_bytes): reads at or beyond kv_end return zero.
    auto kv_rsrc = [&](const char* base, int kv_end, int kv_row_bytes) __attribute__((always_inline)) -> i32x4 {
        const uint32_t nrec = kv_end > 0 ? (uint32_t)((int64_t)(kv_end - 1) * kv_row_bytes + ROW_BYTES) : 0u;
        const uint64_t a = (uint64_t)(uintptr_t)base;
        return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)nrec, 0x00020000};
    };
    // ---- Q fragments (operand B of S^T = K Q^T): lane (g, j) holds query row
    // 16*qb + j of this wave, dims 32*ks + 8*g .. +7, for the whole key loop.
    // Rows past Sq are clamped (their results are never stored).
    bf16x8 qf[NQB][NKS];

    // The plan's block that this work-group runs in round k: block k*G + w
    // (w = the work-group, G = the grid).  Causal items run longest first, so
    // odd rounds walk back (the groups of 8 in reverse order, each block's
    // position within its group, and so its XCD, kept): a work-group that
    // had one of the longest items in a round gets one of the shortest in the
    // next, and the work-groups' totals stay close.
    auto round_block = [&](KParams& p, int k) __attribute__((always_inline)) -> int {
        const int w = blockIdx.x, G = p.grid;
        const int off = (CAUSAL && (k & 1) && (G & 7) == 0) ? G - 8 - (w & ~7) + (w & 7) : w;
        return k * G + off;
    };
    int vb = blockIdx.x;
    int round = 0;             // this work-group's item count so far
    bool prefetched = false;   // this item's Q and first K tile came with the previous item
    for (;;) {
        // The lane indices, from an opaque copy of the thread index: nothing
        // derived from them (fragment and DMA addresses, row offsets) is
        // hoisted out of the item loop and held across the key loop.
        int tid = threadIdx.x;
        if (PERSIST) __asm__ volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
        const int g = lane >> 4;       // lane group (0..3)
        const int j = lane & 15;       // lane within group
        auto load_q = [&](KParams& p, const uint16_t* qb_base, int qrow0, int sq) __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) {
                const int row = min(qrow0 + qb * 16 + j, sq - 1);
                const uint16_t* src = qb_base + (int64_t)row * p.q_row + 8 * g;
#pragma unroll
                for (int ks = 0; ks < NKS; ks++) qf[qb][ks] = *(const bf16x8*)(src + 32 * ks);
            }
        };
        KParams& P = kernel_params<PERSIST>();
        const Loc L = locate(P, vb);
        const int kv_row_bytes = (int)(P.kv_row * 2);
        const int item = L.item, split = L.split, nsplit = L.nsplit, qt = L.qt;
        const int coff = L.coff, kv_begin = L.kv_begin, kv_end = L.kv_end, sq = L.sq;
        const int T = (kv_end - kv_begin + BN - 1) / BN;

        const uint16_t* qbase = P.q + q_off(P, L);
        const char* kbase = (const char*)(P.k + k_off(P, L));
        const char* vbase = (const char*)(P.v + k_off(P, L));

        // an item past the last query row of its entry (packed sequences of
        // different lengths): nothing to do
        if (KVL && qt * BM >= sq) return;
        if ((CAUSAL || KVL) && kv_end <= kv_begin) {
            // No query row of the tile sees a key (a causal tile entirely above
            // the diagonal, or a batch entry with no keys): its rows are zeros
            // and their log-sum-exp is -inf.  Uniform across the work-group,
            // before any barrier or DMA.
            uint16_t* obase = P.o + q_off(P, L);
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) {
                const int row = qt * BM + wave * 16 * NQB + qb * 16 + j;
                if (row >= sq) continue;
#pragma unroll
                for (int db = 0; db < NDB; db++) *(uint2*)(obase + (int64_t)row * P.q_row + 4 * g + 16 * db) = uint2{0u, 0u};
                if (P.lse && g == 0) P.lse[lse_base(P, L) + row] = -__builtin_inff();
            }
            if (!PERSIST) return;
            // a persistent work-group goes on with its next item (nothing was
            // prefetched for it here)
            vb = round_block(P, ++round);
            if (vb >= P.n_blocks) return;
            prefetched = false;
            continue;
        }

        // The first four waves issue all K/V DMA: lane l of wave w in round r
        // lands at LDS slot (4*r + w)*64 + l, i.e. row by row in order: row
        // RPR*r + RPW*w + l / CPR, chunk l % CPR (CPR chunks per row, RPW rows per
        // wave, RPR rows per round: 16, 4, 16 for HD = 128 and 8, 8, 32 for 64);
        // rows RPR apart share the swizzle, so one per-lane source offset serves
        // every round.  The DMA is issued with inline assembly:
        // the compiler then does not track it and inserts no vmcnt wait before
        // LDS reads of other buffers (its alias tracking is lost at loop heads);
        // the issuing waves wait for their DMA explicitly (vmcnt(0)) before the
        // barrier that publishes a tile.
        const bool late = NW == 8 && wave >= 4;   // second wave of each SIMD (see the key loop)
        constexpr int CPR = ROW_BYTES / 16, RPW = 64 / CPR, RPR = 4 * RPW;
        constexpr int DMA_ROUNDS = BN / RPR;
        static_assert(DMA_ROUNDS * RPR == BN && RPR % 16 == 0, "rounds of whole swizzle periods");
        const int dma_row = (wave & 3) * RPW + lane / CPR, dma_chunk = lane % CPR;
        const int dma_off_k = dma_row * kv_row_bytes + ((dma_chunk ^ swz_k<HD>(dma_row)) << 4);
        const int dma_off_v = dma_row * kv_row_bytes + ((dma_chunk ^ swz_v<HD>(dma_row)) << 4);
        const i32x4 krs4 = kv_rsrc(kbase, kv_end, kv_row_bytes), vrs4 = kv_rsrc(vbase, kv_end, kv_row_bytes);
        auto dma16 = [&](const i32x4 rs, uint8_t* dst, int voff, int soff) __attribute__((always_inline)) {
            // the LDS address, the descriptor and the tile offset are
            // wave-uniform; say so, so they stay in scalar registers.  The
            // LDS address is the low half of the generic pointer (the shared
            // aperture sits in the high half): a cast to the LDS address
            // space would add a null test, two scalar instructions per
            // transfer in the MFMA phase.
            const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
            const int so = __builtin_amdgcn_readfirstlane(soff);
            const i32x4 rsu = {__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                               __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
            // m0 (the LDS destination) is written in the same statement as the
            // load, so nothing is scheduled between the two; no other code of the
            // kernel uses m0, which makes the clobber safe.  Handing the address
            // in as an {m0} operand lets the compiler move the write away from
            // the load, and that form gave wrong results here.  An LDS-bound
            // buffer load reads m0 one wait state after a scalar write of it at
            // the earliest (the compiler puts the same s_nop after its own m0
            // write for the builtin form of this load); inline assembly is opaque
            // to the hazard recognizer, so the statement carries the nop itself.
            __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                             :: "s"(lds), "v"(voff), "s"(rsu), "s"(so) : "memory", "m0");
        };
        // Where a K or V tile comes from: a descriptor and the key of its first
        // row.  Keys in place in a paged cache (per-entry counts with a block
        // table): the tile's page -- a page holds whole tiles -- with rows up to
        // the entry's last key in it, and no rows at all for a table entry
        // outside the pool; otherwise the item's descriptor from row 0.
        struct TileSrc {
            i32x4 rs;
            int first;
        };
        auto tile_src = [&](const char* head_base, const i32x4& item_rs, int k0) __attribute__((always_inline)) -> TileSrc {
            if (!KVL || !P.block_table) return TileSrc{item_rs, 0};
            const int i = k0 >> P.page_shift;
            const int first = i << P.page_shift;
            // the table through the constant address space: it does not change
            // during the kernel, so the read is a scalar load (no vector memory
            // wait at the head of the MFMA phase)
            typedef const __attribute__((address_space(4))) int const_int;
            const_int* bt = (const_int*)(uintptr_t)P.block_table;
            const int pg = bt[(int64_t)L.b * P.pages_per_seq + i];
            const bool ok = pg >= 0 && pg < P.num_pages;
            const int end = min(kv_end, first + (1 << P.page_shift));
            const char* pb = head_base + (ok ? ((int64_t)pg << P.page_shift) * kv_row_bytes : (int64_t)0);
            return TileSrc{kv_rsrc(pb, ok ? end - first : 0, kv_row_bytes), first};
        };
        // round r of the K (or V) tile that starts at key k0, from src
        auto dma_k = [&](int r, const TileSrc& src, int k0, uint8_t* dst) __attribute__((always_inline)) {
            dma16(src.rs, dst + ((r * 4 + (wave & 3)) * 64) * 16, dma_off_k, (k0 - src.first + RPR * r) * kv_row_bytes);
        };
        auto dma_v = [&](int r, const TileSrc& src, int k0, uint8_t* dst) __attribute__((always_inline)) {
            dma16(src.rs, dst + ((r * 4 + (wave & 3)) * 64) * 16, dma_off_v, (k0 - src.first + RPR * r) * kv_row_bytes);
        };
        const int qrow0 = qt * BM + wave * 16 * NQB;   // first query row of this wave
        if (!prefetched) {
            if (!late) {
                const TileSrc src = tile_src(kbase, krs4, kv_begin);
#pragma unroll
                for (int r = 0; r < DMA_ROUNDS; r++) dma_k(r, src, kv_begin, sk0);
            }
            load_q(P, qbase, qrow0, sq);
        } else if (PERSIST) {
            // the fragments this wave staged during the previous item (its own
            // transfers, complete since that item's epilogue wait)
#pragma unroll
            for (int qb = 0; qb < NQB; qb++)
#pragma unroll
                for (int ks = 0; ks < NKS; ks++)
                    qf[qb][ks] = *(const LDS_AS bf16x8*)(LDS_AS const uint8_t*)(sq_stage + wave * QSTAGE_WAVE + (qb * NKS + ks) * 1024 + lane * 16);
        }
        f32x4 o_acc[NDB][NQB];
#pragma unroll
        for (int db = 0; db < NDB; db++)
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) o_acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        float moff[NQB], l_run[NQB];    // power-of-two offset of the weights (integer-valued), row-sum partials
        f32x4 l_acc[NQB];               // MFMA_SUM: row sums, every element the lane's query
        f32x4 bias4[NQB];               // c > 0: S^T accumulates from -moff/c, so c * S^T = x - moff
#pragma unroll
        for (int qb = 0; qb < NQB; qb++) {
            moff[qb] = 0.f; l_run[qb] = 0.f;
            bias4[qb] = f32x4{0.f, 0.f, 0.f, 0.f}; l_acc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const bf16x8 ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                              (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
        const float rc = 1.0f / P.c;
        f32x4 s_acc[4][NQB];
        bf16x8 pf[NQB][2];
        const float c = P.c;

        // ---- MFMA phase: steps [S0, S1) of a fixed sequence of ST fragment steps.
        // Steps 0..SS-1 compute S^T = K Q^T: step 4*ks + kb reads the K fragment of
        // key block kb, k-step ks (one ds_read_b128: lane (g, j) gets row 16*kb + j,
        // dims 32*ks + 8*g .. +7) and feeds NQB MFMAs; k-steps are the outer index
        // so consecutive MFMAs hit different accumulators.  The score fragment of
        // lane (g, j) then holds query j and keys 16*kb + 4*g + r, r = 0..3.
        // Steps SS..ST-1 compute O^T += V^T P^T: step SS + NDB*ks + db reads the
        // V^T fragment of dim block db for the 32 keys of step ks with two
        // ds_read_b64_tr_b16 (rows 32*ks + 16*hf + 4*g + r), matching the keys
        // of P's elements 4*hf + r.  Fragment reads run PF steps ahead of their
        // MFMAs so LDS latency hides behind the matrix core.
        int k_addr[NKS], v_addr[NDB];   // per-lane byte offsets within a tile
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) k_addr[ks] = j * ROW_BYTES + ((((4 * ks + g) ^ swz_k<HD>(j))) << 4);
#pragma unroll
        for (int db = 0; db < NDB; db++) {
            const int row = 4 * g + (j >> 2);                    // + 32*ks + 16*hf (multiples of 8)
            const int chunk = (2 * db + ((j & 3) >> 1)) ^ swz_v<HD>(row);
            v_addr[db] = row * ROW_BYTES + (chunk << 4) + ((j & 1) << 3);
        }
        auto read_frag = [&](int st, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) -> bf16x8 {
            if (st < SS) {
                const int kb = st & 3, ks = st >> 2;
                return *(const LDS_AS bf16x8*)(LDS_AS const uint8_t*)(kt + k_addr[ks] + kb * 16 * ROW_BYTES);
            }
            const int db = (st - SS) % NDB, ks = (st - SS) / NDB;
            bf16x4 half[2];
#pragma unroll
            for (int hf = 0; hf < 2; hf++) {
                const LDS_AS s16x4* src = (const LDS_AS s16x4*)(LDS_AS const uint8_t*)(vt + v_addr[db] + (32 * ks + 16 * hf) * ROW_BYTES);
                half[hf] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)src));
            }
            return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
        };
        auto use_frag = [&](int st, const bf16x8 f) __attribute__((always_inline)) {
            if (st < SS) {
                const int kb = st & 3, ks = st >> 2;
#pragma unroll
                for (int qb = 0; qb < NQB; qb++)
                    s_acc[kb][qb] = mfma16x16x32(f, qf[qb][ks], ks == 0 ? (CPOS ? bias4[qb] : f32x4{0.f, 0.f, 0.f, 0.f}) : s_acc[kb][qb]);
            } else {
                const int db = (st - SS) % NDB, ks = (st - SS) / NDB;
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) o_acc[db][qb] = mfma16x16x32(f, pf[qb][ks], o_acc[db][qb]);
                if (MFMA_SUM && db == NDB - 1) {
                    // ones^T P^T: every lane gets the sum of the step's 32 bf16
                    // weights of its query (exact products, fp32 sums)
#pragma unroll
                    for (int qb = 0; qb < NQB; qb++) l_acc[qb] = mfma16x16x32(ones8, pf[qb][ks], l_acc[qb]);
                }
            }
        };
        constexpr int PF = 4;   // fragment prefetch distance (steps)
        // The DMA of iteration t (K_{t+1} into kn, V_t into vc) is spread over the
        // issuing waves' MFMA phase, one instruction every STRIDE steps, so the
        // CU's address unit drains it while the matrix core runs instead of
        // stalling a wave that issues all of it at once.
        constexpr int NDMA = 2 * DMA_ROUNDS;   // instructions per wave and tile
        // The phase has no branch: the issuing group is a compile-time choice
        // (LATE), and past the last tile the K DMA re-reads that tile into the
        // free buffer, so the scheduler sees the whole phase as one region.
        auto mfma_phase = [&](const uint8_t* kt, const uint8_t* vt, auto s0c, auto s1c, int t, uint8_t* kn, uint8_t* vc,
                              auto latec) __attribute__((always_inline)) {
            constexpr int S0 = decltype(s0c)::value, S1 = decltype(s1c)::value;
            constexpr bool LATE = decltype(latec)::value;
            constexpr int STRIDE = (S1 - S0) / NDMA;
            static_assert(S0 != 0 || STRIDE * NDMA <= S1 - S0, "the DMA fits the phase");
            // Opaque per-lane offsets: stops the compiler from hoisting every
            // buffer x fragment address combination out of the loop (and spilling
            // them); each phase adds its buffer base to these offsets instead.
#pragma unroll
            for (int i = 0; i < NKS; i++) __asm__ volatile("" : "+v"(k_addr[i]));
#pragma unroll
            for (int i = 0; i < NDB; i++) __asm__ volatile("" : "+v"(v_addr[i]));
            // the sources of this iteration's transfers (K_{t+1}, V_t), looked up
            // before the first fragment read, so a page-table read waits for no
            // LDS read
            const int kk0 = kv_begin + min(t + 1, T - 1) * BN, vk0 = kv_begin + t * BN;
            TileSrc ksrc{krs4, 0}, vsrc{vrs4, 0};
            if (KVL && S0 == 0 && !LATE) {
                ksrc = tile_src(kbase, krs4, kk0);
                vsrc = tile_src(vbase, vrs4, vk0);
                __asm__ volatile("" :: "s"(ksrc.rs), "s"(vsrc.rs));
            }
            // a persistent work-group's last iteration (P.V only) reads two
            // steps ahead: its accumulators and the epilogue's values leave
            // fewer registers there
            constexpr int PFL = PERSIST && S0 != 0 ? 2 : PF;
            bf16x8 fr[PFL];
#pragma unroll
            for (int st = S0; st < S0 + PFL && st < S1; st++) fr[(st - S0) % PFL] = read_frag(st, kt, vt);
#pragma unroll
            for (int st = S0; st < S1; st++) {
                const bf16x8 cur = fr[(st - S0) % PFL];
                if (st + PFL < S1) fr[(st - S0) % PFL] = read_frag(st + PFL, kt, vt);
                if (S0 == 0 && (st - S0) % STRIDE == 0 && (st - S0) / STRIDE < NDMA && !LATE) {
                    const int k = (st - S0) / STRIDE;     // K and V rounds alternate
                    if (k & 1) dma_v(k >> 1, vsrc, vk0, vc);
                    else dma_k(k >> 1, ksrc, kk0, kn);
                }
                use_frag(st, cur);
            }
            // keep the interleave: the reads of step st+PFL, then the MFMAs of step st
#pragma unroll
            for (int st = S0; st < S0 + PFL && st < S1; st++) {
                if (st < SS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
#pragma unroll
            for (int st = S0; st < S1; st++) {
                if (st + PFL < S1) {
                    if (st + PFL < SS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                if (MFMA_SUM && st >= SS && (st - SS) % NDB == NDB - 1) __builtin_amdgcn_sched_group_barrier(0x008, 2 * NQB, 0);
                else __builtin_amdgcn_sched_group_barrier(0x008, NQB, 0);
            }
        };
        using C0 = std::integral_constant<int, 0>;
        using CS = std::integral_constant<int, SS>;
        using CT = std::integral_constant<int, ST>;

        // Two weights (>= 0, or NaN) to packed bf16 in the weights' rounding mode.
        // Nearest-even: the hardware conversion.  Ties away: the same conversion
        // after setting the lowest fp32 bit, which turns an exact tie into a value
        // just above it and changes no other decision (an infinite weight would
        // become NaN, but it only arises in rows whose output is NaN anyway).
        // Toward zero: the high half of the bit pattern, after clamping every NaN
        // to the canonical one so truncation cannot make it an infinity.
        auto weight_pair = [&](const f32x2 two) __attribute__((always_inline)) -> bf16x2 {
            if (PMODE == ROUND_RTNE) return __builtin_convertvector(two, bf16x2);
            if (PMODE == ROUND_RTNA) {
                const f32x2 up = {__uint_as_float(__float_as_uint(two[0]) | 1u), __uint_as_float(__float_as_uint(two[1]) | 1u)};
                return __builtin_convertvector(up, bf16x2);
            }
            const uint32_t u0 = min(__float_as_uint(two[0]), 0x7fc00000u);
            const uint32_t u1 = min(__float_as_uint(two[1]), 0x7fc00000u);
            return __builtin_bit_cast(bf16x2, (u1 & 0xffff0000u) | (u0 >> 16));
        };
        // Weights of query block qb against offset m: p = 2^(x - m) (v_exp_f32),
        // rounded to bf16 pairs for the P.V product (pf), and this lane's sum of
        // those bf16 weights -- the row sum adds the same values the product uses,
        // so O is normalised by exactly its own weights.
        auto weights = [&](int qb, float m, auto biasc) __attribute__((always_inline)) -> float {
            constexpr bool BIASED = decltype(biasc)::value;   // S^T already holds s - moff/c: exponent = c * S^T
            const float negm = -m;
            f32x4 pv4[4];
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float x = BIASED ? s_acc[kb][qb][r] * c
                                           : (CPOS ? __builtin_fmaf(s_acc[kb][qb][r], c, negm) : (s_acc[kb][qb][r] + negm));
                    pv4[kb][r] = __builtin_amdgcn_exp2f(x);
                }
            float tlo = 0.f, thi = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                bf16x2 pr[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4& src = pv4[2 * ks + (i >> 1)];
                    const f32x2 two = {src[2 * (i & 1)], src[2 * (i & 1) + 1]};
                    pr[i] = weight_pair(two);
                    if (!MFMA_SUM) {
                        // the two bf16 weights as fp32 (bit placement), summed with
                        // plain adds: v_dot2c would wait for the matrix core a
                        // co-resident wave keeps busy
                        const uint32_t u = __builtin_bit_cast(uint32_t, pr[i]);
                        tlo += __uint_as_float(u << 16);
                        thi += __uint_as_float(u & 0xffff0000u);
                    }
                }
                const bf16x4 lo = __builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3);
                const bf16x4 hi = __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3);
                pf[qb][ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            return tlo + thi;
        };
        // ceil of the tile's largest x for query block qb (NaN-propagating
        // v_maximum3_f32 in the lane, then across the 4 lanes of a row)
        auto tile_max_ceil = [&](int qb) __attribute__((always_inline)) -> float {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) mx = __builtin_elementwise_maximum(mx, s_acc[kb][qb][r]);
            mx = rowmax4(mx);
            if (CPOS) mx *= c;
            return ceilf(mx);
        };
        auto set_bias = [&](int qb) __attribute__((always_inline)) {
            if (CPOS) {
                const float bb = -moff[qb] * rc;
                bias4[qb] = f32x4{bb, bb, bb, bb};
            }
        };

        // ---- online softmax of S_t with a power-of-two running offset.
        auto softmax = [&](int t, auto firstc) __attribute__((always_inline)) {
            constexpr bool FIRST = decltype(firstc)::value;
            const int valid = kv_end - (kv_begin + t * BN);   // keys of this tile inside the range
            // Keys outside the range are masked by select, never by arithmetic:
            // key 16*kb + 4*g + r of the tile is inside iff 16*kb + r < lim[qb],
            // lim = valid - 4*g, and under the causal mask also key <= row + off.
            // With c > 0 only a ragged last tile or a tile crossing this wave's
            // diagonal needs it, and one branch covers both query blocks so the
            // compares stay inside it.
            const int ts = kv_begin + t * BN;              // first key of the tile
            const bool diag = CAUSAL && ts + BN - 1 > qrow0 + coff;
            int lim[NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) {
                lim[qb] = valid - 4 * g;
                if (CAUSAL) lim[qb] = min(lim[qb], qrow0 + qb * 16 + j + coff - ts + 1 - 4 * g);
            }
            if (CPOS && (valid < BN || diag)) {
#pragma unroll
                for (int qb = 0; qb < NQB; qb++)
#pragma unroll
                    for (int kb = 0; kb < 4; kb++)
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            s_acc[kb][qb][r] = (16 * kb + r < lim[qb]) ? s_acc[kb][qb][r] : -__builtin_inff();
            }
            if (!CPOS) {
                // general scale (c <= 0): x = s*c explicitly, masked keys -> -inf
#pragma unroll
                for (int qb = 0; qb < NQB; qb++)
#pragma unroll
                    for (int kb = 0; kb < 4; kb++)
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            s_acc[kb][qb][r] = (16 * kb + r < lim[qb]) ? s_acc[kb][qb][r] * c : -__builtin_inff();
            }
            if (FIRST) {
                // first tile: the offset starts at ceil(max x) (0 for a row whose
                // scores are all -inf or NaN; its weights are then 0 or NaN)
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) {
                    const float m = tile_max_ceil(qb);
                    moff[qb] = __builtin_isfinite(m) ? m : 0.f;
                    l_run[qb] = weights(qb, moff[qb], std::false_type{});
                    set_bias(qb);
                }
                return;
            }
            // Later tiles: weights against the running offset, with no max.  A
            // weight can exceed 2^16 only if its lane's tile sum does (with the
            // MFMA row sums: only if the lane's largest exponent exceeds 16); then
            // (rare: the row max moved far past the offset) the tile is redone with
            // the offset at ceil(max) and O and l rescaled by the exact power of two.
            float tsum[NQB];
            bool big = false;
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) {
                if (MFMA_SUM) {
                    float mx = -__builtin_inff();
#pragma unroll
                    for (int kb = 0; kb < 4; kb++)
#pragma unroll
                        for (int r = 0; r < 4; r++) mx = __builtin_elementwise_maximum(mx, s_acc[kb][qb][r]);
                    big |= (CPOS ? mx * c : mx - moff[qb]) > 16.0f;
                }
                tsum[qb] = weights(qb, moff[qb], std::integral_constant<bool, CPOS>{});
                if (!MFMA_SUM) big |= tsum[qb] > WEIGHT_LIMIT;
            }
            if (__builtin_amdgcn_ballot_w64(big) != 0) {
                float alpha[NQB];
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) {
                    // with c > 0 the scores hold s - moff/c: x = c * S^T + moff
                    const float m_new = fmaxf(moff[qb], tile_max_ceil(qb) + (CPOS ? moff[qb] : 0.f));
                    alpha[qb] = ldexpf(1.0f, (int)fmaxf(moff[qb] - m_new, -200.f));
                    tsum[qb] = weights(qb, CPOS ? m_new - moff[qb] : m_new, std::false_type{});
                    moff[qb] = m_new;
                    set_bias(qb);
                    l_run[qb] *= alpha[qb];
                    l_acc[qb] *= alpha[qb];
                }
#pragma unroll
                for (int db = 0; db < NDB; db++)
#pragma unroll
                    for (int qb = 0; qb < NQB; qb++) o_acc[db][qb] *= alpha[qb];
            }
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) l_run[qb] += tsum[qb];
        };

        // ---- key loop: one barrier per tile.  Iteration t computes S_t = K_t Q^T
        // and O += V_{t-1}^T P_{t-1}^T (with the DMA of K_{t+1} into the buffer
        // K_{t-1} used and of V_t into V_{t-2}'s), then the softmax of S_t; the
        // issuing waves wait for their DMA before the barrier.  Iteration 0 has
        // no P.V step and iteration T (past the last tile) only the P.V step; the
        // steady-state loop in between is branch-free in vector state, which
        // keeps the accumulators in place.  Before it, this wave's share of K_0
        // and its Q have landed (a prefetched item's before the previous item's
        // stores, so no store is waited for here) and the barrier publishes K_0.
        if (!prefetched) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        lds_barrier();
        // Waves w and w + 4 share a SIMD.  The second group takes the barrier
        // between its MFMA phase and its softmax instead of after the softmax, so
        // between two barriers it runs the softmax of S_{t-1} and then the MFMA
        // phase of tile t while the first group runs the MFMA phase of tile t and
        // then the softmax of S_t: the two waves of a SIMD are in opposite phases
        // and one's softmax fills the gaps of the other's MFMAs.  Both groups
        // read K_t and V_{t-1} between the same two barriers, so the buffer
        // protocol is the same for both.
        auto sync = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(0x0f70);
            lds_barrier();
        };
        auto iter = [&](int t, uint8_t* kc, uint8_t* kn, uint8_t* vc, uint8_t* vp, auto s0c, auto s1c, auto latec) __attribute__((always_inline)) {
            constexpr bool LATE = decltype(latec)::value;
            // A wave in its MFMA phase takes issue priority over one in its
            // softmax, so the matrix core of a SIMD stays fed; the softmax VALU
            // work fills the MFMA phase's gaps.
            __builtin_amdgcn_s_setprio(1);
            mfma_phase(kc, vp, s0c, s1c, t, kn, vc, latec);
            __builtin_amdgcn_s_setprio(0);
            // The last iteration (P.V only) ends without a barrier: no LDS
            // buffer is written after it before the next item's first barrier.
            constexpr bool LAST = decltype(s0c)::value != 0;
            if (LATE && !LAST) sync();
            if (!LAST)
                softmax(t, std::integral_constant<bool, decltype(s1c)::value == SS>{});
            if (!LATE && !LAST) sync();
        };
        // The next block of a persistent work-group: each wave's rows of its Q
        // tile into the wave's stage and, from the issuing waves, its first K
        // tile into sk0 (no K buffer is read in the last iteration).  Q rows
        // past the entry's end read as zero (the descriptor ends at its last
        // row; one-block-per-item runs repeat the last row instead, and
        // neither kind can trigger the tile redo, so both give the same bits).
        auto prefetch_next = [&]() __attribute__((always_inline)) {
            KParams& PN = kernel_params<true>();
            const int nv = round_block(PN, round + 1);
            if (nv >= PN.n_blocks) return;
            const Loc N = locate(PN, nv);
            const uint16_t* nq = PN.q + q_off(PN, N);
            if (!late) {
                const char* nk = (const char*)(PN.k + k_off(PN, N));
                const i32x4 nrs = kv_rsrc(nk, N.kv_end, (int)(PN.kv_row * 2));
#pragma unroll
                for (int r = 0; r < DMA_ROUNDS; r++)
                    dma16(nrs, sk0 + ((r * 4 + (wave & 3)) * 64) * 16, dma_off_k, (N.kv_begin + RPR * r) * kv_row_bytes);
            }
            const int qrow_bytes = (int)(PN.q_row * 2);
            const i32x4 qrs = kv_rsrc((const char*)(nq + (int64_t)N.qt * BM * PN.q_row), min(BM, N.sq - N.qt * BM), qrow_bytes);
            const int qvoff = j * qrow_bytes + 16 * g;   // lane (g, j): row 16 qb + j, dims 32 ks + 8 g
#pragma unroll
            for (int qb = 0; qb < NQB; qb++)
#pragma unroll
                for (int ks = 0; ks < NKS; ks++)
                    dma16(qrs, sq_stage + wave * QSTAGE_WAVE + (qb * NKS + ks) * 1024, qvoff,
                          (wave * 16 * NQB + 16 * qb) * qrow_bytes + 64 * ks);
        };
        // the key loop, compiled once per wave group
        auto key_loop = [&](auto latec) __attribute__((always_inline)) {
            iter(0, sk0, sk1, sv0, sv1, C0{}, CS{}, latec);
            int t = 1;
            for (; t + 1 < T; t += 2) {
                iter(t, sk1, sk0, sv1, sv0, C0{}, CT{}, latec);
                iter(t + 1, sk0, sk1, sv0, sv1, C0{}, CT{}, latec);
            }
            if (t < T) {
                iter(t, sk1, sk0, sv1, sv0, C0{}, CT{}, latec);
                t++;
            }
            // the last iteration reads neither Q nor a K buffer: the next item's
            // Q fragments and first K tile are fetched under it
            if (PERSIST) prefetch_next();
            if (T & 1) iter(T, sk1, sk0, sv1, sv0, CS{}, CT{}, latec);
            else iter(T, sk0, sk1, sv0, sv1, CS{}, CT{}, latec);
        };
        if (late) key_loop(std::true_type{});
        else key_loop(std::false_type{});

        // ---- epilogue: the 4 lanes of a row hold partial row sums
        float l_row[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; qb++) l_row[qb] = MFMA_SUM ? l_acc[qb][0] : rowsum4(l_run[qb]);

        // A persistent work-group's loads for the next item (issued in the last
        // iteration) complete before this item's stores enter the same counter,
        // so the next item's first barrier waits for no store.
        if (PERSIST) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        if (nsplit == 1) {
            if (P.lse && g == 0) {
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) {
                    const int row = qrow0 + qb * 16 + j;
                    if (row >= sq) continue;
                    float v = (moff[qb] + __builtin_amdgcn_logf(l_row[qb])) * LN2;
                    if (CAUSAL && row + coff < 0) v = -__builtin_inff();
                    P.lse[lse_base(P, L) + row] = v;
                }
            }
            uint16_t* obase = P.o + q_off(P, L);
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) {
                const int row = qrow0 + qb * 16 + j;
                if (row >= sq) continue;
                const float lr = l_row[qb];
                const float inv = 1.0f / lr;
                const bool no_key = CAUSAL && row + coff < 0;
                const Bf16Round rm = bf16_round(P.round_mode);
                uint16_t* dst = obase + (int64_t)row * P.q_row + 4 * g;
#pragma unroll
                for (int db = 0; db < NDB; db++) {
                    f32x4 ov;
#pragma unroll
                    for (int r = 0; r < 4; r++) ov[r] = no_key ? 0.f : div_corrected(o_acc[db][qb][r], lr, inv);
                    uint2 packed;
                    packed.x = bf16_pack2(ov[0], ov[1], rm);
                    packed.y = bf16_pack2(ov[2], ov[3], rm);
                    *(uint2*)(dst + 16 * db) = packed;
                }
            }
        } else {
            // partial results: O (unnormalised, fp32) [item][split][BM][HD], M and l [item][split][BM]
            // (items counted from n_full)
            const int64_t part = (int64_t)(item - P.n_full) * nsplit + split;
            float* ow = P.ws_o + part * (int64_t)BM * HD;
            float* mw = P.ws_ml + part * (int64_t)BM * 2;
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) {
                const int lrow = wave * 16 * NQB + qb * 16 + j;   // row within the tile
#pragma unroll
                for (int db = 0; db < NDB; db++) *(f32x4*)(ow + (int64_t)lrow * HD + 16 * db + 4 * g) = o_acc[db][qb];
                if (g == 0) {
                    mw[2 * lrow] = moff[qb];
                    mw[2 * lrow + 1] = l_row[qb];
                }
            }
        }
        if (!PERSIST) break;
        vb = round_block(P, ++round);
        if (vb >= P.n_blocks) break;
        prefetched = true;
    }
#endif
}

// ---------------------------------------------------------- combine kernel
// One thread per (row, 4 dims): merges the splits of a query tile in split
// order: M = max_s M_s, O = sum_s 2^(M_s - M) O_s / sum_s 2^(M_s - M) l_s.
template <int BM, int HD>
__global__ __launch_bounds__(256) void attn_fwd_combine(const AttnParams p) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)(p.n_items - p.n_full) * BM * (HD / 4);
    if (gid >= total) return;
    const int d4 = (int)(gid % (HD / 4));
    const int64_t r = gid / (HD / 4);
    const int lrow = (int)(r % BM);
    const int sidx = (int)(r / BM);          // index among the split items
    const int item = p.n_full + sidx;
    const int qt = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int h = bh % p.H, b = bh / p.H;
    const int row = qt * BM + lrow;
    if (row >= p.Sq) return;

    const int ns = p.kv_splits;
    const float* mw = p.ws_ml + (int64_t)sidx * ns * BM * 2;
    float M = -__builtin_inff();
    for (int s = 0; s < ns; s++) M = fmaxf(M, mw[(int64_t)s * BM * 2 + 2 * lrow]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int s = 0; s < ns; s++) {
        const float ms = mw[(int64_t)s * BM * 2 + 2 * lrow];
        const float ls = mw[(int64_t)s * BM * 2 + 2 * lrow + 1];
        const float wgt = ldexpf(1.0f, (int)fmaxf(ms - M, -200.f));
        const f32x4 os = *(const f32x4*)(p.ws_o + ((int64_t)sidx * ns + s) * BM * HD + (int64_t)lrow * HD + 4 * d4);
        acc += os * wgt;
        l += ls * wgt;
    }
    if (p.lse && d4 == 0) p.lse[((int64_t)b * p.H + h) * p.Sq + row] = (M + __builtin_amdgcn_logf(l)) * LN2;
    const float inv = 1.0f / l;
    f32x4 ov;
    for (int r = 0; r < 4; r++) ov[r] = div_corrected(acc[r], l, inv);
    uint16_t* dst = p.o + (int64_t)b * p.q_batch + (int64_t)h * p.q_head + (int64_t)row * p.q_row + 4 * d4;
    uint2 packed;
    const Bf16Round rm = bf16_round(p.round_mode);
    packed.x = bf16_pack2(ov[0], ov[1], rm);
    packed.y = bf16_pack2(ov[2], ov[3], rm);
    *(uint2*)dst = packed;
}

// ------------------------------------------------------------------ launch
int launch(const AttnParams& p, hipStream_t stream) {
    // The head dimension, c > 0 (the usual positive scale), the causal mask,
    // per-entry key counts, the weights' rounding mode and the work-group size are compile-time
    // variants, so the plain path carries no code for any alternative.  The
    // 4-wave work-group exists for head dimension 128 without the causal mask.
    const bool short_wg = p.nw == KERNEL_NW_SHORT;
    if (p.nw != KERNEL_NW && !(short_wg && p.head_dim == 128 && !p.causal)) return -1;
    dim3 grid(p.grid), block(p.nw * 64);
    auto go_kv = [&](auto hd, auto cpos, auto causal, auto kvl, auto nw) {
        constexpr int H_ = decltype(hd)::value, N_ = decltype(nw)::value;
        constexpr bool CP = decltype(cpos)::value, CA = decltype(causal)::value, KV = decltype(kvl)::value;
        if (p.p_mode == ROUND_RTNA)
            hipLaunchKernelGGL((attn_fwd_main<H_, CP, CA, KV, ROUND_RTNA, N_>), grid, block, 0, stream, p);
        else if (p.p_mode == ROUND_RTZ)
            hipLaunchKernelGGL((attn_fwd_main<H_, CP, CA, KV, ROUND_RTZ, N_>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_main<H_, CP, CA, KV, ROUND_RTNE, N_>), grid, block, 0, stream, p);
    };
    // per-entry key counts are a variant of their own: the kernels without
    // them carry none of their code
    auto go_nw = [&](auto hd, auto cpos, auto causal, auto nw) {
        if (p.kv_lens || p.cu_k) go_kv(hd, cpos, causal, std::true_type{}, nw);
        else go_kv(hd, cpos, causal, std::false_type{}, nw);
    };
    auto go = [&](auto hd, auto cpos, auto causal) {
        constexpr int H_ = decltype(hd)::value;
        constexpr bool CA = decltype(causal)::value;
        if constexpr (H_ == 128 && !CA) {
            if (short_wg) {
                go_nw(hd, cpos, causal, std::integral_constant<int, KERNEL_NW_SHORT>{});
                return;
            }
        }
        go_nw(hd, cpos, causal, std::integral_constant<int, KERNEL_NW>{});
    };
    auto go_hd = [&](auto hd) {
        if (p.causal) {
            if (p.c > 0.f) go(hd, std::true_type{}, std::true_type{});
            else go(hd, std::false_type{}, std::true_type{});
        } else {
            if (p.c > 0.f) go(hd, std::true_type{}, std::false_type{});
            else go(hd, std::false_type{}, std::false_type{});
        }
    };
    if (p.head_dim == 64) go_hd(std::integral_constant<int, 64>{});
    else go_hd(std::integral_constant<int, 128>{});
    if (hipGetLastError() != hipSuccess) return -1;
    if (p.n_full < p.n_items) {
        const int bm = p.nw * 16 * KERNEL_NQB;
        const int64_t total = (int64_t)(p.n_items - p.n_full) * bm * (p.head_dim / 4);
        dim3 cgrid((unsigned)((total + 255) / 256));
        if (p.head_dim == 64)
            hipLaunchKernelGGL((attn_fwd_combine<KERNEL_BM, 64>), cgrid, dim3(256), 0, stream, p);
        else if (short_wg)
            hipLaunchKernelGGL((attn_fwd_combine<KERNEL_NW_SHORT * 16 * KERNEL_NQB, 128>), cgrid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_combine<KERNEL_BM, 128>), cgrid, dim3(256), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

// ------------------------------------------------- fixed scratch array
// Split partials of the allocation-free entry point.  Each GPU holds its own
// copy at its own address, until the process ends.  In host code the name
// `scratch` is a host-side stand-in, not a device address: host code only ever
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __attribute__((aligned(256))) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

int scratch_address(int dev, void** out) {
    static std::mutex mu;
    static void* addr[NOALLOC_MAX_DEVICES] = {};
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return -1;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        // once per device, with that device current (the caller's)
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return -1;
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return 0;
}

}  // namespace attn
