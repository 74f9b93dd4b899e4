// attn_bwd_kernel.hip -- gfx950 (MI355X, CDNA4) kernels for the backward pass
// of bf16 attention, head dimension 128 or 64, for O = softmax(Q K^T * scale) V.
//
// The HipKittens summary's kernel suite pairs the attention forward kernels
// with their backward; the gradients follow from the chain rule on the
// forward's definition, restated here with the forward's saved output O and
// its per-row log-sum-exp L (natural log):
//     P = exp(S * scale - L),  dV = P^T dO,  dP = dO V^T,
//     dS = P o (dP - delta),   delta_i = <dO_i, O_i>,
//     dQ = scale dS K,         dK = scale dS^T Q.
// Three kernels:
//  * attn_bwd_delta: delta_i, HD / 8 lanes per query row (fp32 from bf16),
//    stored negated so that the dP products start from it, and the
//    log-sum-exp in base 2.
//  * attn_bwd_dq: one work-group of 8 waves owns 256 query rows (32 per wave,
//    Q and dO fragments in registers as MFMA operand B) and streams 64-key
//    K and V tiles through LDS.  Per tile: S^T = K Q^T and dP^T = V dO^T (K and
//    V read as operand A, the forward's K-as-A layout, so each lane holds one
//    query), then dS^T elementwise, then dQ^T += K^T dS^T with K^T read by
//    ds_read_b64_tr_b16 in the order of dS^T's keys (the forward's V^T read).
//  * attn_bwd_dkdv: the mirror image -- a work-group owns 128 keys (4 waves x
//    32, K and V fragments in registers as operand B) and streams 64-query Q
//    and dO tiles.  Per tile: S = Q K^T and dP = dO V^T (Q and dO as
//    operand A: each lane holds one key), then P and dS, then dV^T += dO^T P
//    and dK^T += Q^T dS with dO^T and Q^T transposed out of LDS.
// With grouped-query heads (query head h reads key/value head h / group) the
// dQ kernel reads its head's key/value head, and a dK/dV work-group streams
// the query tiles of every query head of its group in turn, so dK and dV add
// up over the group in registers.
// Under the causal mask (query i sees keys j <= i + Skv - Sq, the forward's
// bottom-right alignment) the dQ key loop ends at the tile's diagonal and the
// dK/dV query loop starts at it; the weights of masked pairs are zero by
// select, and work-groups that see no pair write zeros and exit.
// Every LDS tile is read both straight (ds_read_b128) and transposed, so all
// tiles keep one layout: 16-byte chunk c of row r at c ^ swz(r), with
// swz(r) = 2 (r & 7) for 256-byte rows (head dimension 128) and
// 2 ((r >> 1) & 3) for 128-byte rows (64), the forward's V layouts.  It
// keeps chunk pairs together with 8 distinct pair positions over any 8 rows
// (transposed reads: 8 rows x one 32-byte pair per half-wave), and the
// straight reads of 16 rows at one chunk column showed no bank conflicts
// either (SQ_LDS_BANK_CONFLICT; a swizzle that also flipped the low chunk
// bit on rows 8..15 conflicted on them).  P and dS enter the
// MFMAs as bf16 (round to nearest-even); all sums are fp32; the gradients are
// rounded to bf16 (nearest-even).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_bwd_internal.h"

namespace attn_bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS uint8_t lds_u8;   // a byte of LDS (pointers to it are 32-bit LDS addresses)

constexpr int TILE_ROWS = 64;
constexpr int NW = 8;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest-even; NaN -> 0x7FC0
__device__ __forceinline__ uint32_t rtne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// LDS barrier: this wave's LDS reads are done (lgkmcnt) and every wave has
// arrived; each wave waits for its own DMA (vmcnt) before it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The 64-row tile at row r0 of a tensor (row stride row_elems) into LDS with
// buffer_load ... lds: one instruction moves RPW rows (RPW = 64 / CPR, CPR
// the 16-byte chunks of a row: 4 rows at head dimension 128, 8 at 64), and NWK
// waves move the tile in 64 / (RPW * NWK) rounds; lane l of wave w in round i
// writes row RPW*(NWK*i + w) + l / CPR, chunk position l % CPR, holding the
// source chunk (l % CPR) ^ swz(row) (RPW*NWK is a multiple of 16, so one
// swizzle serves every round).  Rows past `rows` read as zero (the
// buffer's range check).  The loads are issued from inline assembly: the
// compiler then adds no vmcnt waits of its own in front of the LDS reads of
// the other buffer (it cannot tell the two buffers apart); every wave waits
// for its own transfers in lds_barrier.
// chunk swizzle of row r (only r mod 16 matters)
template <int HD> __device__ __forceinline__ int swz(int r) {
    return HD == 128 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1);
}
struct TileSrc {
    i32x4 rs;
    int row_bytes;
};
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
template <int HD> __device__ __forceinline__ TileSrc tile_src(const uint16_t* base, int64_t row_elems, int rows) {
    TileSrc t;
    t.row_bytes = (int)(row_elems * 2);
    t.rs = buffer_rsrc(base, (uint32_t)((int64_t)(rows - 1) * t.row_bytes + 2 * HD));
    return t;
}
// 16 bytes per lane from rs at voff + soff to LDS dst + 16 * lane
// (the LDS address, the descriptor and the offset are wave-uniform: say so,
// so they stay in scalar registers)
__device__ __forceinline__ i32x4 uniform4(const i32x4 rs) {
    return i32x4{__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                 __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
}
__device__ __forceinline__ void dma16(const i32x4 rs, lds_u8* dst, int voff, int soff) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    const i32x4 rsu = uniform4(rs);
    const int so = __builtin_amdgcn_readfirstlane(soff);
    // m0 is written in the same statement as the load (as in the forward
    // kernel): nothing can be scheduled between them, and no other code of
    // these kernels uses m0.  The s_nop is the one wait state an LDS-bound
    // buffer load needs after a scalar write of m0 (the hazard recognizer
    // does not see into inline assembly).
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsu), "s"(so) : "memory", "m0");
}
// 4 bytes per lane from rs at voff + soff to LDS dst + 4 * lane
__device__ __forceinline__ void dma4(const i32x4 rs, lds_u8* dst, int voff, int soff) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    const i32x4 rsu = uniform4(rs);
    const int so = __builtin_amdgcn_readfirstlane(soff);
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsu), "s"(so) : "memory", "m0");
}
template <int HD, int NWK>
__device__ __forceinline__ void issue_tile_n(const TileSrc& s, int r0, lds_u8* dst, int wave, int g, int j) {
    static_assert(NWK == 4 || NWK == 8, "4 or 8 waves");
    constexpr int CPR = HD / 8, RPW = 64 / CPR;      // 16-byte chunks per row, rows per wave and round
    const int lane = 16 * g + j;
    const int row = wave * RPW + lane / CPR;
    const int voff = row * s.row_bytes + (((lane % CPR) ^ swz<HD>(row)) << 4);
#pragma unroll
    for (int i = 0; i < TILE_ROWS / (RPW * NWK); i++)
        dma16(s.rs, dst + ((i * NWK + wave) * 64) * 16, voff, (r0 + RPW * NWK * i) * s.row_bytes);
}

// Straight fragment (operand A): lane (g, j) gets row 16*rb + j, dims
// 32*ks + 8*g .. +7.
template <int HD> __device__ __forceinline__ bf16x8 read_rows(const lds_u8* tile, int addr0, int rb) {
    return *(const LDS_AS bf16x8*)(tile + addr0 + rb * 16 * (2 * HD));
}
// Transposed fragment (operand A of a product over the tile's rows): lane
// (g, j) gets, as elements 4*hf + e, rows 32*ks + 16*hf + 4*g + e of dim
// 16*db + j (the order of the B operand built from a C fragment).
template <int HD> __device__ __forceinline__ bf16x8 read_cols(const lds_u8* tile, int addr0, int ks) {
    bf16x4 half[2];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
        const LDS_AS s16x4* src = (const LDS_AS s16x4*)(tile + addr0 + (32 * ks + 16 * hf) * (2 * HD));
        half[hf] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)src));
    }
    return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// Packs a C fragment pair (row blocks 2*ks, 2*ks+1 of 16 rows, 4 per lane)
// into the bf16 B operand whose k index runs over those 32 rows (hardware
// conversion, round to nearest-even).
__device__ __forceinline__ bf16x8 pack_b(const float* lo4, const float* hi4) {
    const bf16x2 a = __builtin_convertvector((f32x2{lo4[0], lo4[1]}), bf16x2);
    const bf16x2 b = __builtin_convertvector((f32x2{lo4[2], lo4[3]}), bf16x2);
    const bf16x2 c = __builtin_convertvector((f32x2{hi4[0], hi4[1]}), bf16x2);
    const bf16x2 d = __builtin_convertvector((f32x2{hi4[2], hi4[3]}), bf16x2);
    const bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------ block order
// The hardware deals work-groups to the 8 XCDs round-robin (XCD = block id
// mod 8), each XCD with its own L2.  A head's work-groups all stream the
// same tiles (dQ: the head's K and V; dK/dV: its Q, dO, L and delta), so
// without the mask block b runs work item order(b), XCD x holding the x-th
// eighth of the items (head-major: a run of whole heads).  Under the mask
// the items run longest first, rank-major (item = rank * BH + head), and
// block b runs item b: when BH is a multiple of 8 each XCD already holds the
// heads congruent to it mod 8 at every rank.
__device__ __forceinline__ int bwd_item(int bid, int n, bool causal) {
    if (causal) return bid;
    const int x = bid & 7, s = bid >> 3;
    const int per = n >> 3, rem = n & 7;
    return x * per + (x < rem ? x : rem) + s;
}

// ---------------------------------------------------------------- delta
// A row's 16-byte chunks go to consecutive lanes (HD / 8 lanes per row, so
// each load of a wave reads whole rows, each one contiguous span), each lane
// accumulates its 8 products and the row's lanes add theirs up by lane
// exchange.  Each thread takes DELTA_PASSES rows, all loads issued before the
// arithmetic, so enough bytes are in flight to stream O and dO at the memory
// rate (one thread per row, each walking its own row, reached half of it).
constexpr int DELTA_PASSES = 4;
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_delta(const BwdParams p) {
    constexpr int LPR = HD / 8;        // lanes per row
    constexpr int RPP = 256 / LPR;     // rows per work-group and pass
    const int64_t n = (int64_t)p.B * p.H * p.Sq;
    const int c = threadIdx.x % LPR;
    int64_t row[DELTA_PASSES];
    uint4 a[DELTA_PASSES], g[DELTA_PASSES];
#pragma unroll
    for (int k = 0; k < DELTA_PASSES; k++) {
        const int64_t r = ((int64_t)blockIdx.x * DELTA_PASSES + k) * RPP + threadIdx.x / LPR;   // (b*H + h)*Sq + i
        row[k] = r;
        a[k] = g[k] = uint4{0u, 0u, 0u, 0u};
        if (r < n) {
            const int i = (int)(r % p.Sq);
            const int64_t bh = r / p.Sq;
            const int h = (int)(bh % p.H), b = (int)(bh / p.H);
            const int64_t off = (int64_t)b * p.q_batch + (int64_t)h * p.q_head + (int64_t)i * p.q_row;
            a[k] = ((const uint4*)(p.o + off))[c];
            g[k] = ((const uint4*)(p.dO + off))[c];
        }
    }
#pragma unroll
    for (int k = 0; k < DELTA_PASSES; k++) {
        const uint32_t av[4] = {a[k].x, a[k].y, a[k].z, a[k].w}, gv[4] = {g[k].x, g[k].y, g[k].z, g[k].w};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc = __builtin_fmaf(__uint_as_float(av[e] << 16), __uint_as_float(gv[e] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(av[e] & 0xffff0000u), __uint_as_float(gv[e] & 0xffff0000u), acc);
        }
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, LPR);
        // stored negated: the dP products start from it, so dP - delta comes
        // out of the matrix core; and the log-sum-exp in base 2, as the
        // exponents use it
        if (c == 0 && row[k] < n) {
            p.delta[row[k]] = -acc;
            p.lse2[row[k]] = p.lse[row[k]] * LOG2E;
        }
    }
}

// ------------------------------------------------------------------- dQ
// 8 waves, each owning 32 query rows (Q and dO fragments in registers as
// operand B).  The same software pipeline and out-of-phase wave groups as the
// dK/dV kernel below: iteration t runs dQ^T += K_{t-1}^T dS^T_{t-1} (K_{t-1}
// read transposed) and S^T_t = K_t Q^T, dP^T_t = V_t dO^T (tiles t read
// straight), then the elementwise step of tile t.  Four K/V slots: waves 0-3
// issue the transfers of tile t+2 after their elementwise step of tile t,
// where the SIMD's scalar and memory issue is idle (at the head of the
// products they delayed the matrix work: 1.6-2.6% of the whole backward),
// and their barrier leaves those transfers in flight.
constexpr int NSLOT = 4;

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(HD == 128 || HD == 64, "head dimension 128 or 64");
    constexpr int ROW_BYTES = 2 * HD, TILE_BYTES = TILE_ROWS * ROW_BYTES;
    constexpr int NKK = HD / 32, NDB = HD / 16;   // k-steps over the dims, 16-dim blocks
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[NSLOT * 2 * TILE_BYTES];   // per slot: K, V
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool late = wave >= 4;
    const int g = lane >> 4, j = lane & 15;
    constexpr int BMQ = NW * 32;
    // under the mask a query tile's key range grows with its index: blocks
    // take the longest first (the last query tile of every head, then the
    // second last, ...) so the short ones fill the end of the launch
    const int BH = p.B * p.H;
    const int it = bwd_item((int)blockIdx.x, (int)gridDim.x, CAUSAL);
    const int qt = CAUSAL ? p.n_qblocks - 1 - it / BH : it % p.n_qblocks;
    const int bh = CAUSAL ? it % BH : it / p.n_qblocks;
    const int h = bh % p.H, b = bh / p.H;
    const int qrow0 = qt * BMQ + wave * 32;
    // keys up to the diagonal of the work-group's last row under the mask
    const int kv_end = CAUSAL ? min(p.Skv, min(p.Sq, (qt + 1) * BMQ) - 1 + p.causal_off + 1) : p.Skv;
    const int T = (kv_end + TILE_ROWS - 1) / TILE_ROWS;
    if (kv_end <= 0) {
        // no row of this work-group sees a key (Sq > Skv): dQ is zero
        // (uniform across the work-group, before any transfer or barrier)
        uint16_t* dqz = p.dq + (int64_t)b * p.q_batch + (int64_t)h * p.q_head;
#pragma unroll
        for (int qb = 0; qb < 2; qb++) {
            const int row = qrow0 + qb * 16 + j;
            if (row >= p.Sq) continue;
#pragma unroll
            for (int db = 0; db < NDB; db++) *(uint2*)(dqz + (int64_t)row * p.q_row + 4 * g + 16 * db) = uint2{0u, 0u};
        }
        return;
    }

    const int hk = h / p.group;                          // key/value head of query head h
    const TileSrc ks = tile_src<HD>(p.k + (int64_t)b * p.kv_batch + (int64_t)hk * p.kv_head, p.kv_row, p.Skv);
    const TileSrc vs = tile_src<HD>(p.v + (int64_t)b * p.kv_batch + (int64_t)hk * p.kv_head, p.kv_row, p.Skv);
    auto kslot = [&](int sl) { return (lds_u8*)tiles + sl * (2 * TILE_BYTES); };
    auto vslot = [&](int sl) { return (lds_u8*)tiles + sl * (2 * TILE_BYTES) + TILE_BYTES; };
    // tile 0: all 8 waves; later tiles: waves 0-3
    issue_tile_n<HD, NW>(ks, 0, kslot(0), wave, g, j);
    issue_tile_n<HD, NW>(vs, 0, vslot(0), wave, g, j);
    // tile t (past the last tile: the last tile again) into slot t % NSLOT,
    // from waves 0-3
    auto issue_tile = [&](int t) __attribute__((always_inline)) {
        const int tt = min(t, T - 1);
        const int sl = t % NSLOT;
        issue_tile_n<HD, 4>(ks, tt * TILE_ROWS, kslot(sl), wave, g, j);
        issue_tile_n<HD, 4>(vs, tt * TILE_ROWS, vslot(sl), wave, g, j);
    };
    constexpr int NDMA_Q = 2 * (TILE_ROWS / ((64 / (HD / 8)) * 4));   // transfers of one issue_tile per wave

    // Q and dO of query rows qrow0 + 16*qb + j (clamped; results of rows past
    // Sq are never stored), dims 32*kk + 8*g .. +7: operand B.
    const int64_t qoff = (int64_t)b * p.q_batch + (int64_t)h * p.q_head;
    bf16x8 qf[2][NKK], gf[2][NKK];
    float lse2[2], dlt[2];
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
        const int row = min(qrow0 + qb * 16 + j, p.Sq - 1);
        const uint16_t* qs = p.q + qoff + (int64_t)row * p.q_row + 8 * g;
        const uint16_t* gs = p.dO + qoff + (int64_t)row * p.q_row + 8 * g;
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) {
            qf[qb][kk] = *(const bf16x8*)(qs + 32 * kk);
            gf[qb][kk] = *(const bf16x8*)(gs + 32 * kk);
        }
        const int64_t ri = ((int64_t)b * p.H + h) * p.Sq + row;
        lse2[qb] = p.lse2[ri];
        dlt[qb] = p.delta[ri];   // -delta
    }
    // Wait for these loads here, once: the register uses below make the
    // compiler place the waits before the loop instead of inside it, where
    // they would also wait for the tile transfers in flight.
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) __asm__ volatile("" : "+v"(qf[qb][kk]), "+v"(gf[qb][kk]));
        __asm__ volatile("" : "+v"(lse2[qb]), "+v"(dlt[qb]));
    }
    f32x4 dq[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; db++)
#pragma unroll
        for (int qb = 0; qb < 2; qb++) dq[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // per-lane fragment offsets: straight reads of row j, transposed reads of
    // rows 4*g + j/4 (+ multiples of 16: same swizzle)
    int a_row[NKK], a_col[NDB];
#pragma unroll
    for (int kk = 0; kk < NKK; kk++) a_row[kk] = j * ROW_BYTES + (((4 * kk + g) ^ swz<HD>(j)) << 4);
#pragma unroll
    for (int db = 0; db < NDB; db++) {
        const int row = 4 * g + (j >> 2);
        a_col[db] = row * ROW_BYTES + (((2 * db + ((j & 3) >> 1)) ^ swz<HD>(row)) << 4) + ((j & 1) << 3);
    }
    if (!late) issue_tile(1);   // waves 0-3: tile 1 (the first barrier waits for it)
    lds_barrier();

    f32x4 s[4][2], dp[4][2];   // S^T, dP^T of tile t: lane (g, j) holds keys 16*kb + 4*g + r of query j
    bf16x8 dsf[2][2];          // dS^T of the previous tile as operand B (k = keys)
    // S^T = K Q^T and dP^T = V dO^T of the tiles in slot sl
    auto products_a = [&](int sl) __attribute__((always_inline)) {
        const lds_u8* kt = kslot(sl);
        const lds_u8* vt = vslot(sl);
#pragma unroll
        for (int kk = 0; kk < NKK; kk++)
#pragma unroll
            for (int kb = 0; kb < 4; kb++) {
                const bf16x8 kf = read_rows<HD>(kt, a_row[kk], kb);
                const bf16x8 vf = read_rows<HD>(vt, a_row[kk], kb);
#pragma unroll
                for (int qb = 0; qb < 2; qb++) {
                    s[kb][qb] = mfma(kf, qf[qb][kk], kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kb][qb]);
                    // from -delta: the product is dP - delta
                    dp[kb][qb] = mfma(vf, gf[qb][kk], kk == 0 ? f32x4{dlt[qb], dlt[qb], dlt[qb], dlt[qb]} : dp[kb][qb]);
                }
            }
    };
    // dQ^T += K^T dS^T with the K tile in slot sl
    auto products_b = [&](int sl) __attribute__((always_inline)) {
        const lds_u8* kt = kslot(sl);
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
#pragma unroll
            for (int db = 0; db < NDB; db++) {
                const bf16x8 kt_f = read_cols<HD>(kt, a_col[db], kk);
#pragma unroll
                for (int qb = 0; qb < 2; qb++) dq[db][qb] = mfma(kt_f, dsf[qb][kk], dq[db][qb]);
            }
    };
    // dS^T = P^T o (dP^T - delta), P^T = 2^(c s - L log2 e) of tile t; keys past
    // Skv (and, under the mask, past the row's diagonal) -> 0 by select
    auto elementwise = [&](int t) __attribute__((always_inline)) {
        auto ew = [&](auto maskc) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(maskc)::value;
            const int valid = p.Skv - t * TILE_ROWS - 4 * g;
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
                const int lim = CAUSAL ? min(valid, qrow0 + qb * 16 + j + p.causal_off + 1 - t * TILE_ROWS - 4 * g)
                                       : valid;
                float dsv[4][4];
#pragma unroll
                for (int kb = 0; kb < 4; kb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const float pw = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], p.c, -lse2[qb]));
                        dsv[kb][r] = (!MASKED || 16 * kb + r < lim) ? pw * dp[kb][qb][r] : 0.f;
                    }
#pragma unroll
                for (int kk = 0; kk < 2; kk++) dsf[qb][kk] = pack_b(dsv[2 * kk], dsv[2 * kk + 1]);
            }
        };
        // Keys past Skv, and under the mask keys past a row's diagonal, occur
        // only in the ragged last tile and the tiles crossing this wave's
        // diagonal (its first row's is the lowest): one uniform branch keeps
        // the selects out of every other tile.
        const bool edge = (t + 1) * TILE_ROWS > p.Skv ||
                          (CAUSAL && (t + 1) * TILE_ROWS - 1 > qrow0 + p.causal_off);
        if (edge) ew(std::true_type{});
        else ew(std::false_type{});
    };
    // barrier of waves 0-3: after their elementwise step (the operands keep the
    // compiler from sinking that step below the barrier) and the transfers
    // of the tile two ahead, which stay in flight (in-order completion: the
    // tile one ahead, issued an iteration earlier, has landed)
    auto early_barrier = [&]() __attribute__((always_inline)) {
        __asm__ volatile("" :: "v"(dsf[0][0]), "v"(dsf[0][1]), "v"(dsf[1][0]), "v"(dsf[1][1]));
        __builtin_amdgcn_sched_barrier(0);
        __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(NDMA_Q) : "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto pin_addr = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NKK; i++) __asm__ volatile("" : "+v"(a_row[i]));
#pragma unroll
        for (int i = 0; i < NDB; i++) __asm__ volatile("" : "+v"(a_col[i]));
    };

    // iteration 0: products of tile 0 only
    pin_addr();
    __builtin_amdgcn_s_setprio(1);
    products_a(0);
    __builtin_amdgcn_s_setprio(0);
    if (late) lds_barrier();
    elementwise(0);
    if (!late) { issue_tile(2); early_barrier(); }
    int cur = 1 % NSLOT, prev = 0;
    for (int t = 1; t < T; t++) {
        pin_addr();
        __builtin_amdgcn_s_setprio(1);
        products_b(prev);   // first: dS^T of tile t-1 is then dead while S^T, dP^T accumulate
        products_a(cur);
        __builtin_amdgcn_s_setprio(0);
        if (late) lds_barrier();
        elementwise(t);
        if (!late) { issue_tile(t + 2); early_barrier(); }
        prev = cur;
        cur = cur == NSLOT - 1 ? 0 : cur + 1;
    }
    // the transfers still in flight (the last iteration's repeat of the last
    // tile) land before the waves end
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the last tile's dQ products (no LDS writes follow: no barrier)
    pin_addr();
    products_b(prev);

    // dQ = scale (dQ^T)^T: lane (g, j) holds dims 16*db + 4*g + r of query j
    uint16_t* dqb = p.dq + qoff;
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
        const int row = qrow0 + qb * 16 + j;
        if (row >= p.Sq) continue;
        uint16_t* dst = dqb + (int64_t)row * p.q_row + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; db++) {
            uint2 pk;
            pk.x = rtne_bits(dq[db][qb][0] * p.scale) | (rtne_bits(dq[db][qb][1] * p.scale) << 16);
            pk.y = rtne_bits(dq[db][qb][2] * p.scale) | (rtne_bits(dq[db][qb][3] * p.scale) << 16);
            *(uint2*)(dst + 16 * db) = pk;
        }
    }
#endif
}

// ----------------------------------------------------------------- dK, dV
// 4 waves, one per SIMD, each owning 32 keys in two 16-key blocks kb (K and
// V fragments in registers as operand B): every Q or dO fragment read from
// LDS feeds two MFMAs.  With 16 keys per wave a 16-cycle MFMA needs a fresh
// 1 KiB fragment, the whole LDS read rate of a CU when all four SIMDs do
// it; 32 keys halve that.  One wave per SIMD has the 512-register budget
// that the 32 keys' dK and dV accumulators (128 registers, kept in AGPRs)
// need beside the rest.  With no second wave on the SIMD, the overlap of
// the elementwise step with the products is built inside the wave: a step
// (one 64-query tile) runs as a fixed sequence of chunks, each a few MFMAs
// with the LDS reads of a later chunk and a share of the VALU work placed
// between them:
//     A0 | A1 + E0 + DMA | A2 + E1 + DMA | A3 + E2 | B0 + E3 |
//     barrier | B1 + the next tile's A0 reads
// (A mb: S and dP of query block mb; E mb: P and dS of block mb, packed to
// bf16 as they are made; B ks: dV and dK over queries 32 ks .. 32 ks + 31;
// DMA: the transfers of step t+2).  Four LDS slots: the Q, dO, L and delta
// tiles of step t+2 go into the slot of step t-2, whose last reads ended
// before the barrier of step t-1; the barrier of step t follows each wave's
// wait for its own transfers of step t+1 (in-order completion: only those
// of step t+2 may remain).  On gfx950 a lone wave's MFMAs overlap little of
// its own other instructions (per-phase timestamps: a phase takes about the
// MFMA time plus the issue time of the rest), so this layout is bound by
// its instruction count more than by LDS; it runs 5-10% faster than eight
// waves of 16 keys.
constexpr int DKV_NW = 4;
constexpr int DKV_NSLOT = 4;                   // a power of two
constexpr int LS_BYTES = 2 * TILE_ROWS * 4;   // L (base 2) and -delta of a tile's 64 queries

// dK and dV accumulate in the accumulation registers (AGPRs): the product
// is written as inline assembly with its C/D operand bound to an AGPR, while
// every other product (built-in, VGPR form) leaves S and dP in VGPRs for the
// elementwise step.  The compiler's hazard checks do not see into inline
// assembly, so the schedule itself keeps the distances these products need:
// their P and dS operands are made a whole phase (or a barrier) before
// their use, the fragments come from LDS reads (waited for by lgkmcnt), no
// accumulator is used by two products less than 16 products apart, and the
// AGPRs are read only after the settling wait at the end; a CPU test checks
// the distances on the built code.
__device__ __forceinline__ void mfma_acc(f32x4& acc, bf16x8 a, bf16x8 b) {
    __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// LDS barrier that leaves this wave's last N transfers in flight
template <int N> __device__ __forceinline__ void lds_barrier_vm() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Chunk boundary: the chunk's reads first, then its NM MFMAs each followed
// by up to NV VALU instructions; nothing moves across the boundary.
template <int NM, int NV> __device__ __forceinline__ void chunk_end(int nr) {
    // LDS reads (nr is a constant once the chunk loops are unrolled)
    switch (nr) {
        case 2: __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); break;
        case 4: __builtin_amdgcn_sched_group_barrier(0x100, 4, 0); break;
        case 6: __builtin_amdgcn_sched_group_barrier(0x100, 6, 0); break;
        default: break;
    }
#pragma unroll
    for (int i = 0; i < NM; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(DKV_NW * 64, 1) void attn_bwd_dkdv(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(HD == 128 || HD == 64, "head dimension 128 or 64");
    constexpr int ROW_BYTES = 2 * HD, TILE_BYTES = TILE_ROWS * ROW_BYTES;
    constexpr int NKK = HD / 32, NDB = HD / 16;   // k-steps over the dims, 16-dim blocks
    constexpr int RPW = 64 / (HD / 8);            // rows per DMA instruction
    constexpr int NDMA = 2 * TILE_ROWS / (RPW * DKV_NW);   // Q and dO transfers per wave and step
    constexpr int PD = HD == 128 ? 3 : 2;         // B-fragment prefetch distance, in chunks (at most 15 LDS reads in flight)
    static_assert(NKK <= NDB && PD <= NKK, "prefetch placement");
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[DKV_NSLOT * 2 * TILE_BYTES];   // per slot: Q, dO
    __shared__ __attribute__((aligned(16))) uint8_t lsd[DKV_NSLOT * LS_BYTES];           // per slot: L, -delta
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, j = lane & 15;
    // under the mask a key block's query range shrinks with its index:
    // blocks take the longest (first key blocks of every head) first
    const int BH = p.B * p.Hkv;
    const int it = bwd_item((int)blockIdx.x, (int)gridDim.x, CAUSAL);
    const int kt_ = CAUSAL ? it / BH : it % p.n_kblocks;
    const int bh = CAUSAL ? it % BH : it / p.n_kblocks;   // (b, key/value head)
    const int hk = bh % p.Hkv, b = bh / p.Hkv;
    const int kbase = kt_ * 128 + wave * 32;             // key block kb of this wave: keys kbase + 16 kb + j
    // query tiles [t0, t0 + T): under the mask the first query that sees the
    // work-group's first key is k0 - (Skv - Sq)
    const int q_first = CAUSAL ? max(0, kt_ * 128 - p.causal_off) : 0;
    const int t0 = q_first / TILE_ROWS;
    const int T = (p.Sq + TILE_ROWS - 1) / TILE_ROWS - t0;
    const int64_t koff = (int64_t)b * p.kv_batch + (int64_t)hk * p.kv_head;
    if (T <= 0) {
        // no query sees these keys: dK = dV = 0 (with the bottom-right mask
        // the last query sees every key, so this is a guard only; uniform
        // across the work-group, before any transfer or barrier)
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            const int krow = kbase + 16 * kb + j;
            if (krow >= p.Skv) continue;
            const int64_t ko = koff + (int64_t)krow * p.kv_row + 4 * g;
#pragma unroll
            for (int db = 0; db < NDB; db++) {
                *(uint2*)(p.dk + ko + 16 * db) = uint2{0u, 0u};
                *(uint2*)(p.dv + ko + 16 * db) = uint2{0u, 0u};
            }
        }
        return;
    }
    const int q0 = t0 * TILE_ROWS;                       // first query row of tile 0
    // steps u = 0 .. TT-1 run over the query heads of the group (outer) and
    // their query tiles [t0, t0 + T) (inner): step u is tile u % T of query
    // head hk * group + u / T, whose first row is q0 + (u % T) * 64
    const int TT = T * p.group;

    auto qslot = [&](int sl) { return (lds_u8*)tiles + sl * (2 * TILE_BYTES); };
    auto gslot = [&](int sl) { return (lds_u8*)tiles + sl * (2 * TILE_BYTES) + TILE_BYTES; };
    auto lslot = [&](int sl) { return (lds_u8*)lsd + sl * LS_BYTES; };
    // L (base 2) and -delta of queries 16*mb + 4*g .. +3 of a tile's slot
    auto read_l2 = [&](const lds_u8* lt, int mb) __attribute__((always_inline)) {
        return *(const LDS_AS f32x4*)(lt + (16 * mb + 4 * g) * 4);
    };
    auto read_dl = [&](const lds_u8* lt, int mb) __attribute__((always_inline)) {
        return *(const LDS_AS f32x4*)(lt + TILE_ROWS * 4 + (16 * mb + 4 * g) * 4);
    };
    // the L and delta, Q, and dO tiles of tile r0 of query head hq into slot
    // sl, in three parts; each query head's tensors get their own buffer
    // ranges, so rows past Sq read as zero (the range check), never the next
    // head's rows.  Every wave issues the L and delta transfers (the same
    // bytes to the same LDS words), so all waves issue NDMA + 2 transfers
    // per step, L and delta first.
    // The descriptors of query head hq's L, delta, Q and dO rows.  A step's
    // transfers use the ones of the head two steps ahead, kept across steps
    // and rebuilt only when that head changes (the 64-bit offsets cost about
    // twenty scalar instructions, in a step whose one wave issues every
    // instruction itself).
    struct HeadSrc {
        i32x4 lse, dlt;
        TileSrc q, g;
    };
    auto head_src = [&](int hq) __attribute__((always_inline)) -> HeadSrc {
        const int64_t rbh = ((int64_t)b * p.H + hq) * p.Sq;
        const int64_t qoff = (int64_t)b * p.q_batch + (int64_t)hq * p.q_head;
        return HeadSrc{buffer_rsrc(p.lse2 + rbh, (uint32_t)p.Sq * 4u), buffer_rsrc(p.delta + rbh, (uint32_t)p.Sq * 4u),
                       tile_src<HD>(p.q + qoff, p.q_row, p.Sq), tile_src<HD>(p.dO + qoff, p.q_row, p.Sq)};
    };
    auto issue_ld = [&](int sl, const HeadSrc& h, int r0) __attribute__((always_inline)) {
        dma4(h.lse, lslot(sl), lane * 4, r0 * 4);
        dma4(h.dlt, lslot(sl) + TILE_ROWS * 4, lane * 4, r0 * 4);
    };
    auto issue_q = [&](int sl, const HeadSrc& h, int r0) __attribute__((always_inline)) {
        issue_tile_n<HD, DKV_NW>(h.q, r0, qslot(sl), wave, g, j);
    };
    auto issue_g = [&](int sl, const HeadSrc& h, int r0) __attribute__((always_inline)) {
        issue_tile_n<HD, DKV_NW>(h.g, r0, gslot(sl), wave, g, j);
    };
    // step u runs tile u % T of the group's query head u / T
    auto step_hq = [&](int u) { return hk * p.group + u / T; };
    auto step_r0 = [&](int u) { return q0 + (u % T) * TILE_ROWS; };

    // K and V of keys kbase + 16 kb + j (clamped; rows past Skv are never stored)
    bf16x8 kf[2][NKK], vf[2][NKK];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        const int row = min(kbase + 16 * kb + j, p.Skv - 1);
        const uint16_t* ksrc = p.k + koff + (int64_t)row * p.kv_row + 8 * g;
        const uint16_t* vsrc = p.v + koff + (int64_t)row * p.kv_row + 8 * g;
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) {
            kf[kb][kk] = *(const bf16x8*)(ksrc + 32 * kk);
            vf[kb][kk] = *(const bf16x8*)(vsrc + 32 * kk);
        }
    }
    // steps 0 and 1 (past the last step, the transfers of step t + 2 repeat
    // the last step's tiles into the free slot, so every step issues the
    // same transfers)
    {
        const HeadSrc h0 = head_src(step_hq(0));
        issue_ld(0, h0, step_r0(0));
        issue_q(0, h0, step_r0(0));
        issue_g(0, h0, step_r0(0));
        const int u = min(1, TT - 1);
        const HeadSrc h1 = head_src(step_hq(u));
        issue_ld(1, h1, step_r0(u));
        issue_q(1, h1, step_r0(u));
        issue_g(1, h1, step_r0(u));
    }
    int uh = min(2, TT - 1) / T, utq = min(2, TT - 1) % T;   // query head and tile of step min(t + 2, TT - 1)
    HeadSrc hsrc = head_src(hk * p.group + uh);                // that head's descriptors
    // wait for the K and V loads here, once (not inside the loop, where the
    // wait would also hold for the transfers in flight)
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) __asm__ volatile("" : "+v"(kf[kb][kk]), "+v"(vf[kb][kk]));
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) __asm__ volatile("" : "+a"(kf[kb][kk]), "+a"(vf[kb][kk]));
    f32x4 dk[2][NDB], dv[2][NDB];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int db = 0; db < NDB; db++) { dk[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f}; dv[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f}; }
    int a_row[NKK], a_col[NDB];
#pragma unroll
    for (int kk = 0; kk < NKK; kk++) a_row[kk] = j * ROW_BYTES + (((4 * kk + g) ^ swz<HD>(j)) << 4);
#pragma unroll
    for (int db = 0; db < NDB; db++) {
        const int row = 4 * g + (j >> 2);
        a_col[db] = row * ROW_BYTES + (((2 * db + ((j & 3) >> 1)) ^ swz<HD>(row)) << 4) + ((j & 1) << 3);
    }
    lds_barrier_vm<NDMA + 2>();

    // the straight fragments, L and -delta of query block 0 of the first tile
    bf16x8 fa0[NKK][2];
#pragma unroll
    for (int kk = 0; kk < NKK; kk++) {
        fa0[kk][0] = read_rows<HD>(qslot(0), a_row[kk], 0);
        fa0[kk][1] = read_rows<HD>(gslot(0), a_row[kk], 0);
    }
    f32x4 l20 = read_l2(lslot(0), 0), dl0 = read_dl(lslot(0), 0);

    // one step on the tile in slot sl (first query row r0), issuing the
    // transfers of tile dr0 of the head whose descriptors are dh into slot
    // dsl among its products;
    // MASK: apply the causal mask by select.  Rows past Sq need no select: their Q, dO, L
    // and delta read as zero, so their weight is 2^0 = 1 and their dS is
    // 1 * (0 - 0) = 0, and both meet zero rows of dO and Q in the dV and dK
    // products.
    auto run_step = [&](auto mask_c, int sl, int r0, int nsl, int dsl, const HeadSrc& dh, int dr0) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_c)::value;
        const lds_u8* qt = qslot(sl);
        const lds_u8* gt = gslot(sl);
        const lds_u8* lt = lslot(sl);
        f32x4 s[2][4], dp[2][4];   // S and dP: lane (g, j) holds queries 16*mb + 4*g + r of key 16*kb + j
        bf16x2 pp[2][4][2], dsp[2][4][2];   // P and dS of queries 16*mb + 4*g + 2*h, +1, packed as they are made
        bf16x8 fa[4][NKK][2];         // straight Q, dO fragments of query block mb
        bf16x8 fb[2][NDB][2];         // transposed dO, Q fragments of half ks
        f32x4 l2[4], dl[4];
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) { fa[0][kk][0] = fa0[kk][0]; fa[0][kk][1] = fa0[kk][1]; }
        auto read_a = [&](int mb, int kk) __attribute__((always_inline)) {
            fa[mb][kk][0] = read_rows<HD>(qt, a_row[kk], mb);
            fa[mb][kk][1] = read_rows<HD>(gt, a_row[kk], mb);
        };
        auto read_b = [&](int ks, int db) __attribute__((always_inline)) {
            fb[ks][db][0] = read_cols<HD>(gt, a_col[db], ks);
            fb[ks][db][1] = read_cols<HD>(qt, a_col[db], ks);
        };
        auto read_ld = [&](int mb) __attribute__((always_inline)) {
            l2[mb] = read_l2(lt, mb);
            dl[mb] = read_dl(lt, mb);
        };
        auto mfma_a = [&](int mb, int kk) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                s[kb][mb] = mfma(fa[mb][kk][0], kf[kb][kk], kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kb][mb]);
                // from -delta: the product is dP - delta
                dp[kb][mb] = mfma(fa[mb][kk][1], vf[kb][kk], kk == 0 ? dl[mb] : dp[kb][mb]);
            }
        };
        // P and dS as operand B of half ks: k = queries 32 ks + 16 hf + 4 g + e
        // (elements 4 hf + e), the blocks mb = 2 ks, 2 ks + 1 in order
        auto operand = [&](bf16x2 (&v)[2][4][2], int kb, int ks) __attribute__((always_inline)) {
            const bf16x4 lo = __builtin_shufflevector(v[kb][2 * ks][0], v[kb][2 * ks][1], 0, 1, 2, 3);
            const bf16x4 hi = __builtin_shufflevector(v[kb][2 * ks + 1][0], v[kb][2 * ks + 1][1], 0, 1, 2, 3);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        auto mfma_b = [&](int ks, int db) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                mfma_acc(dv[kb][db], fb[ks][db][0], operand(pp, kb, ks));
                mfma_acc(dk[kb][db], fb[ks][db][1], operand(dsp, kb, ks));
            }
        };
        // P = 2^(c s - L log2 e), dS = P o (dP - delta) of the element pair
        // e (kb = e / 2, rows r = 2 (e % 2), +1) of query block mb, rounded to
        // bf16 (nearest-even) in pairs; under MASK, queries before the key's
        // diagonal -> 0 by select
        auto elem2 = [&](int mb, int e) __attribute__((always_inline)) {
            const int kb = e >> 1, h = e & 1;
            float pw[2], ds[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int r = 2 * h + i;
                const float x = __builtin_fmaf(s[kb][mb][r], p.c, -l2[mb][r]);
                if (MASK) {
                    // query 16*mb + 4*g + r of the tile sees key kbase + 16*kb + j iff
                    // 16*mb + r >= kbase + 16*kb + j - (Skv - Sq) - r0 - 4*g
                    const int lo = kbase + 16 * kb + j - p.causal_off - r0 - 4 * g;
                    const bool in = 16 * mb + r >= lo;
                    pw[i] = in ? __builtin_amdgcn_exp2f(x) : 0.f;
                    // by select, like the weight: 0 * (dP - delta) would be NaN
                    // where a pair outside the mask meets a non-finite dP or delta
                    ds[i] = in ? pw[i] * dp[kb][mb][r] : 0.f;
                } else {
                    pw[i] = __builtin_amdgcn_exp2f(x);
                    ds[i] = pw[i] * dp[kb][mb][r];
                }
            }
            pp[kb][mb][h] = __builtin_convertvector((f32x2{pw[0], pw[1]}), bf16x2);
            dsp[kb][mb][h] = __builtin_convertvector((f32x2{ds[0], ds[1]}), bf16x2);
            // made here, in this chunk: otherwise the compiler may move the
            // conversions next to their use by an inline-assembly product,
            // closer than the 2 wait states a VALU write needs before an
            // MFMA reads the register
            __asm__ volatile("" : "+v"(pp[kb][mb][h]), "+v"(dsp[kb][mb][h]));
        };

        // A0 (its L and -delta came with the previous step: the dP products
        // start from -delta), with the reads of A1 and of block 1's L, -delta
        l2[0] = l20;
        dl[0] = dl0;
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) {
            if (kk == 0) read_ld(1);
            read_a(1, kk);
            mfma_a(0, kk);
            chunk_end<4, 0>(2 + (kk == 0 ? 2 : 0));
        }
        // A mb + E mb-1, with the reads of A mb+1 (or, in A3, of B0's first chunks)
#pragma unroll
        for (int mb = 1; mb < 4; mb++) {
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) {
                if (kk == 0 && mb < 3) read_ld(mb + 1);
                if (kk == 0 && mb == 1) { issue_ld(dsl, dh, dr0); issue_q(dsl, dh, dr0); }
                if (kk == 0 && mb == 2) issue_g(dsl, dh, dr0);
                int nr = (kk == 0 && mb < 3) ? 2 : 0;
                if (mb < 3) { read_a(mb + 1, kk); nr += 2; }
                else if (kk < PD) { read_b(0, kk); nr += 4; }
                mfma_a(mb, kk);
#pragma unroll
                for (int e = 0; e < 4 / NKK; e++) elem2(mb - 1, (4 / NKK) * kk + e);
                chunk_end<4, 6>(nr);
            }
        }
        // B0 + E3, with the reads of B0 (the rest) and B1's first chunks
#pragma unroll
        for (int db = 0; db < NDB; db++) {
            if (db + PD < NDB) read_b(0, db + PD);
            else read_b(1, db + PD - NDB);
            mfma_b(0, db);
            // (in the later chunks: S and dP of block 3 come from the last
            // products of A3, whose results a VALU read has to wait for)
            if (db >= NDB - 4) elem2(3, db - (NDB - 4));
            chunk_end<4, 4>(4);
        }
        // P and dS of blocks 2 and 3 are used only after the barrier: the
        // register uses keep the compiler from sinking their computation
        // below it
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int mb = 2; mb < 4; mb++)
#pragma unroll
                for (int h = 0; h < 2; h++) __asm__ volatile("" : "+v"(pp[kb][mb][h]), "+v"(dsp[kb][mb][h]));
        // every wave has its transfers of the next step in LDS, and has
        // issued its last reads of the slot that step t+1's transfers reuse
        lds_barrier_vm<NDMA + 2>();
        // B1, with the reads of B1 (the rest) and of the next tile's A0 and its
        // L, -delta
        const lds_u8* qn = qslot(nsl);
        const lds_u8* gn = gslot(nsl);
        const lds_u8* ln = lslot(nsl);
        static_assert(NDB - NKK - 1 >= 0 && NDB - NKK - 1 + PD < NDB, "the chunk before the A0 reads holds 6 reads");
#pragma unroll
        for (int db = 0; db < NDB; db++) {
            if (db + PD < NDB) read_b(1, db + PD);
            if (db == NDB - NKK - 1) {
                l20 = read_l2(ln, 0);
                dl0 = read_dl(ln, 0);
            }
            // the NKK fragment pairs of the next A0, in the last NKK chunks
            if (db >= NDB - NKK) {
                const int kk = db - (NDB - NKK);
                fa0[kk][0] = read_rows<HD>(qn, a_row[kk], 0);
                fa0[kk][1] = read_rows<HD>(gn, a_row[kk], 0);
            }
            mfma_b(1, db);
            chunk_end<4, 0>((db + PD < NDB ? 4 : 0) + (db >= NDB - NKK ? 2 : 0) + (db == NDB - NKK - 1 ? 2 : 0));
        }
    };

    int sl = 0, tq = 0;                                  // slot and tile index (within its head) of step t
    for (int t = 0; t < TT; t++) {
        const int r0 = q0 + tq * TILE_ROWS;             // first query row of the step's tile
        const int nsl = sl == DKV_NSLOT - 1 ? 0 : sl + 1;
        run_step(std::integral_constant<bool, CAUSAL>{}, sl, r0, nsl, (t + 2) & (DKV_NSLOT - 1),
                 hsrc, q0 + utq * TILE_ROWS);
        if (t + 3 < TT) {
            utq = utq == T - 1 ? 0 : utq + 1;
            if (utq == 0) {
                uh++;
                hsrc = head_src(hk * p.group + uh);
            }
        }
        sl = nsl;
        tq = tq == T - 1 ? 0 : tq + 1;
    }
    // the repeated transfers of the last two steps land before the wave ends
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // the last MFMA's results settle before the AGPRs are read (a read of an
    // MFMA result needs up to 18 wait states; 24 here)
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int db = 0; db < NDB; db++) __asm__ volatile("" : "+a"(dk[kb][db]), "+a"(dv[kb][db]));
    __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    // dK = scale (dK^T)^T, dV = (dV^T)^T: lane (g, j) holds dims 16*db + 4*g + r of key 16*kb + j
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        const int krow = kbase + 16 * kb + j;
        if (krow >= p.Skv) continue;
        uint16_t* dkd = p.dk + koff + (int64_t)krow * p.kv_row + 4 * g;
        uint16_t* dvd = p.dv + koff + (int64_t)krow * p.kv_row + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; db++) {
            uint2 a, c;
            a.x = rtne_bits(dk[kb][db][0] * p.scale) | (rtne_bits(dk[kb][db][1] * p.scale) << 16);
            a.y = rtne_bits(dk[kb][db][2] * p.scale) | (rtne_bits(dk[kb][db][3] * p.scale) << 16);
            c.x = rtne_bits(dv[kb][db][0]) | (rtne_bits(dv[kb][db][1]) << 16);
            c.y = rtne_bits(dv[kb][db][2]) | (rtne_bits(dv[kb][db][3]) << 16);
            *(uint2*)(dkd + 16 * db) = a;
            *(uint2*)(dvd + 16 * db) = c;
        }
    }
#endif
}

int launch_bwd(const BwdParams& p, hipStream_t stream) {
    // head dimension and causal mask are compile-time variants
    auto go = [&](auto hd) -> int {
        constexpr int H_ = decltype(hd)::value;
        const int64_t rows = (int64_t)p.B * p.H * p.Sq;
        const int64_t per_group = DELTA_PASSES * 256 / (H_ / 8);
        hipLaunchKernelGGL(attn_bwd_delta<H_>, dim3((unsigned)((rows + per_group - 1) / per_group)), dim3(256), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return -1;
        const dim3 gk((unsigned)((int64_t)p.B * p.Hkv * p.n_kblocks)), gq((unsigned)((int64_t)p.B * p.H * p.n_qblocks));
        if (p.causal) hipLaunchKernelGGL((attn_bwd_dkdv<H_, true>), gk, dim3(DKV_NW * 64), 0, stream, p);
        else hipLaunchKernelGGL((attn_bwd_dkdv<H_, false>), gk, dim3(DKV_NW * 64), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return -1;
        if (p.causal) hipLaunchKernelGGL((attn_bwd_dq<H_, true>), gq, dim3(NW * 64), 0, stream, p);
        else hipLaunchKernelGGL((attn_bwd_dq<H_, false>), gq, dim3(NW * 64), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return -1;
        return 0;
    };
    if (p.head_dim == 64) return go(std::integral_constant<int, 64>{});
    if (p.head_dim == 128) return go(std::integral_constant<int, 128>{});
    return -1;
}

}  // namespace attn_bwd
