// attn_fwd_kernel.hip -- gfx950 (MI355X, CDNA4) kernels for bf16 attention forward.
//
// Computes O = softmax(Q K^T * scale) V for head dimension 128 (the fused
// operation of "MoonMath AI open-sources a HIP attention kernel for AMD
// MI300X that beats AITER", opening paragraphs), streaming K/V tiles with an
// online softmax.  Design, per work-group:
//
//  * Work item = (batch, head, tile of BM query rows, key range).  Each of the
//    NW waves owns 16*NQB query rows; its Q fragments stay in VGPRs for the
//    whole key loop and O accumulates in registers (the MI300X article's data
//    placement section keeps Q and the accumulators in registers too).
//  * K and V tiles of 64 keys go HBM -> LDS with buffer_load ... lds (16 B per
//    lane, lane-contiguous in LDS), double-buffered and shared by all waves.
//    The bank swizzle is applied to the source address of each lane, not to
//    the LDS address (HipKittens summary, method section on global async
//    loads).  Rows past Skv read as zero through the buffer range check.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16, K as operand A and Q as
//    operand B.  With that order each lane ends up holding scores of ONE
//    query for a set of keys, which is exactly the B-operand layout of the
//    next product O^T = V^T P^T, so P never leaves registers (the FlyDSL
//    procedure article, optimisation section, states the operand-order trick
//    for gfx942; here it is re-derived for the 16x16x32 shape: K rows are
//    read in a permuted order so that every lane group holds 8 consecutive
//    keys of each 32-key step).  The AITER docs index names the same bf16
//    16x16x32 MFMA for both attention products on gfx950.
//  * V^T fragments come from the row-major V tile through ds_read_b64_tr_b16,
//    the gfx950 transposing LDS read (FlyDSL article: gfx950 adds
//    LDS-to-register transpose loads), so V needs no shuffle.
//  * Online softmax with a power-of-two running maximum: M = ceil(max x) with
//    x = s * scale * log2(e), p = 2^(x - M).  A change of M rescales O and the
//    row sum by an exact power of two, and is skipped when no row's M moved.
//    Row maxima and sums are reduced across the 4 lanes of a row with the
//    gfx950 v_permlane16/32_swap instructions.
//  * P enters the second product as bf16 rounded to nearest-even
//    (v_cvt_pk_bf16_f32); the row sum adds those same bf16 weights, and the
//    output is divided by it and
//    rounded to bf16 in the requested mode with integer bit arithmetic after
//    a NaN guard.
//  * Optional split of the key range (the flash-decoding style tail split of
//    the MI300X article, section on the two later improvements): each split
//    writes its unnormalised fp32 O, M and row sum; a combine kernel merges the
//    splits in a fixed order with exact power-of-two weights.
//  * The block id -> work item map groups consecutive query tiles of a head
//    onto one XCD (blocks are dealt to the 8 XCDs round-robin), so the K/V of
//    a head is fetched into one XCD's L2 (HipKittens summary, chiplet-aware
//    grid schedule).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int D = 128;          // head dimension
constexpr int BN = 64;          // keys per K/V tile
constexpr int NW = KERNEL_NW;   // waves per work-group (two groups of 4)
constexpr int NQB = KERNEL_NQB; // 16-row query blocks per wave
constexpr int BM = KERNEL_BM;   // query rows per work item
constexpr int ROW_BYTES = D * 2;
constexpr int TILE_BYTES = BN * ROW_BYTES;  // 16 KiB

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over lanes {l, l^16, l^32, l^48}
__device__ __forceinline__ float rowmax4(float x) {
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

// sum over lanes {l, l^16, l^32, l^48}, in a fixed pairing order
__device__ __forceinline__ float rowsum4(float x) {
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// fp32 -> bf16 bits in the requested mode; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16_bits(float f, int mode) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    uint32_t add = (mode == ROUND_RTNE) ? (0x7fffu + ((u >> 16) & 1u)) : (mode == ROUND_RTNA ? 0x8000u : 0u);
    return (u + add) >> 16;
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

// LDS bank swizzles (16-byte chunk index XOR a function of the row).
// K is read with ds_read_b128 by 16 lanes at 16 different rows of one chunk;
// the rows a lane group touches are {0-3, 8-11, 16-19, 24-27} (+4): map them
// to 16 distinct chunks.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
// V is read with ds_read_b64_tr_b16: each 16-lane group reads 4 rows x 32 B;
// the 32-byte pair of chunks moves with the row, keeping pairs intact.
__device__ __forceinline__ int swz_v(int row) { return ((row & 3) | (((row >> 3) & 1) << 2)) << 1; }

// Key (tile row) held by A-row m of key block kb, chosen so that lane group g
// of the score fragments holds keys 32*(kb/2) + 8g + 4*(kb%2) + r, r = 0..3.
__device__ __forceinline__ int k_perm_row(int kb, int m) {
    return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

__device__ __forceinline__ int map_block(int bid, int n, int order) {
    if (order != ORDER_XCD) return bid;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// ------------------------------------------------------------ main kernel
// Workgroup barrier that keeps outstanding K/V DMA (tracked by vmcnt) in
// flight across it: a memory fence here would wait for the DMA's LDS writes.
// Every wave instead waits for its own DMA explicitly before the barrier that
// publishes a tile, and ds_read/ds_write completion (lgkmcnt) is waited for
// here; the "memory" clobber keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 8 waves in two groups of 4 (waves w and w+4 share a SIMD).  Each wave owns
// 32 query rows.  Per key tile t a wave runs an MFMA phase (S_t = K_t Q^T and
// O += V_{t-1}^T P_{t-1}^T) and a VALU phase (softmax of S_t into P_t).  Group 1
// starts one barrier late, so at any time one group is on the matrix cores
// and the other on the vector ALUs, swapping at every barrier (the schedule
// of the MI300X article's architecture section and of the HipKittens 8-wave
// ping-pong).  K_{t+1} and V_t are fetched during the interval in which group
// 0 runs MFMA phase t and must land by the end of the following interval.
template <bool CPOS>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_main(const AttnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    constexpr int NTHREADS = NW * 64;
    constexpr int DMA_PER_TILE = TILE_BYTES / 16 / NTHREADS;   // 16-byte chunks per lane per tile
    static_assert(TILE_BYTES % (16 * NTHREADS) == 0, "tile must split evenly over lanes");
    // Four distinct LDS objects (K and V, two buffers each): with the buffer
    // choice a compile-time constant the compiler can tell that a DMA into one
    // buffer does not alias reads of another and does not wait for it.
    __shared__ __attribute__((aligned(1024))) uint8_t sk0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sk1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sv0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sv1[TILE_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
    const int group = wave >> 2;   // 0 or 1
    const int g = lane >> 4;       // lane group (0..3)
    const int j = lane & 15;       // lane within group

    // ---- work item
    const int w = map_block(blockIdx.x, p.n_blocks, p.block_order);
    const int split = w % p.kv_splits;
    const int item = w / p.kv_splits;
    const int qt = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int h = bh % p.H;
    const int b = bh / p.H;

    // split s covers key tiles [s*T/ns, (s+1)*T/ns) of the T tiles: never empty for ns <= T
    const int kv_begin = (int)(((int64_t)split * p.n_kv_tiles) / p.kv_splits) * BN;
    const int kv_end = min(p.Skv, (int)(((int64_t)(split + 1) * p.n_kv_tiles) / p.kv_splits) * BN);
    const int T = (kv_end - kv_begin + BN - 1) / BN;

    const uint16_t* qbase = p.q + (int64_t)b * p.q_batch + (int64_t)h * p.q_head;
    const char* kbase = (const char*)(p.k + (int64_t)b * p.kv_batch + (int64_t)h * p.kv_head);
    const char* vbase = (const char*)(p.v + (int64_t)b * p.kv_batch + (int64_t)h * p.kv_head);
    const int kv_row_bytes = (int)(p.kv_row * 2);

    // ---- K/V buffer resources: reads at or beyond kv_end return zero.
    const uint32_t nrec = (uint32_t)((int64_t)(kv_end - 1) * kv_row_bytes + ROW_BYTES);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nrec, 0x00020000);

    // Per-lane DMA source offsets (relative to the tile's first row).
    int dma_off_k[DMA_PER_TILE], dma_off_v[DMA_PER_TILE];
#pragma unroll
    for (int i = 0; i < DMA_PER_TILE; i++) {
        const int slot = (i * NW + wave) * 64 + lane;   // 16-byte slot in the LDS tile
        const int row = slot >> 4, cp = slot & 15;
        dma_off_k[i] = row * kv_row_bytes + ((cp ^ swz_k(row)) << 4);
        dma_off_v[i] = row * kv_row_bytes + ((cp ^ swz_v(row)) << 4);
    }
    auto issue_k = [&](int t, uint8_t* dst) {
        const int soff = (kv_begin + t * BN) * kv_row_bytes;
#pragma unroll
        for (int i = 0; i < DMA_PER_TILE; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (LDS_AS void*)(dst + ((i * NW + wave) * 64) * 16), 16,
                                                     dma_off_k[i] + soff, 0, 0, 0);
    };
    auto issue_v = [&](int t, uint8_t* dst) {
        const int soff = (kv_begin + t * BN) * kv_row_bytes;
#pragma unroll
        for (int i = 0; i < DMA_PER_TILE; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (LDS_AS void*)(dst + ((i * NW + wave) * 64) * 16), 16,
                                                     dma_off_v[i] + soff, 0, 0, 0);
    };

    issue_k(0, sk0);

    // ---- Q fragments (operand B of S^T = K Q^T): lane holds query row 16*qb + j,
    // dims 32*ks + 8*g .. +7.  Rows past Sq are clamped (never stored).
    const int qrow0 = qt * BM + wave * 16 * NQB;
    bf16x8 qf[NQB][4];
#pragma unroll
    for (int qb = 0; qb < NQB; qb++) {
        const int row = min(qrow0 + qb * 16 + j, p.Sq - 1);
        const uint16_t* src = qbase + (int64_t)row * p.q_row + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ks++) qf[qb][ks] = *(const bf16x8*)(src + 32 * ks);
    }

    f32x4 o_acc[8][NQB];
#pragma unroll
    for (int db = 0; db < 8; db++)
#pragma unroll
        for (int qb = 0; qb < NQB; qb++) o_acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; qb++) { m_run[qb] = -__builtin_inff(); l_run[qb] = 0.f; }
    f32x4 s_acc[4][NQB];
    bf16x8 pf[NQB][2];
    const float c = p.c;
    const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

    // ---- S^T = K Q^T  (4 key blocks x NQB query blocks, 4 k-steps of 32 dims)
    auto qk = [&](const uint8_t* kt) {
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
#pragma unroll
            for (int qb = 0; qb < NQB; qb++) s_acc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int row = k_perm_row(kb, j);
            const int rsw = swz_k(row);
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const bf16x8 kf = *(const LDS_AS bf16x8*)(LDS_AS const uint8_t*)(kt + row * ROW_BYTES + (((4 * ks + g) ^ rsw) << 4));
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) s_acc[kb][qb] = mfma16x16x32(kf, qf[qb][ks], s_acc[kb][qb]);
            }
        }
    };

    // ---- O^T += V^T P^T (8 dim blocks x NQB query blocks, 2 k-steps of 32 keys)
    auto pv = [&](const uint8_t* vt) {
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
#pragma unroll
            for (int db = 0; db < 8; db++) {
                bf16x4 half[2];
#pragma unroll
                for (int hf = 0; hf < 2; hf++) {
                    const int row = 32 * ks + 8 * g + 4 * hf + (j >> 2);
                    const int chunk = (2 * db + ((j & 3) >> 1)) ^ swz_v(row);
                    const LDS_AS s16x4* src = (const LDS_AS s16x4*)(LDS_AS const uint8_t*)(vt + row * ROW_BYTES + (chunk << 4) + ((j & 1) << 3));
                    half[hf] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)src));
                }
                const bf16x8 vf = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) o_acc[db][qb] = mfma16x16x32(vf, pf[qb][ks], o_acc[db][qb]);
            }
        }
    };

    // ---- online softmax of S_t with a power-of-two running max; rescales O and l.
    auto softmax = [&](int t) {
        const int valid = kv_end - (kv_begin + t * BN);   // keys of this tile inside the range
        bool any_rescale = false;
        float alpha[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; qb++) {
            // keys past the range are masked by select, never by arithmetic
            if (valid < BN) {
#pragma unroll
                for (int kb = 0; kb < 4; kb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int key = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
                        s_acc[kb][qb][r] = key >= valid ? (CPOS ? -__builtin_inff() : __builtin_inff()) : s_acc[kb][qb][r];
                    }
            }
            if (!CPOS) {
                // general scale (c <= 0): x = s*c explicitly (masked keys: +inf * c -> -inf unless c == 0)
#pragma unroll
                for (int kb = 0; kb < 4; kb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int key = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
                        s_acc[kb][qb][r] = key >= valid ? -__builtin_inff() : s_acc[kb][qb][r] * c;
                    }
            }
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) mx = fmaxf(mx, s_acc[kb][qb][r]);
            mx = rowmax4(mx);
            if (CPOS) mx *= c;
            const float m_new = fmaxf(m_run[qb], ceilf(mx));
            const float dm = m_run[qb] - m_new;     // <= 0, integer-valued, or -inf / NaN
            alpha[qb] = ldexpf(1.0f, (int)fmaxf(dm, -200.f));
            any_rescale |= (dm != 0.f);
            m_run[qb] = m_new;
            const float negm = -m_new;
            f32x4 pv4[4];
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float x = CPOS ? __builtin_fmaf(s_acc[kb][qb][r], c, negm) : (s_acc[kb][qb][r] + negm);
                    pv4[kb][r] = __builtin_amdgcn_exp2f(x);
                }
            // The row sum adds the bf16-rounded weights, the same values the
            // P V product uses, so O is normalised by exactly its own weights.
            // (pairs are converted one register at a time and summed with
            // v_dot2c_f32_bf16 against (1, 1): one instruction per two weights)
            float psum = l_run[qb] * alpha[qb];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                bf16x2 pr[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4& src = pv4[2 * ks + (i >> 1)];
                    const f32x2 two = {src[2 * (i & 1)], src[2 * (i & 1) + 1]};
                    pr[i] = __builtin_convertvector(two, bf16x2);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(pr[i], ones2, psum, false);
                }
                const bf16x4 lo = __builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3);
                const bf16x4 hi = __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3);
                pf[qb][ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            l_run[qb] = psum;
        }
        if (__builtin_amdgcn_ballot_w64(any_rescale) != 0) {
#pragma unroll
            for (int db = 0; db < 8; db++)
#pragma unroll
                for (int qb = 0; qb < NQB; qb++) o_acc[db][qb] *= alpha[qb];
        }
    };

    // ---- the ping-pong loop (see the comment above the kernel)
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): K_0 slice and Q landed
    lds_barrier();
    if (group == 1) {
        if (T > 1) issue_k(1, sk1);
        issue_v(0, sv0);
        lds_barrier();                    // the one-phase offset of group 1
    }
    // iteration t: K_t in kc, K_{t+1} -> kn, V_t -> vc, V_{t-1} in vp
    auto iter = [&](int t, uint8_t* kc, uint8_t* kn, uint8_t* vc, uint8_t* vp) {
        // MFMA phase t
        if (group == 0) {
            if (t + 1 < T) issue_k(t + 1, kn);
            if (t < T) issue_v(t, vc);
        }
        if (t < T) qk(kc);
        if (t >= 1) pv(vp);
        if (group == 1) __builtin_amdgcn_s_waitcnt(0x0f70);
        lds_barrier();
        // VALU phase t
        if (group == 1) {
            if (t + 2 < T) issue_k(t + 2, kc);
            if (t + 1 < T) issue_v(t + 1, vp);
        }
        if (t < T) softmax(t);
        if (group == 0) __builtin_amdgcn_s_waitcnt(0x0f70);
        lds_barrier();
    };
    for (int t = 0; t <= T; t += 2) {
        iter(t, sk0, sk1, sv0, sv1);
        if (t + 1 <= T) iter(t + 1, sk1, sk0, sv1, sv0);
    }
    if (group == 0) lds_barrier();        // group 0 matches group 1's extra barrier

    // ---- epilogue: the 4 lanes of a row hold partial row sums
    float l_row[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; qb++) l_row[qb] = rowsum4(l_run[qb]);

    if (p.kv_splits == 1) {
        uint16_t* obase = p.o + (int64_t)b * p.q_batch + (int64_t)h * p.q_head;
#pragma unroll
        for (int qb = 0; qb < NQB; qb++) {
            const int row = qrow0 + qb * 16 + j;
            if (row >= p.Sq) continue;
            const float lr = l_row[qb];
            const float inv = 1.0f / lr;
            uint16_t* dst = obase + (int64_t)row * p.q_row + 4 * g;
#pragma unroll
            for (int db = 0; db < 8; db++) {
                f32x4 ov;
#pragma unroll
                for (int r = 0; r < 4; r++) ov[r] = div_corrected(o_acc[db][qb][r], lr, inv);
                const uint32_t b0 = to_bf16_bits(ov[0], p.round_mode), b1 = to_bf16_bits(ov[1], p.round_mode);
                const uint32_t b2 = to_bf16_bits(ov[2], p.round_mode), b3 = to_bf16_bits(ov[3], p.round_mode);
                uint2 packed;
                packed.x = b0 | (b1 << 16);
                packed.y = b2 | (b3 << 16);
                *(uint2*)(dst + 16 * db) = packed;
            }
        }
    } else {
        // partial results: O (unnormalised, fp32) [item][split][BM][128], M and l [item][split][BM]
        const int64_t part = (int64_t)item * p.kv_splits + split;
        float* ow = p.ws_o + part * (int64_t)BM * D;
        float* mw = p.ws_ml + part * (int64_t)BM * 2;
#pragma unroll
        for (int qb = 0; qb < NQB; qb++) {
            const int lrow = wave * 16 * NQB + qb * 16 + j;   // row within the tile
#pragma unroll
            for (int db = 0; db < 8; db++) *(f32x4*)(ow + (int64_t)lrow * D + 16 * db + 4 * g) = o_acc[db][qb];
            if (g == 0) {
                mw[2 * lrow] = m_run[qb];
                mw[2 * lrow + 1] = l_row[qb];
            }
        }
    }
#endif
}

// ---------------------------------------------------------- combine kernel
// One thread per (row, 4 dims): merges the splits of a query tile in split
// order: M = max_s M_s, O = sum_s 2^(M_s - M) O_s / sum_s 2^(M_s - M) l_s.
template <int BM>
__global__ __launch_bounds__(256) void attn_fwd_combine(const AttnParams p) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.n_items * BM * (D / 4);
    if (gid >= total) return;
    const int d4 = (int)(gid % (D / 4));
    const int64_t r = gid / (D / 4);
    const int lrow = (int)(r % BM);
    const int item = (int)(r / BM);
    const int qt = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int h = bh % p.H, b = bh / p.H;
    const int row = qt * BM + lrow;
    if (row >= p.Sq) return;

    const int ns = p.kv_splits;
    const float* mw = p.ws_ml + (int64_t)item * ns * BM * 2;
    float M = -__builtin_inff();
    for (int s = 0; s < ns; s++) M = fmaxf(M, mw[(int64_t)s * BM * 2 + 2 * lrow]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int s = 0; s < ns; s++) {
        const float ms = mw[(int64_t)s * BM * 2 + 2 * lrow];
        const float ls = mw[(int64_t)s * BM * 2 + 2 * lrow + 1];
        const float wgt = ldexpf(1.0f, (int)fmaxf(ms - M, -200.f));
        const f32x4 os = *(const f32x4*)(p.ws_o + ((int64_t)item * ns + s) * BM * D + (int64_t)lrow * D + 4 * d4);
        acc += os * wgt;
        l += ls * wgt;
    }
    const float inv = 1.0f / l;
    f32x4 ov;
    for (int r = 0; r < 4; r++) ov[r] = div_corrected(acc[r], l, inv);
    uint16_t* dst = p.o + (int64_t)b * p.q_batch + (int64_t)h * p.q_head + (int64_t)row * p.q_row + 4 * d4;
    uint2 packed;
    packed.x = to_bf16_bits(ov[0], p.round_mode) | (to_bf16_bits(ov[1], p.round_mode) << 16);
    packed.y = to_bf16_bits(ov[2], p.round_mode) | (to_bf16_bits(ov[3], p.round_mode) << 16);
    *(uint2*)dst = packed;
}

// ------------------------------------------------------------------ launch
int launch(const AttnParams& p, hipStream_t stream) {
    dim3 grid(p.n_blocks), block(NW * 64);
    if (p.c > 0.f)
        hipLaunchKernelGGL((attn_fwd_main<true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_main<false>), grid, block, 0, stream, p);
    if (hipGetLastError() != hipSuccess) return -1;
    if (p.kv_splits > 1) {
        const int64_t total = (int64_t)p.n_items * KERNEL_BM * (D / 4);
        dim3 cgrid((unsigned)((total + 255) / 256));
        hipLaunchKernelGGL((attn_fwd_combine<KERNEL_BM>), cgrid, dim3(256), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

}  // namespace attn
