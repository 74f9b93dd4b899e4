// attn_fwd_internal.h -- parameters shared by the host planner and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Tiling of the kernels: KERNEL_NW waves per work-group, each owning
// KERNEL_NQB blocks of 16 query rows; KERNEL_BM query rows per work item.
// Short key ranges (at most KERNEL_SHORT_KV_TILES tiles of 64 keys, head
// dimension 128, no causal mask) use work-groups of KERNEL_NW_SHORT waves
// instead, two per CU: a work item then spends a large share of its time
// loading Q and storing O, and a second resident work-group keeps the
// matrix cores busy meanwhile.
#ifndef KERNEL_NQB
#define KERNEL_NQB 2
#endif
#ifndef KERNEL_NW
#define KERNEL_NW 8
#endif
#ifndef KERNEL_NW_SHORT
#define KERNEL_NW_SHORT 4
#endif
#ifndef KERNEL_SHORT_KV_TILES
#define KERNEL_SHORT_KV_TILES 16
#endif
#define KERNEL_BM (KERNEL_NW * 16 * KERNEL_NQB)
// work-groups resident per CU: two waves per SIMD in total (the register
// budget of a wave is then 256 VGPRs)
#define KERNEL_WG_PER_CU (8 / KERNEL_NW)

// Size of the fixed device array behind the allocation-free entry point: the
// largest split workspace the planner asks for on a 256-CU device (256
// partial query tiles of 256 rows, fp32 O of 128 dims plus (M, l)).
#define NOALLOC_SCRATCH_BYTES (256 * 256 * (128 + 2) * 4)
#define NOALLOC_MAX_DEVICES 64

namespace attn {

// Address of the fixed scratch array on device `dev` (which must be the
// current device); looked up once per device.  0 on success.
int scratch_address(int dev, void** out);

enum { ROUND_RTNE = 0, ROUND_RTNA = 1, ROUND_RTZ = 2 };
enum { ORDER_NAIVE = 1, ORDER_XCD = 2 };

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;        // optional [B][H][Sq] natural-log log-sum-exp per query row (NULL: not written)
    const int* kv_lens;  // optional [B] keys of each batch entry, clamped to [0, Skv] (NULL: Skv each)
    const int* cu_q;     // optional packed sequences: [B + 1] prefix sums of the query rows (Sq: the longest)
    const int* cu_k;     // and of the key rows (Skv: the longest); q, o, k, v hold the rows of all entries
    int total_q, total_k;  // rows of the packed tensors
    // keys and values read in place from a paged cache (k, v: [pages][page_size][Hkv][D])
    const int* block_table;  // optional [B][pages_per_seq]: page of each page_size rows of an entry
    int page_shift;          // log2(page_size), page_size a power of two >= 64 (one key tile per page at most)
    int pages_per_seq;
    int64_t num_pages;
    float* ws_o;       // split partial outputs [n_items - n_full][kv_splits][BM][128] (fp32)
    float* ws_ml;      // split partial (M, l) pairs [n_items - n_full][kv_splits][BM][2]
    int64_t q_row, q_head, q_batch;      // element strides of q and o
    int64_t kv_row, kv_head, kv_batch;   // element strides of k and v
    int B, H, Sq, Skv;  // H = query heads
    int group;         // query heads per key/value head (query head h reads key/value head h / group)
    int causal;        // 1: query i sees keys j <= i + causal_off (items never split, longest first)
    int causal_off;    // Skv - Sq
    int n_qtiles;      // ceil(Sq / BM)
    int n_items;       // B * H * n_qtiles
    int n_full;        // work items [0, n_full) run unsplit (one block each)
    int kv_splits;     // key ranges of each item in [n_full, n_items) (1 = no split)
    int n_kv_tiles;    // ceil(Skv / 64)
    int n_blocks;      // n_full + (n_items - n_full) * kv_splits
    int grid;          // work-groups launched: n_blocks, or fewer (a multiple of 8) for a persistent grid
    int block_order;   // ORDER_NAIVE or ORDER_XCD
    int round_mode;
    int head_dim;      // 128 or 64
    int p_mode;        // rounding of the in-loop bf16 weights (ROUND_RTNE unless asked otherwise)
    int nw;            // waves per work-group: KERNEL_NW, or KERNEL_NW_SHORT (query tile nw * 16 * KERNEL_NQB rows)
    float c;           // fp32(scale * log2(e))
};

int launch(const AttnParams& p, hipStream_t stream);

// Copy of a paged key/value cache into contiguous BSHD rows, for the
// attention kernel: row i < kv_lens[b] of batch entry b comes from row
// i % page_size of page block_table[b][i / page_size] of the cache.
struct GatherParams {
    const uint16_t* k_cache;   // [num_pages][page_size][Hkv][D]
    const uint16_t* v_cache;
    const int* block_table;    // [B][pages_per_seq]
    const int* kv_lens;        // [B]
    uint16_t* k_out;           // [B][max_kv][Hkv][D]
    uint16_t* v_out;
    int64_t num_pages;
    int B, max_kv, page_size, pages_per_seq;
    int row_elems;             // Hkv * D
};

int launch_gather(const GatherParams& p, hipStream_t stream);

}  // namespace attn
