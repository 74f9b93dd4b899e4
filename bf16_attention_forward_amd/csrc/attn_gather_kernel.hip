// attn_gather_kernel.hip -- gfx950 copy of a paged key/value cache into
// contiguous rows, ahead of the attention kernel.
//
// The FlyDSL diffusion-attention article (the section on what diffusion
// inference needs from an attention kernel) names flexible and paged
// KV-cache layouts.  A paged cache holds each sequence's keys and values in
// fixed-size pages of page_size token rows, [num_pages][page_size][Hkv][D],
// and a block table maps the sequence's logical page i to a physical page.
// This kernel writes batch entry b's first kv_lens[b] rows, in order, into
// [B][max_kv][Hkv][D]; the attention kernel then reads them like any
// contiguous BSHD key/value tensor, with kv_lens[b] keys in entry b.  It is
// a pure copy, bound by HBM: 16-byte loads and stores, one thread per
// 16-byte chunk of a row, the chunks of a row on consecutive lanes.
// Block-table entries outside [0, num_pages) give zero rows (the copy never
// reads outside the cache); rows at or past kv_lens[b] are not written (the
// attention kernel does not read them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"

namespace attn {

constexpr int GATHER_ROWS = 16;   // token rows per work-group

__global__ __launch_bounds__(256) void attn_gather_kv(const GatherParams p) {
    const int b = blockIdx.y;
    const int kvl = min(max(p.kv_lens[b], 0), p.max_kv);
    const int r0 = blockIdx.x * GATHER_ROWS;
    if (r0 >= kvl) return;
    const int chunks = p.row_elems / 8;            // 16-byte chunks per row
    const int n = GATHER_ROWS * chunks;
    const int* bt = p.block_table + (int64_t)b * p.pages_per_seq;
    for (int idx = threadIdx.x; idx < n; idx += 256) {
        const int i = r0 + idx / chunks, c = idx % chunks;
        if (i >= kvl) break;                        // rows run in order within the loop
        const int pg = bt[i / p.page_size];
        uint4 kq = make_uint4(0u, 0u, 0u, 0u), vq = make_uint4(0u, 0u, 0u, 0u);
        if (pg >= 0 && (int64_t)pg < p.num_pages) {
            const int64_t src = ((int64_t)pg * p.page_size + i % p.page_size) * p.row_elems + 8 * c;
            kq = *(const uint4*)(p.k_cache + src);
            vq = *(const uint4*)(p.v_cache + src);
        }
        const int64_t dst = ((int64_t)b * p.max_kv + i) * p.row_elems + 8 * c;
        *(uint4*)(p.k_out + dst) = kq;
        *(uint4*)(p.v_out + dst) = vq;
    }
}

int launch_gather(const GatherParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((p.max_kv + GATHER_ROWS - 1) / GATHER_ROWS), (unsigned)p.B);
    hipLaunchKernelGGL(attn_gather_kv, grid, dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace attn
