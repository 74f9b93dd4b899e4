// attn_api.cpp -- C ABI of the gfx950 bf16 attention-forward library.
//
// Host side only: argument validation, the device check (gfx950 only), the
// work planner (query tiles, optional key-range split, block order) and the
// per-(device, stream) split workspace.  Every step of the computation runs
// in the kernels of attn_fwd_kernel.hip; nothing here touches tensor data.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <functional>
#include <mutex>
#include <vector>

#include "attn_bwd_internal.h"
#include "attn_fwd_internal.h"
#include "../../include/attn_fwd.h"

static_assert(NOALLOC_SCRATCH_BYTES == ATTN_NOALLOC_SCRATCH_BYTES, "the header states the fixed array's size");

namespace {

constexpr int kKeyTile = 64;
constexpr int kMaxSplits = 64;
constexpr int kMaxDevices = 64;

struct DeviceInfo {
    bool probed = false;
    bool gfx950 = false;
    int n_cu = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

struct Workspace {
    int device;
    void* stream;
    void* ptr;
    size_t bytes;
};
std::vector<Workspace> g_ws;

struct Cleanup {
    ~Cleanup() {
        for (auto& w : g_ws) if (w.ptr) (void)hipFree(w.ptr);
    }
} g_cleanup;

int probe_device(int* dev_out, DeviceInfo* info) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceInfo& d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
        d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.n_cu = prop.multiProcessorCount;
        d.probed = true;
    }
    *dev_out = dev;
    *info = d;
    return d.gfx950 ? ATTN_OK : ATTN_ERR_DEVICE;
}

// Workspace of at least `bytes` for (device, stream).  Buffers come from the
// stream-ordered allocator on that stream: an outgrown buffer is released
// with hipFreeAsync on the same stream, so the release waits for the launches
// already queued there (the only users of a per-stream buffer) without the
// host waiting for anything.  Grows to at least twice the old size.  Never
// allocates while the stream is being captured into a graph.
int get_workspace(int dev, void* stream, size_t bytes, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace* w = nullptr;
    for (auto& e : g_ws)
        if (e.device == dev && e.stream == stream) w = &e;
    if (w && w->bytes >= bytes) {
        *out = w->ptr;
        return ATTN_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return ATTN_ERR_WORKSPACE;
    const size_t want = w ? std::max(bytes, 2 * w->bytes) : bytes;
    void* p = nullptr;
    if (hipMallocAsync(&p, want, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_WORKSPACE;
    if (w) {
        if (hipFreeAsync(w->ptr, (hipStream_t)stream) != hipSuccess) {
            (void)hipFreeAsync(p, (hipStream_t)stream);
            return ATTN_ERR_WORKSPACE;
        }
        w->ptr = p;
        w->bytes = want;
    } else {
        g_ws.push_back(Workspace{dev, stream, p, want});
    }
    *out = p;
    return ATTN_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int attn_version(void) { return 10600; }

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_LAYOUT: return "layout must be ATTN_LAYOUT_BSHD or ATTN_LAYOUT_BHSD";
        case ATTN_ERR_ROUND_MODE: return "round_mode must be ATTN_ROUND_RTNE, _RTNA or _RTZ, optionally | ATTN_ROUND_WEIGHTS";
        case ATTN_ERR_SHAPE: return "B, H (Hq, Hkv), Sq and Skv must be >= 1, Hq a multiple of Hkv, head_dim 128 or 64, and the sizes must fit the kernel's index range";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned";
        case ATTN_ERR_ALIAS: return "o must not overlap q, k or v";
        case ATTN_ERR_DEVICE: return "the current device is not a gfx950 GPU";
        case ATTN_ERR_WORKSPACE: return "split workspace unavailable (allocation failed or stream is being captured)";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_OPTION: return "kv_splits, block_order, waves or causal out of range";
        case ATTN_ERR_SCRATCH: return "the call's split partials need more than the fixed scratch array of the "
                                      "allocation-free entry point holds (ATTN_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

namespace {

// Options of run_attention beyond the operation itself.
struct RunOpts {
    int kv_splits = 0, block_order = 0, waves = 0;   // planner overrides (0: the planner's choice)
    int grid = 0;                  // at most this many work-groups (0: the planner's choice)
    bool noalloc = false;          // split partials in the fixed device array
    const int* kv_lens = nullptr;  // device [B]: keys of each batch entry (per-entry lengths run unsplit)
    const int* cu_q = nullptr;     // device [B + 1]: packed sequences, prefix sums of the query rows
    const int* cu_k = nullptr;     // and of the key rows (Sq, Skv: the longest sequence)
    int64_t total_q = 0, total_k = 0;   // rows of the packed tensors
    const int* block_table = nullptr;   // device [B][pages_per_seq]: k, v are a paged cache read in place
    int page_shift = 0, pages_per_seq = 0;
    int64_t num_pages = 0;
    bool kv_internal = false;      // k, v: the library's own BSHD copy (no alias or alignment check)
    bool check_only = false;       // validate the arguments, touch no device
    std::function<int(int)> pre_launch;   // runs after every check, right before the kernels are queued
};

// Shared by every entry point: H = query heads, Hkv = key/value heads.
int run_attention(const void* q, const void* k, const void* v, void* o, float* lse,
                  int layout, int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t head_dim,
                  float scale, int causal, int round_mode, void* stream, const RunOpts& opt) {
    const int kv_splits = opt.kv_splits, block_order = opt.block_order, waves = opt.waves;
    const bool noalloc = opt.noalloc;
    const int* kv_lens = opt.kv_lens;
    const bool packed = opt.cu_q != nullptr;             // packed sequences (rows of all entries in one tensor)
    const bool per_entry = kv_lens || packed;            // per-entry key counts: unsplit, one block per work-group
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    if (packed && (!opt.cu_k || layout != ATTN_LAYOUT_BSHD)) return ATTN_ERR_NULL;
    if (layout != ATTN_LAYOUT_BSHD && layout != ATTN_LAYOUT_BHSD) return ATTN_ERR_LAYOUT;
    const int out_mode = round_mode & ~ATTN_ROUND_WEIGHTS;
    if (out_mode != ATTN_ROUND_RTNE && out_mode != ATTN_ROUND_RTNA && out_mode != ATTN_ROUND_RTZ)
        return ATTN_ERR_ROUND_MODE;
    if (B < 1 || H < 1 || Hkv < 1 || Sq < 1 || Skv < 1) return ATTN_ERR_SHAPE;
    if (head_dim != 128 && head_dim != 64) return ATTN_ERR_SHAPE;
    const int64_t kHeadDim = head_dim;
    if (H % Hkv != 0) return ATTN_ERR_SHAPE;
    // index-range limits of the kernels: 32-bit counts and per-head buffer extents
    const int64_t lim31 = (int64_t)1 << 31;
    if (B >= lim31 || H >= lim31 || Sq >= lim31 || Skv >= lim31) return ATTN_ERR_SHAPE;
    if (B * H >= lim31) return ATTN_ERR_SHAPE;
    if (packed && (opt.total_q < 1 || opt.total_k < 1 || opt.total_q >= lim31 || opt.total_k >= lim31))
        return ATTN_ERR_SHAPE;
    // elements of q (and o) and of k (and v): packed tensors hold total rows
    const int64_t n_q = packed ? opt.total_q * H : B * H * Sq;
    const int64_t n_kv = packed ? opt.total_k * Hkv : B * Hkv * Skv;
    if (n_q > ((int64_t)1 << 52) / kHeadDim || n_kv > ((int64_t)1 << 52) / kHeadDim) return ATTN_ERR_SHAPE;
    const bool kv_rows_bshd = opt.kv_internal || layout == ATTN_LAYOUT_BSHD;
    const int64_t kv_row = kv_rows_bshd ? Hkv * kHeadDim : kHeadDim;
    if ((Skv - 1) * kv_row * 2 + kHeadDim * 2 >= lim31) return ATTN_ERR_SHAPE;
    // work-group size: the 4-wave group (two per CU) for short key ranges
    const int64_t n_kv_tiles64 = (Skv + kKeyTile - 1) / kKeyTile;
    const bool short_ok = head_dim == 128 && !causal;   // where the 4-wave variant exists
    if (waves != 0 && waves != KERNEL_NW && !(waves == KERNEL_NW_SHORT && short_ok)) return ATTN_ERR_OPTION;
    const int nw = waves ? waves
                         : ((short_ok && n_kv_tiles64 <= KERNEL_SHORT_KV_TILES) ? KERNEL_NW_SHORT : KERNEL_NW);
    const int64_t bm = (int64_t)nw * 16 * KERNEL_NQB;   // query rows per work item
    const int64_t n_qtiles = (Sq + bm - 1) / bm;
    if (B * H * n_qtiles * kMaxSplits >= lim31) return ATTN_ERR_SHAPE;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)o | (opt.kv_internal ? 0 : ((uintptr_t)k | (uintptr_t)v))) & 15) return ATTN_ERR_ALIGN;
    // (the library's own key/value copy overlaps nothing of the caller's)
    const size_t q_bytes = (size_t)n_q * kHeadDim * 2, kv_bytes = opt.kv_internal ? 0 : (size_t)n_kv * kHeadDim * 2;
    if (ranges_overlap(o, q_bytes, q, q_bytes) || ranges_overlap(o, q_bytes, k, kv_bytes) ||
        ranges_overlap(o, q_bytes, v, kv_bytes))
        return ATTN_ERR_ALIAS;
    if (lse) {
        if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
        const size_t lse_bytes = (size_t)n_q * sizeof(float);
        if (ranges_overlap(lse, lse_bytes, q, q_bytes) || ranges_overlap(lse, lse_bytes, k, kv_bytes) ||
            ranges_overlap(lse, lse_bytes, v, kv_bytes) || ranges_overlap(lse, lse_bytes, o, q_bytes))
            return ATTN_ERR_ALIAS;
    }
    if (kv_splits < 0 || kv_splits > kMaxSplits || block_order < 0 || block_order > 2) return ATTN_ERR_OPTION;
    if (causal != 0 && causal != 1) return ATTN_ERR_OPTION;
    if (causal && (kv_splits > 1 || block_order == 2)) return ATTN_ERR_OPTION;
    if (per_entry && kv_splits > 1) return ATTN_ERR_OPTION;
    if (opt.grid < 0 || (opt.grid > 0 && per_entry)) return ATTN_ERR_OPTION;
    if (kv_lens && ((uintptr_t)kv_lens & 3)) return ATTN_ERR_ALIGN;
    if (packed && (((uintptr_t)opt.cu_q | (uintptr_t)opt.cu_k) & 3)) return ATTN_ERR_ALIGN;
    if (opt.check_only) return ATTN_OK;

    int dev = -1;
    DeviceInfo info;
    const int drc = probe_device(&dev, &info);
    if (drc != ATTN_OK) return drc;

    attn::AttnParams p;
    std::memset(&p, 0, sizeof p);
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.kv_lens = kv_lens;
    p.cu_q = opt.cu_q;
    p.cu_k = opt.cu_k;
    p.total_q = (int)opt.total_q;
    p.total_k = (int)opt.total_k;
    p.block_table = opt.block_table;
    p.page_shift = opt.page_shift;
    p.pages_per_seq = opt.pages_per_seq;
    p.num_pages = opt.num_pages;
    if (layout == ATTN_LAYOUT_BSHD) {
        p.q_row = H * kHeadDim; p.q_head = kHeadDim; p.q_batch = Sq * H * kHeadDim;
    } else {
        p.q_row = kHeadDim; p.q_head = Sq * kHeadDim; p.q_batch = H * Sq * kHeadDim;
    }
    if (kv_rows_bshd) {
        p.kv_row = Hkv * kHeadDim; p.kv_head = kHeadDim; p.kv_batch = Skv * Hkv * kHeadDim;
    } else {
        p.kv_row = kHeadDim; p.kv_head = Skv * kHeadDim; p.kv_batch = Hkv * Skv * kHeadDim;
    }
    if (opt.block_table) p.kv_batch = 0;   // a paged cache: an entry's rows come from its pages
    p.B = (int)B; p.H = (int)H; p.Sq = (int)Sq; p.Skv = (int)Skv;
    p.group = (int)(H / Hkv);
    p.causal = causal;
    p.causal_off = (int)(Skv - Sq);
    p.n_qtiles = (int)n_qtiles;
    p.n_items = (int)(B * H * n_qtiles);
    p.round_mode = out_mode;
    p.p_mode = (round_mode & ATTN_ROUND_WEIGHTS) ? out_mode : ATTN_ROUND_RTNE;
    p.head_dim = (int)head_dim;
    p.nw = nw;
    p.c = (float)((double)scale * 1.4426950408889634073599246810018921);

    // ---- plan the key-range split
    // The resident work-groups (one 8-wave or two 4-wave groups per CU: two
    // waves per SIMD) run the items in rounds of `slots` items.  When the
    // last round is ragged, the items of that
    // round have their key range split so that the round fills the chip (the
    // tail split); when there is less than one round of items, every item is
    // split.  A forced kv_splits = n splits every item n ways.
    const int n_kv_tiles = (int)((Skv + kKeyTile - 1) / kKeyTile);
    const int slots = info.n_cu * (8 / nw);   // resident work-groups: two waves per SIMD
    int n_full = p.n_items, splits = 1;
    if (causal || per_entry) {
        // Causal items differ in length (the diagonal), and so do the items
        // of batch entries with their own key counts: they run unsplit
        // (causal ones longest first, in naive block order: the kernel
        // numbers them so).
    } else if (kv_splits > 0) {
        if (kv_splits > n_kv_tiles) return ATTN_ERR_OPTION;   // every range must hold a key
        splits = kv_splits;
        n_full = (splits == 1) ? p.n_items : 0;
    } else {
        const int rem = p.n_items % slots;
        const int tail = (p.n_items < slots) ? p.n_items : rem;
        if (tail > 0 && tail <= slots / 2) {
            int s_auto = slots / tail;                           // blocks per tail item
            s_auto = std::min(s_auto, n_kv_tiles / 2);           // keep >= 2 key tiles per range
            s_auto = std::min(s_auto, kMaxSplits);
            if (s_auto >= 2) {
                splits = s_auto;
                n_full = p.n_items - tail;
            }
        }
    }
    p.n_full = n_full;
    p.kv_splits = splits;
    p.n_kv_tiles = n_kv_tiles;
    p.n_blocks = n_full + (p.n_items - n_full) * splits;
    // An 8-wave plan at head dimension 128 without per-entry key counts and
    // with more blocks than resident work-groups runs on a persistent grid
    // of one work-group per slot (the item loop does not pay at head
    // dimension 64): each runs one block per round and fetches the next
    // one's Q and first K tile under its current item's last iteration.
    // Without the causal mask every block costs the same and work-group w
    // takes blocks w, w + G, w + 2G, ...; causal blocks, longest first, are
    // walked back in every other round so that a long item pairs with a
    // short one.  The grid is a multiple of 8, so each block keeps the XCD
    // its order gave it.  Per-entry-length items keep one block per
    // work-group, so the hardware balances them as they finish; so do
    // 4-wave work-groups, two per CU, whose item boundaries overlap the
    // other's work only when they run out of step.  The next item's Q tile
    // moves through one buffer descriptor, so its extent must fit 31 bits.
    p.grid = p.n_blocks;
    const bool qtile_fits = (bm - 1) * (int64_t)p.q_row * 2 + kHeadDim * 2 < lim31;
    if (!per_entry && nw == KERNEL_NW && head_dim == 128 && qtile_fits) {
        const int cap = std::max(8, (opt.grid > 0 ? opt.grid : slots) & ~7);
        if (cap < p.n_blocks) p.grid = cap;
    }
    p.block_order = (block_order == 1 || causal) ? attn::ORDER_NAIVE : attn::ORDER_XCD;

    if (n_full < p.n_items) {
        const size_t n_part = (size_t)(p.n_items - n_full) * splits;
        const size_t need = n_part * bm * (kHeadDim + 2) * sizeof(float);
        void* ws = nullptr;
        if (noalloc) {
            // the fixed device array; nothing is allocated
            if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
            if (attn::scratch_address(dev, &ws) != 0) return ATTN_ERR_DEVICE;
        } else {
            const int wrc = get_workspace(dev, stream, need, &ws);
            if (wrc != ATTN_OK) return wrc;
        }
        p.ws_o = (float*)ws;
        p.ws_ml = (float*)((char*)ws + n_part * bm * kHeadDim * sizeof(float));
    }

    if (opt.pre_launch) {
        const int prc = opt.pre_launch(dev);
        if (prc != ATTN_OK) return prc;
    }
    if (attn::launch(p, (hipStream_t)stream) != 0) return ATTN_ERR_LAUNCH;
    return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_bf16_ex(const void* q, const void* k, const void* v, void* o,
                                int layout, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                float scale, int round_mode, void* stream,
                                int kv_splits, int block_order, int waves, int grid) {
    RunOpts opt;
    opt.kv_splits = kv_splits; opt.block_order = block_order; opt.waves = waves; opt.grid = grid;
    return run_attention(q, k, v, o, nullptr, layout, B, H, H, Sq, Skv, 128, scale, 0, round_mode, stream, opt);
}

extern "C" int attn_fwd_bf16_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                 float scale, int causal, int round_mode, void* stream) {
    return run_attention(q, k, v, o, lse, layout, B, Hq, Hkv, Sq, Skv, 128, scale, causal, round_mode, stream, RunOpts());
}

extern "C" int attn_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int64_t B, int64_t Hq, int64_t Hkv, int64_t total_q, int64_t total_k,
                                    int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t head_dim,
                                    float scale, int causal, int round_mode, void* stream) {
    if (!cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
    RunOpts opt;
    opt.cu_q = cu_seqlens_q;
    opt.cu_k = cu_seqlens_k;
    opt.total_q = total_q;
    opt.total_k = total_k;
    return run_attention(q, k, v, o, lse, ATTN_LAYOUT_BSHD, B, Hq, Hkv, max_seqlen_q, max_seqlen_k, head_dim,
                         scale, causal, round_mode, stream, opt);
}

extern "C" int attn_fwd_bf16_paged(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* kv_lens, void* o, float* lse,
                                   int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t max_kv_len,
                                   int64_t page_size, int64_t pages_per_seq, int64_t num_pages, int64_t head_dim,
                                   float scale, int causal, int round_mode, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !kv_lens || !o) return ATTN_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || max_kv_len < 1) return ATTN_ERR_SHAPE;
    if (head_dim != 128 && head_dim != 64) return ATTN_ERR_SHAPE;
    const int64_t lim31 = (int64_t)1 << 31;
    if (B >= lim31 || Hq >= lim31 || Hkv >= lim31 || Sq >= lim31 || max_kv_len >= lim31) return ATTN_ERR_SHAPE;
    if (page_size < 1 || page_size >= lim31 || num_pages < 1 || pages_per_seq < 1 || pages_per_seq >= lim31)
        return ATTN_ERR_SHAPE;
    if (pages_per_seq < (max_kv_len + page_size - 1) / page_size) return ATTN_ERR_SHAPE;   // the table covers max_kv_len
    if (B * pages_per_seq >= lim31 || Hkv * head_dim >= lim31) return ATTN_ERR_SHAPE;
    const int64_t row_elems = Hkv * head_dim;
    if (num_pages > ((int64_t)1 << 52) / page_size / row_elems) return ATTN_ERR_SHAPE;
    if (((uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return ATTN_ERR_ALIGN;
    if (((uintptr_t)block_table | (uintptr_t)kv_lens) & 3) return ATTN_ERR_ALIGN;
    const size_t cache_bytes = (size_t)num_pages * (size_t)page_size * (size_t)row_elems * 2;
    const size_t q_bytes = (size_t)B * Hq * Sq * head_dim * 2;
    if (ranges_overlap(o, q_bytes, k_cache, cache_bytes) || ranges_overlap(o, q_bytes, v_cache, cache_bytes))
        return ATTN_ERR_ALIAS;
    if (lse && (ranges_overlap(lse, (size_t)B * Hq * Sq * 4, k_cache, cache_bytes) ||
                ranges_overlap(lse, (size_t)B * Hq * Sq * 4, v_cache, cache_bytes)))
        return ATTN_ERR_ALIAS;
    if (max_kv_len > ((int64_t)1 << 52) / row_elems / B) return ATTN_ERR_SHAPE;   // the copy's size
    // every check of q, o, lse, the mode and the sizes before anything is
    // allocated or queued (the key/value arguments are the library's copy)
    RunOpts opt;
    opt.kv_lens = kv_lens;
    opt.kv_internal = true;
    opt.kv_splits = 1;
    opt.check_only = true;
    const void* placeholder = k_cache;   // stands for the copy: not read while checking
    const int crc = run_attention(q, placeholder, placeholder, o, lse, layout, B, Hq, Hkv, Sq, max_kv_len, head_dim,
                                  scale, causal, round_mode, stream, opt);
    if (crc != ATTN_OK) return crc;
    // Pages of a power-of-two number of rows, at least one key tile: the
    // attention kernel reads the keys and values in place (a key tile never
    // straddles two pages); other page sizes go through a contiguous copy.
    if (page_size >= kKeyTile && (page_size & (page_size - 1)) == 0) {
        int shift = 0;
        while (((int64_t)1 << shift) < page_size) shift++;
        opt.check_only = false;
        opt.block_table = block_table;
        opt.page_shift = shift;
        opt.pages_per_seq = (int)pages_per_seq;
        opt.num_pages = num_pages;
        return run_attention(q, k_cache, v_cache, o, lse, layout, B, Hq, Hkv, Sq, max_kv_len, head_dim, scale,
                             causal, round_mode, stream, opt);
    }
    int dev = -1;
    DeviceInfo info;
    const int drc = probe_device(&dev, &info);
    if (drc != ATTN_OK) return drc;
    // the contiguous copy of the keys and values the attention kernel reads
    const size_t kv_bytes = (size_t)B * max_kv_len * row_elems * 2;
    void* ws = nullptr;
    const int wrc = get_workspace(dev, stream, 2 * kv_bytes, &ws);
    if (wrc != ATTN_OK) return wrc;
    uint16_t* kws = (uint16_t*)ws;
    uint16_t* vws = (uint16_t*)((char*)ws + kv_bytes);
    opt.check_only = false;
    opt.pre_launch = [&](int) -> int {
        attn::GatherParams g;
        g.k_cache = (const uint16_t*)k_cache; g.v_cache = (const uint16_t*)v_cache;
        g.block_table = block_table; g.kv_lens = kv_lens;
        g.k_out = kws; g.v_out = vws;
        g.num_pages = num_pages;
        g.B = (int)B; g.max_kv = (int)max_kv_len; g.page_size = (int)page_size; g.pages_per_seq = (int)pages_per_seq;
        g.row_elems = (int)row_elems;
        return attn::launch_gather(g, (hipStream_t)stream) == 0 ? ATTN_OK : ATTN_ERR_LAUNCH;
    };
    // the attention on the copy, unsplit, with the per-entry key counts
    return run_attention(q, kws, vws, o, lse, layout, B, Hq, Hkv, Sq, max_kv_len, head_dim, scale, causal,
                         round_mode, stream, opt);
}

extern "C" int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dO,
                             const float* lse, void* dq, void* dk, void* dv, int layout, int64_t B, int64_t H,
                             int64_t Hkv, int64_t Sq, int64_t Skv, int64_t head_dim, float scale, int causal,
                             void* stream) {
    if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
    if (layout != ATTN_LAYOUT_BSHD && layout != ATTN_LAYOUT_BHSD) return ATTN_ERR_LAYOUT;
    if (B < 1 || H < 1 || Hkv < 1 || Sq < 1 || Skv < 1) return ATTN_ERR_SHAPE;
    if (H % Hkv != 0) return ATTN_ERR_SHAPE;
    if (head_dim != 128 && head_dim != 64) return ATTN_ERR_SHAPE;
    const int64_t lim31 = (int64_t)1 << 31, hd = head_dim;
    if (B >= lim31 || H >= lim31 || Sq >= lim31 || Skv >= lim31 || B * H >= lim31) return ATTN_ERR_SHAPE;
    const int64_t n_q = B * H * Sq, n_kv = B * Hkv * Skv;
    if (n_q > ((int64_t)1 << 52) / hd || n_kv > ((int64_t)1 << 52) / hd) return ATTN_ERR_SHAPE;
    const int64_t q_rowe = (layout == ATTN_LAYOUT_BSHD) ? H * hd : hd;
    const int64_t kv_rowe = (layout == ATTN_LAYOUT_BSHD) ? Hkv * hd : hd;
    if ((Sq - 1) * q_rowe * 2 + hd * 2 >= lim31 || (Skv - 1) * kv_rowe * 2 + hd * 2 >= lim31) return ATTN_ERR_SHAPE;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (causal != 0 && causal != 1) return ATTN_ERR_OPTION;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dO | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv) & 15)
        return ATTN_ERR_ALIGN;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    const size_t qb = (size_t)n_q * hd * 2, kb = (size_t)n_kv * hd * 2, lb = (size_t)n_q * 4;
    // outputs overlap no input and no other output
    const void* ins[6] = {q, k, v, o, dO, lse};
    const size_t insz[6] = {qb, kb, kb, qb, qb, lb};
    const void* outs[3] = {dq, dk, dv};
    const size_t outsz[3] = {qb, kb, kb};
    for (int a = 0; a < 3; a++) {
        for (int i = 0; i < 6; i++)
            if (ranges_overlap(outs[a], outsz[a], ins[i], insz[i])) return ATTN_ERR_ALIAS;
        for (int c = a + 1; c < 3; c++)
            if (ranges_overlap(outs[a], outsz[a], outs[c], outsz[c])) return ATTN_ERR_ALIAS;
    }
    int dev = -1;
    DeviceInfo info;
    const int drc = probe_device(&dev, &info);
    if (drc != ATTN_OK) return drc;

    attn_bwd::BwdParams p;
    std::memset(&p, 0, sizeof p);
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.o = (const uint16_t*)o; p.dO = (const uint16_t*)dO; p.lse = lse;
    p.dq = (uint16_t*)dq; p.dk = (uint16_t*)dk; p.dv = (uint16_t*)dv;
    if (layout == ATTN_LAYOUT_BSHD) {
        p.q_row = H * hd; p.q_head = hd; p.q_batch = Sq * H * hd;
        p.kv_row = Hkv * hd; p.kv_head = hd; p.kv_batch = Skv * Hkv * hd;
    } else {
        p.q_row = hd; p.q_head = Sq * hd; p.q_batch = H * Sq * hd;
        p.kv_row = hd; p.kv_head = Skv * hd; p.kv_batch = Hkv * Skv * hd;
    }
    p.B = (int)B; p.H = (int)H; p.Sq = (int)Sq; p.Skv = (int)Skv;
    p.Hkv = (int)Hkv; p.group = (int)(H / Hkv);
    p.n_qblocks = (int)((Sq + 255) / 256);
    p.n_kblocks = (int)((Skv + 127) / 128);
    if (B * H * std::max(p.n_qblocks, p.n_kblocks) >= lim31) return ATTN_ERR_SHAPE;
    p.c = (float)((double)scale * 1.4426950408889634073599246810018921);
    p.scale = scale;
    p.causal = causal;
    p.causal_off = (int)(Skv - Sq);
    p.head_dim = (int)head_dim;
    void* ws = nullptr;
    const int wrc = get_workspace(dev, stream, 2 * (size_t)n_q * sizeof(float), &ws);
    if (wrc != ATTN_OK) return wrc;
    p.delta = (float*)ws;
    p.lse2 = (float*)ws + n_q;
    if (attn_bwd::launch_bwd(p, (hipStream_t)stream) != 0) return ATTN_ERR_LAUNCH;
    return ATTN_OK;
}

extern "C" int attn_fwd_bf16_hd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                int64_t head_dim, float scale, int causal, int round_mode, void* stream) {
    return run_attention(q, k, v, o, lse, layout, B, Hq, Hkv, Sq, Skv, head_dim, scale, causal, round_mode,
                         stream, RunOpts());
}

extern "C" int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                             int layout, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                             float scale, int round_mode, void* stream) {
    return attn_fwd_bf16_ex(q, k, v, o, layout, B, H, Sq, Skv, scale, round_mode, stream, 0, 0, 0, 0);
}

extern "C" int attn_fwd_bf16_hd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                        int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                        int64_t head_dim, float scale, int causal, int round_mode, void* stream) {
    RunOpts opt;
    opt.noalloc = true;
    return run_attention(q, k, v, o, lse, layout, B, Hq, Hkv, Sq, Skv, head_dim, scale, causal, round_mode,
                         stream, opt);
}
