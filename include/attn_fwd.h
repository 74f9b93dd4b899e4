/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) bf16 attention-forward library.
 *
 * One call computes non-causal attention
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * <Q[b,h,i,:], K[b,h,j,:]>) * V[b,h,j,:]
 *
 * for head dimension 128, with bf16 inputs and a bf16 output rounded in a
 * caller-selected mode.  The operation, the fixed head dimension, the two
 * storage layouts (BSHD and BHSD, used as they are, never transposed), the
 * freedom of Sq and Skv (cross-attention included) and the three rounding
 * modes are those of the bf16 forward kernel in "MoonMath AI open-sources a
 * HIP attention kernel for AMD MI300X that beats AITER" (opening paragraphs
 * on what the kernel computes, its interface and its numerics).  Causal
 * masking, grouped-query attention and variable-length batches are not part
 * of this interface (the same article lists them as limitations).
 *
 * Like that kernel, a call launches asynchronously on the caller's stream
 * (same article, use-case section), so it can overlap with other work.
 *
 * No HIP or torch type appears here: pointers are plain device addresses and
 * the stream is passed as an opaque pointer (a hipStream_t, NULL = the
 * legacy default stream).
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage layouts of q, k, v and o (all four share one layout). */
enum {
    ATTN_LAYOUT_BSHD = 0, /* [B, S, H, 128], element (b,s,h,d) at ((b*S + s)*H + h)*128 + d */
    ATTN_LAYOUT_BHSD = 1  /* [B, H, S, 128], element (b,h,s,d) at ((b*H + h)*S + s)*128 + d */
};

/* Rounding of the fp32 result to the bf16 output (IEEE 754 meanings). */
enum {
    ATTN_ROUND_RTNE = 0, /* to nearest, ties to even                      */
    ATTN_ROUND_RTNA = 1, /* to nearest, ties away from zero               */
    ATTN_ROUND_RTZ  = 2  /* toward zero (finite overflow -> max finite)   */
};

/* Flag OR'ed into round_mode: the softmax weights that enter the bf16 P.V
 * product are rounded with the same mode as the output (without it they are
 * rounded to nearest-even).  The MoonMath article measures each output mode
 * at a different speed (benchmark section), which reads as the weights being
 * rounded in the loop with the selected mode too; this flag selects that
 * reading.  RTNA and RTNE weights differ only on exact ties. */
enum { ATTN_ROUND_WEIGHTS = 0x100 };

/* Status codes.  Every argument error is detected on the host before any
 * launch; on error nothing is launched and o is not written. */
enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,        /* a required pointer is NULL                        */
    ATTN_ERR_LAYOUT = -2,      /* layout is not one of ATTN_LAYOUT_*                */
    ATTN_ERR_ROUND_MODE = -3,  /* round_mode is not ATTN_ROUND_* [| ATTN_ROUND_WEIGHTS] */
    ATTN_ERR_SHAPE = -4,       /* a size < 1, Hq not a multiple of Hkv, head_dim not
                                  64 or 128, or overflow                            */
    ATTN_ERR_SCALE = -5,       /* scale is NaN or infinite                          */
    ATTN_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned                  */
    ATTN_ERR_ALIAS = -7,       /* o overlaps q, k or v                              */
    ATTN_ERR_DEVICE = -8,      /* current device is not gfx950, or no device        */
    ATTN_ERR_WORKSPACE = -9,   /* split workspace could not be obtained             */
    ATTN_ERR_LAUNCH = -10,     /* the HIP runtime rejected a launch                 */
    ATTN_ERR_OPTION = -11,     /* kv_splits, block_order or causal out of range     */
    ATTN_ERR_SCRATCH = -12     /* attn_fwd_bf16_hd_noalloc: the split partials need
                                  more than ATTN_NOALLOC_SCRATCH_BYTES              */
};

/*
 * attn_fwd_bf16 -- O = softmax(Q K^T * scale) V, bf16 in, bf16 out.
 *
 *   q   [B,Sq,H,128] or [B,H,Sq,128] bf16, contiguous, device memory (read)
 *   k   [B,Skv,H,128] or [B,H,Skv,128] bf16, contiguous, device (read)
 *   v   same shape as k (read)
 *   o   same shape as q, bf16, device (written; must not overlap q/k/v)
 *   layout       ATTN_LAYOUT_BSHD or ATTN_LAYOUT_BHSD, shared by all four
 *   B, H         batch and heads (>= 1); H is shared by q and k/v
 *   Sq, Skv      query and key/value lengths (>= 1), independent
 *   scale        finite fp32 multiplier of the scores (1/sqrt(128) is usual;
 *                0 gives the uniform average of V)
 *   round_mode   ATTN_ROUND_* for the final fp32 -> bf16 conversion, optionally
 *                | ATTN_ROUND_WEIGHTS to round the in-loop weights the same way
 *   stream       hipStream_t to launch on (NULL = default stream)
 *
 * Ownership: the caller owns q, k, v, o and keeps them alive until the
 * stream's work completes.  The library keeps a workspace per (device,
 * stream) for the split-KV partial results.  It comes from the stream-ordered
 * allocator on that stream and grows on demand (at least doubling; the
 * outgrown buffer is released in stream order, after the launches already
 * queued on the stream); it is never allocated while the stream is being
 * captured into a graph (ATTN_ERR_WORKSPACE instead, so capture needs one
 * eager call of the same shape first), and lives until unload.
 *
 * Returns ATTN_OK or an ATTN_ERR_* code.  The call never synchronizes:
 * device faults surface at the caller's next synchronization.  NaN and Inf
 * inputs propagate as IEEE arithmetic on the definition implies; the output
 * NaN is 0x7FC0.  Results are bitwise deterministic for a given device,
 * shape, layout and mode.
 */
int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                  int layout, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                  float scale, int round_mode, void* stream);

/*
 * attn_fwd_bf16_ex -- attn_fwd_bf16 with planner overrides, for tests and
 * ablations.
 *
 * The planner (kv_splits = 0) runs the work items in rounds that fill every
 * CU; when the last round of query tiles is ragged (or there is less than
 * one round), the query tiles of that round have their key range split so
 * the round fills the GPU, and a combine kernel merges the partial results
 * in a fixed order (the flash-decoding style tail split of "MoonMath AI
 * open-sources a HIP attention kernel for AMD MI300X", section on the two
 * later improvements).  Work-groups have 8 waves (256 query rows, one per
 * CU), or, for key ranges of at most 16 tiles of 64 keys, 4 waves (128
 * rows, two per CU, so one's Q loads and O stores overlap the other's
 * matrix work).
 *
 * kv_splits: 0 = planner's choice; 1 = never split; n >= 2 splits every
 * query tile's keys into n contiguous ranges of whole 64-key tiles (n must
 * not exceed the number of 64-key tiles, n <= 64).  block_order: 0 =
 * planner's choice (XCD-aware), 1 = naive (work item = block id), 2 =
 * XCD-aware.  waves: 0 = planner's choice, 8 or 4 waves per work-group.
 * grid: 0 = planner's choice (an 8-wave plan of more work-groups than the
 * GPU holds at once runs on a persistent grid of one work-group per CU,
 * each taking every grid-th block of the plan); n >= 1 = at most n 8-wave
 * work-groups (n rounded down to a multiple of 8, at least 8; 4-wave
 * work-groups always run one per block, and so does every plan whose
 * 256-row query tile spans 2 GiB or more of q).  Other values return
 * ATTN_ERR_OPTION.  The result does not depend on block_order, waves or
 * grid; it may differ in the last bits with kv_splits.
 */
int attn_fwd_bf16_ex(const void* q, const void* k, const void* v, void* o,
                     int layout, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                     float scale, int round_mode, void* stream,
                     int kv_splits, int block_order, int waves, int grid);

/*
 * attn_fwd_bf16_gqa -- attn_fwd_bf16 with grouped-query heads and an optional
 * causal mask, the two limitations the MoonMath article lists first
 * (limitations paragraph); the mask alignment is this library's choice.
 *
 *   q, o   [B,Sq,Hq,128] or [B,Hq,Sq,128] bf16 (as attn_fwd_bf16)
 *   k, v   [B,Skv,Hkv,128] or [B,Hkv,Skv,128] bf16
 *   Hq, Hkv  query and key/value heads (>= 1), Hq a multiple of Hkv; query
 *            head h reads key/value head h / (Hq / Hkv).  Hq == Hkv is
 *            plain multi-head attention.
 *   causal   0: every key; 1: query i sees keys j <= i + (Skv - Sq), i.e.
 *            the queries are the last Sq positions of the key sequence
 *            (for Sq == Skv the usual lower-triangular mask).  A query row
 *            that sees no key (only when Sq > Skv) is written as zeros.
 *            Non-finite values under the mask: a 256-row query tile runs
 *            every key below its last row's diagonal through the P.V
 *            product with zero weights for the keys a row does not see, so
 *            a NaN or Inf in V[j, d] makes column d NaN (0 * Inf) in the
 *            rows of such a tile that do not see key j.  Rows that see j,
 *            rows of tiles whose key range ends before j, and every finite
 *            input follow the definition.
 *   lse      NULL, or fp32 [B, Hq, Sq] (this order in both layouts), device
 *            memory, 4-byte aligned, not overlapping q/k/v/o: receives each
 *            row's natural-log log-sum-exp of its scaled scores,
 *            log(sum_j exp(scale * <q_i, k_j>)) over the keys it sees
 *            (-inf for a row that sees none) -- the softmax statistic a
 *            backward pass needs, and the intermediate the FlyDSL procedure
 *            article (debugging advice) compares against a reference.  It is
 *            computed from the bf16-rounded weights the product uses, so it
 *            differs from the exact value by about their rounding (< 2^-8).
 *
 * All other arguments, ownership, asynchrony and error behaviour are those of
 * attn_fwd_bf16; Hq not a multiple of Hkv gives ATTN_ERR_SHAPE, a causal
 * value other than 0 or 1 gives ATTN_ERR_OPTION, a misaligned lse
 * ATTN_ERR_ALIGN and an lse overlapping q, k, v or o ATTN_ERR_ALIAS.  Causal calls never split
 * the key range (no workspace): their work items, of unequal length, run
 * longest first instead.
 */
int attn_fwd_bf16_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                      int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                      float scale, int causal, int round_mode, void* stream);

/*
 * attn_fwd_bf16_hd -- attn_fwd_bf16_gqa for head dimension 128 or 64 (the two
 * sizes of the attention forward kernels in the HipKittens summary's kernel
 * suite).
 *
 *   q, o   [B,Sq,Hq,head_dim] or [B,Hq,Sq,head_dim] bf16
 *   k, v   [B,Skv,Hkv,head_dim] or [B,Hkv,Skv,head_dim] bf16
 *   head_dim 128 or 64; other values give ATTN_ERR_SHAPE.  The usual scale
 *            is 1/sqrt(head_dim).
 *
 * Every other argument, the lse output, ownership, asynchrony and error
 * behaviour are those of attn_fwd_bf16_gqa; with head_dim 128 the two calls
 * are the same.
 */
int attn_fwd_bf16_hd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                     int64_t head_dim, float scale, int causal, int round_mode, void* stream);

/*
 * attn_fwd_bf16_paged -- attn_fwd_bf16_hd with the keys and values in a paged
 * cache and a key count per batch entry: the flexible and paged KV-cache
 * layouts the FlyDSL diffusion-attention article lists among diffusion
 * inference's needs (its section on what such a kernel must offer).
 *
 *   q, o        [B,Sq,Hq,head_dim] or [B,Hq,Sq,head_dim] bf16 (`layout`, as
 *               attn_fwd_bf16_hd); lse as attn_fwd_bf16_gqa
 *   k_cache, v_cache  [num_pages][page_size][Hkv][head_dim] bf16, device
 *               memory, 16-byte aligned: page p holds page_size token rows
 *   block_table int32 [B][pages_per_seq], device memory: token row i of
 *               batch entry b is row i % page_size of page
 *               block_table[b][i / page_size]; pages may be shared between
 *               entries; an entry outside [0, num_pages) reads as zero rows
 *   kv_lens     int32 [B], device memory: keys of batch entry b, clamped to
 *               [0, max_kv_len]; a batch entry with no keys gives zero rows
 *               (and lse -inf)
 *   max_kv_len  >= 1, at least every kv_lens[b] that should count whole;
 *               pages_per_seq must cover it (pages_per_seq * page_size >=
 *               max_kv_len)
 *   causal      0, or 1: query i of entry b sees keys j <= i + kv_lens[b] -
 *               Sq (its queries are the last Sq positions of its keys)
 *
 * With page_size a power of two of at least 64 (a 64-key tile never
 * straddles two pages) the attention kernel reads the keys and values in
 * place, looking up each tile's page in the table; nothing is allocated.
 * Other page sizes go through a copy: the library first copies each entry's
 * kv_lens[b] key and value rows into a contiguous per-(device, stream)
 * workspace of 2 * B * max_kv_len * Hkv * head_dim bf16 values (HIP's
 * stream-ordered allocator, as for the split partials; ATTN_ERR_WORKSPACE
 * while the stream is being captured), then runs the attention kernel on it
 * with the per-entry key counts.  Either way the key range is never split
 * and the results are the same bits.  Every other argument, ownership, asynchrony and
 * error behaviour are those of attn_fwd_bf16_hd; page_size, pages_per_seq
 * or num_pages below 1, or a table too narrow for max_kv_len, give
 * ATTN_ERR_SHAPE; a misaligned cache, table or kv_lens ATTN_ERR_ALIGN; o or
 * lse overlapping a cache ATTN_ERR_ALIAS.
 */
int attn_fwd_bf16_paged(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* kv_lens, void* o, float* lse,
                        int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t max_kv_len,
                        int64_t page_size, int64_t pages_per_seq, int64_t num_pages, int64_t head_dim,
                        float scale, int causal, int round_mode, void* stream);

/*
 * attn_fwd_bf16_varlen -- attn_fwd_bf16_hd over a batch of packed sequences of
 * different lengths: the variable-length batches the MoonMath article lists
 * among its kernel's limitations (limitations paragraph), with the rows of all
 * sequences in one tensor and no padding (the flexible layouts of the FlyDSL
 * diffusion-attention article's section on what diffusion inference needs).
 *
 *   q, o        [total_q][Hq][head_dim] bf16, device, 16-byte aligned: the
 *               query (and output) rows of sequence b are rows
 *               cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   k, v        [total_k][Hkv][head_dim] bf16, device, 16-byte aligned: the
 *               key/value rows of sequence b are rows cu_seqlens_k[b] ..
 *               cu_seqlens_k[b+1]-1
 *   lse         NULL, or fp32 [Hq][total_q], device, 4-byte aligned: the
 *               natural-log log-sum-exp of each row's scaled scores (-inf
 *               for a row that sees no key)
 *   cu_seqlens_q, cu_seqlens_k  int32 [B+1], device, 4-byte aligned:
 *               non-decreasing prefix sums of the sequences' row counts
 *               (element 0 is 0, element B the total).  The kernel clamps
 *               every entry into [0, total] and each length to
 *               max_seqlen_q / max_seqlen_k, so no row outside the tensors
 *               is ever read or written
 *   B           sequences (>= 1); Hq, Hkv, head_dim as attn_fwd_bf16_hd
 *   total_q, total_k   rows of the packed tensors (>= 1)
 *   max_seqlen_q, max_seqlen_k  >= 1, at least every sequence's length
 *   causal      0, or 1: query i of sequence b sees keys j <= i + (len_k(b)
 *               - len_q(b)) (its queries are the last len_q(b) positions of
 *               its keys); rows of a sequence with no keys are zeros
 *
 * Each sequence attends only to its own keys; the key range is never split.
 * Ownership, asynchrony and error behaviour are those of attn_fwd_bf16_hd
 * (no workspace is used); missing cu_seqlens give ATTN_ERR_NULL, sizes
 * below 1 ATTN_ERR_SHAPE, misaligned cu_seqlens ATTN_ERR_ALIGN.
 */
int attn_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t total_q, int64_t total_k,
                         int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t head_dim,
                         float scale, int causal, int round_mode, void* stream);

/* Size in bytes of the fixed device array behind attn_fwd_bf16_hd_noalloc:
 * 256 partial query tiles x 256 rows x (128 + 2) fp32 values, the largest
 * split workspace the planner asks for on a 256-CU gfx950 device. */
#define ATTN_NOALLOC_SCRATCH_BYTES 34078720

/*
 * attn_fwd_bf16_hd_noalloc -- attn_fwd_bf16_hd for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It makes the same plan and gives the
 * same result bit for bit, but the split partials go to a fixed device
 * array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends, instead of a workspace it allocates.  The
 * call itself allocates nothing (no hipMalloc, no library allocation).
 *
 * Arguments, ownership of q, k, v, o and lse, asynchrony and errors are
 * those of attn_fwd_bf16_hd.  A call whose split partials would need more
 * than the array holds returns ATTN_ERR_SCRATCH and launches nothing; on a
 * 256-CU gfx950 the planner never asks for more.
 *
 * The array is shared by every call on the same GPU and keeps the last
 * call's partials (each call writes every partial it reads, so nothing has
 * to start at zero).  Calls on one GPU that overlap in time, e.g. on two
 * streams without ordering between them, race on it: order them on one
 * stream or through events.
 */
int attn_fwd_bf16_hd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                             int64_t head_dim, float scale, int causal, int round_mode, void* stream);

/*
 * attn_bwd_bf16 -- backward pass of attn_fwd_bf16 / attn_fwd_bf16_gqa /
 * attn_fwd_bf16_hd: dQ, dK, dV for a given dO.
 *
 * The gradients of O = softmax(Q K^T * scale) V follow from the chain rule on
 * the forward's definition (the HipKittens summary's kernel suite pairs the
 * attention forward with its backward); the pass starts, as usual, from the
 * forward's saved output and per-row log-sum-exp:
 *     P = exp(scale * Q K^T - lse),   dV = P^T dO,   dP = dO V^T,
 *     dS = P o (dP - delta),  delta_i = <dO_i, O_i>,
 *     dQ = scale * dS K,      dK = scale * dS^T Q.
 *
 *   q, o, dO   [B,Sq,H,D] or [B,H,Sq,D] bf16, device (read), D = head_dim;
 *              o is the forward output for these q, k, v, scale
 *   k, v       [B,Skv,Hkv,D] or [B,Hkv,Skv,D] bf16, device (read); query
 *              head h reads key/value head h / (H / Hkv) (attn_fwd_bf16_gqa's
 *              grouping; H a multiple of Hkv, else ATTN_ERR_SHAPE), and dK, dV
 *              of a key/value head sum over its query heads
 *   lse        fp32 [B, H, Sq], device (read): the forward's log-sum-exp
 *              (attn_fwd_bf16_gqa's lse output), 4-byte aligned
 *   dq         shaped like q; dk, dv shaped like k (bf16, written, rounded to
 *              nearest-even); no output may overlap an input or another output
 *   head_dim   128 or 64 (else ATTN_ERR_SHAPE)
 *   layout, B, H, Sq, Skv, scale, stream  as attn_fwd_bf16 (H: query heads)
 *   causal     0: every key; 1: the mask of attn_fwd_bf16_gqa (query i sees
 *              keys j <= i + Skv - Sq); lse must come from the forward with
 *              the same mask (-inf for rows that see no key, whose dQ is 0;
 *              keys no query sees get dK = dV = 0).  Other values:
 *              ATTN_ERR_OPTION.
 *
 * The accuracy of the gradients follows that of lse and o.  Errors as for
 * attn_fwd_bf16 (pointers 16-byte aligned, lse 4-byte aligned); the library's
 * workspace for (device, stream) holds delta.  Asynchronous on `stream`.
 */
int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv, int layout, int64_t B, int64_t H,
                  int64_t Hkv, int64_t Sq, int64_t Skv, int64_t head_dim, float scale, int causal,
                  void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* attn_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
