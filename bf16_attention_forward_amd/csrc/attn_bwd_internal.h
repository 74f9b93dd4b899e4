// attn_bwd_internal.h -- parameters shared by the host and the backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_bwd {

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;    // forward output
    const uint16_t* dO;   // gradient of the output
    const float* lse;     // [B][H][Sq] forward log-sum-exp (natural log)
    float* delta;         // [B][H][Sq] workspace: -<dO_i, O_i> (negated: the dP products start from it)
    float* lse2;          // [B][H][Sq] workspace: lse * log2(e)
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int64_t q_row, q_head, q_batch;      // element strides of q, o, dO, dq
    int64_t kv_row, kv_head, kv_batch;   // element strides of k, v, dk, dv
    int B, H, Sq, Skv;    // H = query heads
    int Hkv;              // key/value heads (H a multiple of Hkv)
    int group;            // H / Hkv: query head h reads key/value head h / group
    int n_qblocks;        // ceil(Sq / 256): work-groups per (b, h) of the dQ kernel
    int n_kblocks;        // ceil(Skv / 128): work-groups per (b, key/value head) of the dK/dV kernel
    float c;              // fp32(scale * log2(e))
    float scale;
    int causal;           // 1: query i sees keys j <= i + causal_off (the forward's mask)
    int causal_off;       // Skv - Sq
    int head_dim;         // 128 or 64
};

int launch_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace attn_bwd
