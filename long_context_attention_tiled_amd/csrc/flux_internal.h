// flux_internal.h -- argument blocks and launchers shared by the host layer
// (flux_api.cpp) and the gfx950 kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {

constexpr int kBlock = 64;  // block-sparse granularity and key-tile width
constexpr int kAbsmaxChunks = 128;  // backward: token chunks of the |x| maximum per (batch, KV head, tensor)

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;            // [B, Hq, S] or nullptr
    int64_t batch;
    int64_t seq;
    int hq;
    int hkv;
    int head_dim;
    float scale;           // softmax scale
    float scale_log2;      // scale * log2(e): scores enter exp2
    int causal;
    int sparse;
    int out_f32;
    int n_qblk;            // ceil(seq / 64)
    const int32_t* row_ptr;  // sparse CSR (device) or nullptr
    const int32_t* col_idx;
    const int32_t* mode_dev;  // device-resident mode of this layer (0 dense causal, else sparse),
                              // read by the kernel; nullptr when the mode is fixed by `sparse`
    int num_cu;               // compute units of the device (persistent grid size)
    const float* mix_w;       // soft routing: device [2] weights (w_FA, w_SA)
    float* soft_ws;           // fused soft routing: fp32 [B, S, Hq, d] scratch for the sparse output, or nullptr
    int sink_blocks;          // fused soft routing: the block-sparse pattern (sink and window in blocks)
    int window_blocks;
};

struct DecodeArgs {
    const void* q;         // [B, Hq, d] bf16
    const void* k;         // [B, cap, Hkv, d] bf16
    const void* v;
    void* o;               // [B, Hq, d]
    float* lse;            // [B, Hq] or nullptr
    float* part_o;         // workspace [B, Hq, n_split, d] fp32 (normalised partial outputs)
    float* part_lse;       // workspace [B, Hq, n_split] fp32 (natural log)
    int64_t batch;
    int64_t kv_len;
    int64_t kv_cap;
    int hq;
    int hkv;
    int head_dim;
    float scale;
    float scale_log2;
    int out_f32;
    // active key ranges: [0, r0_end) U [r1_begin, kv_len); n_active = r0_end + (kv_len - r1_begin)
    int64_t r0_end;
    int64_t r1_begin;
    int64_t n_active;
    int n_split;
    int64_t split_len;     // active keys per split (multiple of 64)
    // cache layout: ring == 0 -> token t at row t; ring == 1 (window cache) -> token t at row t when
    // t < sink_rows, else at row sink_rows + ((t / 64) % ring_blocks) * 64 + t % 64
    int ring;
    int64_t sink_rows;
    int ring_blocks;
    // token kv_len-1 [B, Hkv, d], stored into the cache by a launch that precedes the split kernel, or nullptr
    const void* k_new;
    const void* v_new;
};

constexpr int kMaxRouteLayers = 64;

struct RouteArgs {
    const void* xq[kMaxRouteLayers];
    int n_layers;
    int layer0;            // index of xq[0] in the stacked weight arrays
    int64_t seq;
    int n_feat;            // hq * head_dim
    int in_f32;
    int pool_tokens;
    const float* w_enc;
    const float* b_enc;
    int hidden;
    const float* w_head;
    const float* b_head;
    float* logits;         // nullable
    int32_t* modes;
    float* pooled;         // workspace [L_total, n_feat]
    float* z;              // workspace [L_total, hidden]
    int32_t* counters;     // workspace [L_total]: encoder workgroups done (reset by the pool kernel)
};

struct BackwardArgs {
    const void* q;         // [B, S, Hq, d] bf16
    const void* k;         // [B, S, Hkv, d] bf16
    const void* v;
    const void* o;         // [B, S, Hq, d] forward output, bf16 or fp32 (o_f32)
    const void* d_o;       // [B, S, Hq, d] bf16 output gradient
    const float* lse;      // [B, Hq, S] natural-log row sum-exp of the scaled scores
    float* dq;             // [B, S, Hq, d]
    float* dk;             // [B, S, Hkv, d]
    float* dv;
    float* dk_part;        // workspace [B, part_keys, Hq, d]: per-query-head dK of the sink keys (sparse GQA)
    float* dv_part;
    int64_t part_keys;     // keys held by dk_part / dv_part (the sink key pairs' keys), 0 if none
    float* stat;           // workspace [B, Hq, n_qblk, 2, 64]: -lse*log2(e), then rowsum(dO * O)
    int* counters;         // workspace [2]: work-queue heads of the dK/dV and dQ kernels
    // bf16 inputs: fp16 copies of Q, K, V, dO (same layouts) scaled by 2^-e per (batch, KV head) and
    // tensor, the largest magnitude of each group landing in [2^14, 2^15)
    void* q16;
    void* k16;
    void* v16;
    void* do16;
    uint32_t* amax;        // workspace [4][B * Hkv][kAbsmaxChunks]: partial maxima of |x| (bf16 bits)
    int* exps;             // workspace [4][B * Hkv]: e of Q, K, V, dO
    int64_t batch;
    int64_t seq;
    int hq;
    int hkv;
    int head_dim;
    float scale;
    float scale_log2;
    int causal;
    int sparse;
    int sink_blocks;
    int window_blocks;
    int n_qblk;            // ceil(seq / 64)
    int num_cu;            // persistent grid size
    int o_f32;
    int in_f32;            // q, k, v, d_o float32 (vector-ALU path) instead of bf16
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Bytes of the decode's fixed device scratch (the no-allocation decode entry point); the same value as
// FLUX_DECODE_SCRATCH_BYTES in flux_attn.h.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
// Device address of that scratch on the current device (looked up on the first call per device).
hipError_t decode_scratch(void** ptr);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_route_soft(const float* logits, const float* uniforms, float tau, int n_layers, float* weights,
                             hipStream_t s);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);
hipError_t launch_backward_f32(const BackwardArgs& a, hipStream_t s);

}  // namespace flux
