// router.hip -- the per-layer router of Flux Attention (aitrends.kr page, router
// paragraphs): prefix/suffix mean pooling of the layer's query tensor xQ over
// its first and last P tokens, an MLP context encoder (Linear + ReLU), a router
// head producing the two logits (pi_FA, pi_SA), and the inference-time argmax.
//
// Three small kernels over a caller-provided workspace, each spread over the
// whole chip (the encoder weights, 4 MiB per layer at 32 heads x 128 and hidden
// 256, are the bulk of the bytes):
//   pool    -- grid (layers, features/256): a thread owns one feature and sums
//              the P + P pooled rows (coalesced across threads) -> pooled [L, F];
//   encoder -- grid (layers, hidden/4): one wave per hidden unit, 16-byte weight
//              loads, wave reduction, ReLU -> z [L, hidden];
//   head    -- one wave per layer: both logits, argmax (a tie selects dense).
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kEncThreads = 256;   // 4 waves = 4 hidden units per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(256) void route_pool_kernel(RouteArgs a) {
    const int li = blockIdx.x;
    const int f = blockIdx.y * kPoolThreads + threadIdx.x;
    if (f >= a.n_feat) return;
    const int64_t P = a.pool_tokens;
    const int64_t head_end = min<int64_t>(P, a.seq);
    const int64_t tail_begin = max<int64_t>(a.seq - P, head_end);   // token indices counted once
    const int64_t n_tok = head_end + (a.seq - tail_begin);
    const int64_t nf = a.n_feat;
    float acc = 0.0f;
    if (a.in_f32) {
        const float* x = reinterpret_cast<const float*>(a.xq[li]) + f;
        for (int64_t t = 0; t < head_end; ++t) acc += x[t * nf];
        for (int64_t t = tail_begin; t < a.seq; ++t) acc += x[t * nf];
    } else {
        const unsigned short* x = reinterpret_cast<const unsigned short*>(a.xq[li]) + f;
        for (int64_t t = 0; t < head_end; ++t) acc += __uint_as_float((unsigned)x[t * nf] << 16);
        for (int64_t t = tail_begin; t < a.seq; ++t) acc += __uint_as_float((unsigned)x[t * nf] << 16);
    }
    a.pooled[(int64_t)(a.layer0 + li) * nf + f] = acc / (float)n_tok;
}

__global__ __launch_bounds__(256) void route_encoder_kernel(RouteArgs a) {
    const int layer = a.layer0 + blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.y * (kEncThreads / 64) + (threadIdx.x >> 6);
    if (u >= a.hidden) return;
    const int nf4 = a.n_feat / 4;
    const float4* w = reinterpret_cast<const float4*>(a.w_enc + ((int64_t)layer * a.hidden + u) * a.n_feat);
    const float4* x = reinterpret_cast<const float4*>(a.pooled + (int64_t)layer * a.n_feat);
    float acc = 0.0f;
    for (int i = lane; i < nf4; i += 64) {
        const float4 wv = w[i], xv = x[i];
        acc = fmaf(wv.x, xv.x, acc);
        acc = fmaf(wv.y, xv.y, acc);
        acc = fmaf(wv.z, xv.z, acc);
        acc = fmaf(wv.w, xv.w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) a.z[(int64_t)layer * a.hidden + u] = fmaxf(acc + a.b_enc[(int64_t)layer * a.hidden + u], 0.0f);
}

__global__ __launch_bounds__(64) void route_head_kernel(RouteArgs a) {
    const int layer = a.layer0 + blockIdx.x;
    const int lane = threadIdx.x;
    const float* z = a.z + (int64_t)layer * a.hidden;
    const float* wh = a.w_head + (int64_t)layer * 2 * a.hidden;
    float p0 = 0.0f, p1 = 0.0f;
    for (int u = lane; u < a.hidden; u += 64) {
        p0 = fmaf(wh[u], z[u], p0);
        p1 = fmaf(wh[a.hidden + u], z[u], p1);
    }
    p0 = wave_sum(p0) + a.b_head[2 * layer];
    p1 = wave_sum(p1) + a.b_head[2 * layer + 1];
    if (lane == 0) {
        if (a.logits) {
            a.logits[2 * layer] = p0;
            a.logits[2 * layer + 1] = p1;
        }
        a.modes[layer] = p1 > p0 ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(route_pool_kernel, dim3(a.n_layers, (a.n_feat + kPoolThreads - 1) / kPoolThreads),
                       dim3(kPoolThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_encoder_kernel, dim3(a.n_layers, (a.hidden + 3) / 4), dim3(kEncThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_head_kernel, dim3(a.n_layers), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace flux
