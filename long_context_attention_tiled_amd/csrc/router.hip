// router.hip -- the per-layer router of Flux Attention (aitrends.kr page, router
// paragraphs): prefix/suffix mean pooling of the layer's query tensor xQ over
// its first and last P tokens, an MLP context encoder (Linear + ReLU), a router
// head producing the two logits (pi_FA, pi_SA), and the inference-time argmax.
//
// One workgroup of 1024 threads per layer; everything stays on chip:
//   pooling -- threads own features (coalesced rows of xQ), sum the P + P rows,
//              result in LDS;
//   encoder -- 16 waves, one hidden unit per wave at a time, 16-byte weight
//              loads, wave reduction;
//   head    -- one wave computes both logits and the argmax (a tie selects the
//              dense mode).
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxFeat = 8192;
constexpr int kMaxHidden = 1024;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(1024) void route_kernel(RouteArgs a) {
    __shared__ __attribute__((aligned(16))) float pooled[kMaxFeat];
    __shared__ float z[kMaxHidden];
    const int li = blockIdx.x;
    const int layer = a.layer0 + li;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nf = a.n_feat;
    const int64_t P = a.pool_tokens;

    // token index set [0, P) U [seq-P, seq), each index once
    const int64_t head_end = min<int64_t>(P, a.seq);
    const int64_t tail_begin = max<int64_t>(a.seq - P, head_end);
    const int64_t n_tok = head_end + (a.seq - tail_begin);
    const float inv_n = 1.0f / (float)n_tok;
    for (int f = tid; f < nf; f += kThreads) {
        float acc = 0.0f;
        if (a.in_f32) {
            const float* x = reinterpret_cast<const float*>(a.xq[li]);
            for (int64_t t = 0; t < head_end; ++t) acc += x[t * nf + f];
            for (int64_t t = tail_begin; t < a.seq; ++t) acc += x[t * nf + f];
        } else {
            const unsigned short* x = reinterpret_cast<const unsigned short*>(a.xq[li]);
            for (int64_t t = 0; t < head_end; ++t) acc += __uint_as_float((unsigned)x[t * nf + f] << 16);
            for (int64_t t = tail_begin; t < a.seq; ++t) acc += __uint_as_float((unsigned)x[t * nf + f] << 16);
        }
        pooled[f] = acc * inv_n;
    }
    __syncthreads();

    const float* we = a.w_enc + (int64_t)layer * a.hidden * nf;
    for (int u = wave; u < a.hidden; u += kThreads / 64) {
        const float4* wrow = reinterpret_cast<const float4*>(we + (int64_t)u * nf);
        float acc = 0.0f;
        for (int f4 = lane; f4 < nf / 4; f4 += 64) {
            const float4 w = wrow[f4];
            const float4 x = *reinterpret_cast<const float4*>(&pooled[4 * f4]);
            acc = fmaf(w.x, x.x, acc);
            acc = fmaf(w.y, x.y, acc);
            acc = fmaf(w.z, x.z, acc);
            acc = fmaf(w.w, x.w, acc);
        }
        acc = wave_sum(acc) + a.b_enc[(int64_t)layer * a.hidden + u];
        if (lane == 0) z[u] = fmaxf(acc, 0.0f);
    }
    __syncthreads();

    if (wave == 0) {
        float p0 = 0.0f, p1 = 0.0f;
        const float* wh = a.w_head + (int64_t)layer * 2 * a.hidden;
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
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(route_kernel, dim3(a.n_layers), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace flux
