// router.hip -- the per-layer router of Flux Attention (aitrends.kr page, router
// paragraphs): prefix/suffix mean pooling of the layer's query tensor xQ over
// its first and last P tokens, an MLP context encoder (Linear + ReLU), a router
// head producing the two logits (pi_FA, pi_SA), and the inference-time argmax.
//
// Three small kernels over a caller-provided workspace, each spread over the
// whole chip (the encoder weights, 4 MiB per layer at 32 heads x 128 and hidden
// 256, are the bulk of the bytes):
//   pool    -- grid (layers, features/512), 16 waves: a lane owns 8 features (one
//              16-byte load per token), the pooled tokens are dealt to the waves and
//              the 16 partial sums are added in a fixed order -> pooled [L, F];
//   encoder -- grid (layers, hidden/4): one wave per hidden unit, 16-byte weight
//              loads, wave reduction, ReLU -> z [L, hidden];
//   head    -- one wave per layer: both logits, argmax (a tie selects dense).
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kPoolWaves = 16;     // pooled tokens are dealt to 16 waves
constexpr int kPoolFeat = 512;     // features per pooling workgroup (64 lanes x 8)
constexpr int kEncThreads = 256;   // 4 waves = 4 hidden units per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(kPoolWaves * 64) void route_pool_kernel(RouteArgs a) {
    __shared__ float red[kPoolWaves][kPoolFeat];
    const int li = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nf = a.n_feat;
    const int64_t f0 = (int64_t)blockIdx.y * kPoolFeat + lane * 8;   // this lane's 8 features
    const int64_t P = a.pool_tokens;
    const int64_t head_end = min<int64_t>(P, a.seq);
    const int64_t tail_begin = max<int64_t>(a.seq - P, head_end);   // token indices counted once
    const int64_t n_tok = head_end + (a.seq - tail_begin);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (f0 < nf) {
        // pooled token j (wave-strided): j < head_end -> token j, else tail_begin + j - head_end
#pragma unroll 4
        for (int64_t j = wave; j < n_tok; j += kPoolWaves) {
            const int64_t t = j < head_end ? j : tail_begin + (j - head_end);
            if (a.in_f32) {
                const float4* x = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.xq[li]) + t * nf + f0);
                const float4 u0 = x[0], u1 = x[1];
                acc[0] += u0.x; acc[1] += u0.y; acc[2] += u0.z; acc[3] += u0.w;
                acc[4] += u1.x; acc[5] += u1.y; acc[6] += u1.z; acc[7] += u1.w;
            } else {
                const uint4 u = *reinterpret_cast<const uint4*>(
                    reinterpret_cast<const unsigned short*>(a.xq[li]) + t * nf + f0);
                const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += __uint_as_float(w[e] << 16);
                    acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
    __syncthreads();
    // fixed-order sum over the waves: the result does not depend on scheduling
    const int c = threadIdx.x;
    const int64_t f = (int64_t)blockIdx.y * kPoolFeat + c;
    if (c < kPoolFeat && f < nf) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kPoolWaves; ++w) sum += red[w][c];
        a.pooled[(int64_t)(a.layer0 + li) * nf + f] = sum / (float)n_tok;
    }
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
#pragma unroll 4
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

// Gumbel-softmax routing weights (the training-time relaxation of the router head, router
// paragraph of the Flux Attention page): w = softmax((pi + g) / tau), g = -ln(-ln u).
__global__ __launch_bounds__(64) void route_soft_kernel(const float* logits, const float* uniforms, float tau,
                                                        int n_layers, float* weights) {
    const int l = blockIdx.x * 64 + threadIdx.x;
    if (l >= n_layers) return;
    const float x0 = (logits[2 * l] - logf(-logf(uniforms[2 * l]))) / tau;
    const float x1 = (logits[2 * l + 1] - logf(-logf(uniforms[2 * l + 1]))) / tau;
    const float m = fmaxf(x0, x1);
    const float e0 = expf(x0 - m), e1 = expf(x1 - m);
    const float inv = 1.0f / (e0 + e1);
    weights[2 * l] = e0 * inv;
    weights[2 * l + 1] = e1 * inv;
}

}  // namespace

hipError_t launch_route_soft(const float* logits, const float* uniforms, float tau, int n_layers, float* weights,
                             hipStream_t s) {
    hipLaunchKernelGGL(route_soft_kernel, dim3((n_layers + 63) / 64), dim3(64), 0, s, logits, uniforms, tau, n_layers,
                       weights);
    return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(route_pool_kernel, dim3(a.n_layers, (a.n_feat + kPoolFeat - 1) / kPoolFeat),
                       dim3(kPoolWaves * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_encoder_kernel, dim3(a.n_layers, (a.hidden + 3) / 4), dim3(kEncThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_head_kernel, dim3(a.n_layers), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace flux
