// router.hip -- the per-layer router of Flux Attention (aitrends.kr page, router
// paragraphs): prefix/suffix mean pooling of the layer's query tensor xQ over
// its first and last P tokens, an MLP context encoder (Linear + ReLU), a router
// head producing the two logits (pi_FA, pi_SA), and the inference-time argmax.
//
// Two small kernels over a caller-provided workspace, each spread over many CUs
// (the encoder weights, 4 MiB per layer at 32 heads x 128 and hidden 256, are the
// bulk of the bytes; the whole router is latency-bound):
//   pool    -- grid (layers, features/128), 1024 threads: 16 lanes cover 128
//              features of one token (8 each, one 16-byte load), the pooled tokens
//              are dealt to the 64 lane groups, so every lane has at most a few
//              loads in flight at once; the 64 partial sums per feature are added
//              in a fixed two-level order -> pooled [L, F].  It also resets the
//              layer's arrival counter for the encoder;
//   encoder -- grid (layers, hidden/4): one wave per hidden unit, 16-byte weight
//              loads, wave reduction, ReLU -> z [L, hidden]; the last workgroup of
//              a layer to finish (arrival counter) then runs the router head: both
//              logits and the argmax (a tie selects dense).  No launch for the head.
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kPoolThreads = 1024;
constexpr int kPoolFeat = 128;                    // features per pooling workgroup (16 lanes x 8)
constexpr int kPoolGroups = kPoolThreads / 16;    // token groups of 16 lanes
constexpr int kPoolParts = kPoolThreads / kPoolFeat;   // first-level partial sums per feature
constexpr int kEncThreads = 256;                  // 4 waves = 4 hidden units per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(kPoolThreads) void route_pool_kernel(RouteArgs a) {
    __shared__ float red[kPoolGroups][kPoolFeat];
    __shared__ float red2[kPoolParts][kPoolFeat];
    const int li = blockIdx.x;
    const int tg = threadIdx.x >> 4, sub = threadIdx.x & 15;
    const int64_t nf = a.n_feat;
    const int64_t f0 = (int64_t)blockIdx.y * kPoolFeat + sub * 8;   // this lane's 8 features
    const int64_t P = a.pool_tokens;
    const int64_t head_end = min<int64_t>(P, a.seq);
    const int64_t tail_begin = max<int64_t>(a.seq - P, head_end);   // token indices counted once
    const int64_t n_tok = head_end + (a.seq - tail_begin);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (f0 < nf) {
        // pooled token j (group-strided): j < head_end -> token j, else tail_begin + j - head_end
#pragma unroll 4
        for (int64_t j = tg; j < n_tok; j += kPoolGroups) {
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
    for (int e = 0; e < 8; ++e) red[tg][sub * 8 + e] = acc[e];
    if (blockIdx.y == 0 && threadIdx.x == 0) a.counters[a.layer0 + li] = 0;
    __syncthreads();
    // fixed-order sums (groups 8p .. 8p+7, then the 8 parts): the result does not depend on scheduling
    const int c = threadIdx.x % kPoolFeat, part = threadIdx.x / kPoolFeat;
    float s = 0.0f;
#pragma unroll
    for (int g = 0; g < kPoolGroups / kPoolParts; ++g) s += red[part * (kPoolGroups / kPoolParts) + g][c];
    red2[part][c] = s;
    __syncthreads();
    const int64_t f = (int64_t)blockIdx.y * kPoolFeat + threadIdx.x;
    if (threadIdx.x < kPoolFeat && f < nf) {
        float sum = 0.0f;
#pragma unroll
        for (int p = 0; p < kPoolParts; ++p) sum += red2[p][threadIdx.x];
        a.pooled[(int64_t)(a.layer0 + li) * nf + f] = sum / (float)n_tok;
    }
}

__global__ __launch_bounds__(kEncThreads) void route_encoder_kernel(RouteArgs a) {
    __shared__ int is_last;
    const int layer = a.layer0 + blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.y * (kEncThreads / 64) + (threadIdx.x >> 6);
    if (u < a.hidden) {
        const int nf4 = a.n_feat / 4;
        const float4* w = reinterpret_cast<const float4*>(a.w_enc + ((int64_t)layer * a.hidden + u) * a.n_feat);
        const float4* x = reinterpret_cast<const float4*>(a.pooled + (int64_t)layer * a.n_feat);
        float acc = 0.0f;
#pragma unroll 8
        for (int i = lane; i < nf4; i += 64) {
            const float4 wv = w[i], xv = x[i];
            acc = fmaf(wv.x, xv.x, acc);
            acc = fmaf(wv.y, xv.y, acc);
            acc = fmaf(wv.z, xv.z, acc);
            acc = fmaf(wv.w, xv.w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0)
            a.z[(int64_t)layer * a.hidden + u] = fmaxf(acc + a.b_enc[(int64_t)layer * a.hidden + u], 0.0f);
    }
    // release this workgroup's z, count it in; the last of the layer's workgroups runs the head
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(&a.counters[layer], 1) == (int)gridDim.y - 1;
    __syncthreads();
    if (!is_last || threadIdx.x >= 64) return;
    __threadfence();
    const float* z = a.z + (int64_t)layer * a.hidden;
    const float* wh = a.w_head + (int64_t)layer * 2 * a.hidden;
    float p0 = 0.0f, p1 = 0.0f;
    // (the acquire fence above invalidated this CU's cache: plain loads see every workgroup's z)
#pragma unroll 4
    for (int i = lane; i < a.hidden; i += 64) {
        const float zi = z[i];
        p0 = fmaf(wh[i], zi, p0);
        p1 = fmaf(wh[a.hidden + i], zi, p1);
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
                       dim3(kPoolThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_encoder_kernel, dim3(a.n_layers, (a.hidden + 3) / 4), dim3(kEncThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace flux
