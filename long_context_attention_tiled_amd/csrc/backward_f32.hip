// backward_f32.hip -- gradients of tiled attention with float32 inputs (dQ, dK, dV in fp32).
//
// The same chain rule as the bf16 path (dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
// dV = P^T dO, P rebuilt from Q, K and the row LSE), on the vector ALUs like the fp32 forward kernel:
// fp32 is the precision of small layers, where a dense-contraction path is not worth its
// complexity.  The row statistics come from bwd_rowstat_kernel (backward.hip).
//   bwd_f32_dq_kernel    one workgroup = 64 query rows of one (batch, query head); four lanes share a
//                        row, each a quarter of the head dimension; the visible 64-key tiles of K and
//                        V are staged in LDS.
//   bwd_f32_dkdv_kernel  one workgroup = 64 keys of one (batch, KV head); four lanes per key; walks
//                        the query heads of the group and, for each, the 64-query tiles that see the
//                        block (Q, dO and the rows' statistics staged in LDS).  The group's heads are
//                        summed in head order inside the workgroup, so no per-head buffers are needed.
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

// visible for query block qb and key block kb (causal / all keys / sink + window)
__device__ __forceinline__ bool block_visible(const BackwardArgs& a, int qb, int kb) {
    if (!a.causal) return true;
    if (kb > qb) return false;
    return !a.sparse || kb < a.sink_blocks || qb - kb < a.window_blocks;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_f32_dq_kernel(BackwardArgs a) {
    constexpr int DQ = D / 4;          // dims per lane
    constexpr int KS = D + 4;          // LDS row stride (floats)
    __shared__ __attribute__((aligned(16))) float ks[kTile * KS];
    __shared__ __attribute__((aligned(16))) float vs[kTile * KS];

    const int tid = threadIdx.x;
    const int qb = blockIdx.x % a.n_qblk;
    const int bh = blockIdx.x / a.n_qblk;
    const int h = bh % a.hq, b = bh / a.hq;
    const int g = h / (a.hq / a.hkv);
    const int qi = tid >> 2, part = tid & 3;
    const int64_t qpos = (int64_t)qb * kTile + qi;
    const bool live = qpos < a.seq;

    const float* kg = reinterpret_cast<const float*>(a.k) + ((int64_t)b * a.seq * a.hkv + g) * D;
    const float* vg = reinterpret_cast<const float*>(a.v) + ((int64_t)b * a.seq * a.hkv + g) * D;
    const int64_t kv_stride = (int64_t)a.hkv * D;
    const int64_t qoff = (((int64_t)b * a.seq + qpos) * a.hq + h) * D + part * DQ;

    float qv[DQ], gv[DQ], dq[DQ];
#pragma unroll
    for (int t = 0; t < DQ; ++t) {
        qv[t] = live ? reinterpret_cast<const float*>(a.q)[qoff + t] : 0.0f;
        gv[t] = live ? reinterpret_cast<const float*>(a.d_o)[qoff + t] : 0.0f;
        dq[t] = 0.0f;
    }
    const float* st = a.stat + (((int64_t)b * a.hq + h) * a.n_qblk + qb) * 128;
    const float nl = st[qi];          // -LSE * log2(e); -inf for rows past the end
    const float drow = st[64 + qi];   // rowsum(dO * O)
    const float c2 = a.scale_log2;

    for (int kb = 0; kb < a.n_qblk; ++kb) {
        if (!block_visible(a, qb, kb)) continue;   // uniform over the workgroup
        __syncthreads();
        for (int idx = tid; idx < kTile * D / 4; idx += kThreads) {
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int64_t key = (int64_t)kb * kTile + row;
            float4 kx = make_float4(0, 0, 0, 0), vx = make_float4(0, 0, 0, 0);
            if (key < a.seq) {
                kx = *reinterpret_cast<const float4*>(kg + key * kv_stride + 4 * c4);
                vx = *reinterpret_cast<const float4*>(vg + key * kv_stride + 4 * c4);
            }
            *reinterpret_cast<float4*>(ks + row * KS + 4 * c4) = kx;
            *reinterpret_cast<float4*>(vs + row * KS + 4 * c4) = vx;
        }
        __syncthreads();
        for (int jk = 0; jk < kTile; ++jk) {
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int t = 0; t < DQ; ++t) {
                s = fmaf(qv[t], ks[jk * KS + part * DQ + t], s);
                dp = fmaf(gv[t], vs[jk * KS + part * DQ + t], dp);
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            dp += __shfl_xor(dp, 1);
            dp += __shfl_xor(dp, 2);
            const int64_t key = (int64_t)kb * kTile + jk;
            const bool off = key >= a.seq || (a.causal && key > qpos);
            const float p = off ? 0.0f : __builtin_amdgcn_exp2f(fmaf(s, c2, nl));
            const float ds = p * (dp - drow);
#pragma unroll
            for (int t = 0; t < DQ; ++t) dq[t] = fmaf(ds, ks[jk * KS + part * DQ + t], dq[t]);
        }
    }
    if (!live) return;
    float* out = a.dq + qoff;
#pragma unroll
    for (int t = 0; t < DQ; ++t) out[t] = a.scale * dq[t];
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_f32_dkdv_kernel(BackwardArgs a) {
    constexpr int DQ = D / 4;
    constexpr int KS = D + 4;
    __shared__ __attribute__((aligned(16))) float qs[kTile * KS];
    __shared__ __attribute__((aligned(16))) float gs[kTile * KS];
    __shared__ float nls[kTile], drs[kTile];

    const int tid = threadIdx.x;
    const int kb = blockIdx.x % a.n_qblk;
    const int bg = blockIdx.x / a.n_qblk;
    const int g = bg % a.hkv, b = bg / a.hkv;
    const int G = a.hq / a.hkv;
    const int kj = tid >> 2, part = tid & 3;
    const int64_t key = (int64_t)kb * kTile + kj;
    const bool live = key < a.seq;
    const int64_t kvoff = (((int64_t)b * a.seq + key) * a.hkv + g) * D + part * DQ;
    const int64_t q_stride = (int64_t)a.hq * D;

    float kv_[DQ], vv[DQ], dk[DQ], dv[DQ];
#pragma unroll
    for (int t = 0; t < DQ; ++t) {
        kv_[t] = live ? reinterpret_cast<const float*>(a.k)[kvoff + t] : 0.0f;
        vv[t] = live ? reinterpret_cast<const float*>(a.v)[kvoff + t] : 0.0f;
        dk[t] = 0.0f;
        dv[t] = 0.0f;
    }
    const float c2 = a.scale_log2;

    for (int j = 0; j < G; ++j) {   // query heads of the group, in head order
        const int h = g * G + j;
        const float* qg = reinterpret_cast<const float*>(a.q) + ((int64_t)b * a.seq * a.hq + h) * D;
        const float* dog = reinterpret_cast<const float*>(a.d_o) + ((int64_t)b * a.seq * a.hq + h) * D;
        const float* stg = a.stat + ((int64_t)b * a.hq + h) * a.n_qblk * 128;
        for (int qbb = a.causal ? kb : 0; qbb < a.n_qblk; ++qbb) {
            if (!block_visible(a, qbb, kb)) continue;   // uniform over the workgroup
            __syncthreads();
            for (int idx = tid; idx < kTile * D / 4; idx += kThreads) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                const int64_t q = (int64_t)qbb * kTile + row;
                float4 qx = make_float4(0, 0, 0, 0), gx = make_float4(0, 0, 0, 0);
                if (q < a.seq) {
                    qx = *reinterpret_cast<const float4*>(qg + q * q_stride + 4 * c4);
                    gx = *reinterpret_cast<const float4*>(dog + q * q_stride + 4 * c4);
                }
                *reinterpret_cast<float4*>(qs + row * KS + 4 * c4) = qx;
                *reinterpret_cast<float4*>(gs + row * KS + 4 * c4) = gx;
            }
            if (tid < kTile) {
                nls[tid] = stg[qbb * 128 + tid];        // -inf past the end: P = 0 there
                drs[tid] = stg[qbb * 128 + 64 + tid];
            }
            __syncthreads();
            for (int iq = 0; iq < kTile; ++iq) {
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int t = 0; t < DQ; ++t) {
                    s = fmaf(qs[iq * KS + part * DQ + t], kv_[t], s);
                    dp = fmaf(gs[iq * KS + part * DQ + t], vv[t], dp);
                }
                s += __shfl_xor(s, 1);
                s += __shfl_xor(s, 2);
                dp += __shfl_xor(dp, 1);
                dp += __shfl_xor(dp, 2);
                const int64_t q = (int64_t)qbb * kTile + iq;
                const bool off = a.causal && key > q;
                const float p = off ? 0.0f : __builtin_amdgcn_exp2f(fmaf(s, c2, nls[iq]));
                const float ds = p * (dp - drs[iq]);
#pragma unroll
                for (int t = 0; t < DQ; ++t) {
                    dv[t] = fmaf(p, gs[iq * KS + part * DQ + t], dv[t]);
                    dk[t] = fmaf(ds, qs[iq * KS + part * DQ + t], dk[t]);
                }
            }
        }
    }
    if (!live) return;
#pragma unroll
    for (int t = 0; t < DQ; ++t) {
        a.dk[kvoff + t] = a.scale * dk[t];
        a.dv[kvoff + t] = dv[t];
    }
}

}  // namespace

hipError_t launch_backward_f32(const BackwardArgs& a, hipStream_t s) {
    const unsigned grid_q = (unsigned)(a.batch * a.hq * a.n_qblk);
    const unsigned grid_kv = (unsigned)(a.batch * a.hkv * a.n_qblk);
    if (a.head_dim == 128) {
        hipLaunchKernelGGL(bwd_f32_dq_kernel<128>, dim3(grid_q), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(bwd_f32_dkdv_kernel<128>, dim3(grid_kv), dim3(kThreads), 0, s, a);
    } else if (a.head_dim == 64) {
        hipLaunchKernelGGL(bwd_f32_dq_kernel<64>, dim3(grid_q), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(bwd_f32_dkdv_kernel<64>, dim3(grid_kv), dim3(kThreads), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace flux
