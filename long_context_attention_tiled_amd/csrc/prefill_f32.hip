// prefill_f32.hip -- tiled attention prefill with float32 inputs and outputs.
//
// Same computation and masks as the bf16 kernel (online softmax over 64-key
// tiles, only CSR-listed key blocks visited in sparse mode), but on the vector
// ALUs: float32 has no dense-contraction fast path worth the complexity at the
// small shapes this precision is used for.  One workgroup = one 64-row query
// block of one (batch, head); four lanes share a query row, each owning a
// quarter of the head dimension.  K and V tiles are staged in LDS.
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
    constexpr int DQ = D / 4;          // dims per lane
    constexpr int KS = D + 4;          // LDS row stride (floats)
    __shared__ __attribute__((aligned(16))) float ks[kTile * KS];
    __shared__ __attribute__((aligned(16))) float vs[kTile * KS];

    const int tid = threadIdx.x;
    const int qb = blockIdx.x % a.n_qblk;
    const int bh = blockIdx.x / a.n_qblk;
    const int h = bh % a.hq;
    const int b = bh / a.hq;
    const int g = h / (a.hq / a.hkv);
    const int qi = tid >> 2, part = tid & 3;
    const int64_t qpos = (int64_t)qb * kTile + qi;

    const float* qg = reinterpret_cast<const float*>(a.q);
    const float* kg = reinterpret_cast<const float*>(a.k) + ((int64_t)b * a.seq * a.hkv + g) * D;
    const float* vg = reinterpret_cast<const float*>(a.v) + ((int64_t)b * a.seq * a.hkv + g) * D;
    const int64_t kv_stride = (int64_t)a.hkv * D;

    float qv[DQ], o[DQ];
#pragma unroll
    for (int t = 0; t < DQ; ++t) {
        qv[t] = qpos < a.seq ? qg[(((int64_t)b * a.seq + qpos) * a.hq + h) * D + part * DQ + t] : 0.0f;
        o[t] = 0.0f;
    }
    float m_run = kNegBig, l_run = 0.0f;
    const float c2 = a.scale_log2;

    const bool sparse = a.mode_dev ? a.mode_dev[0] != 0 : a.sparse != 0;
    // key blocks of query block qb: the CSR row when one is given; else (and in dense mode) position p
    // of the walk is block p, except that a sparse walk jumps from the end of the sink blocks to the
    // first block of the window (the same blocks the CSR lists)
    const bool csr = sparse && a.row_ptr;
    int p = 0, e = 0, sink_end = 0, win_lo = 0;
    if (csr) {
        p = a.row_ptr[qb];
        e = a.row_ptr[qb + 1];
    } else {
        e = (a.causal || sparse) ? qb + 1 : a.n_qblk;
        sink_end = sparse ? min(a.sink_blocks, qb + 1) : e;
        win_lo = sparse ? max(sink_end, qb - a.window_blocks + 1) : e;
    }
    for (; p < e; ++p) {
        if (!csr && p == sink_end && win_lo > p) p = win_lo;
        const int kb = csr ? a.col_idx[p] : p;
        __syncthreads();
        for (int idx = tid; idx < kTile * D / 4; idx += kThreads) {
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int64_t key = (int64_t)kb * kTile + row;
            float4 kx = make_float4(0, 0, 0, 0), vx = make_float4(0, 0, 0, 0);
            if ((uint64_t)key < (uint64_t)a.seq) {
                kx = *reinterpret_cast<const float4*>(kg + key * kv_stride + 4 * c4);
                vx = *reinterpret_cast<const float4*>(vg + key * kv_stride + 4 * c4);
            }
            *reinterpret_cast<float4*>(ks + row * KS + 4 * c4) = kx;
            *reinterpret_cast<float4*>(vs + row * KS + 4 * c4) = vx;
        }
        __syncthreads();
        float s[kTile];
        float mx = -INFINITY;
#pragma unroll
        for (int jk = 0; jk < kTile; ++jk) {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < DQ; ++t) acc = fmaf(qv[t], ks[jk * KS + part * DQ + t], acc);
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            const int64_t key = (int64_t)kb * kTile + jk;
            const bool off = key >= a.seq || ((a.causal || sparse) && key > qpos);
            s[jk] = off ? -INFINITY : acc;
            mx = fmaxf(mx, s[jk]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
        const float mc = m_new * c2;
        float rs = 0.0f;
#pragma unroll
        for (int t = 0; t < DQ; ++t) o[t] *= alpha;
#pragma unroll
        for (int jk = 0; jk < kTile; ++jk) {
            const float pj = __builtin_amdgcn_exp2f(fmaf(s[jk], c2, -mc));
            rs += pj;
#pragma unroll
            for (int t = 0; t < DQ; ++t) o[t] = fmaf(pj, vs[jk * KS + part * DQ + t], o[t]);
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
    }
    if (qpos >= a.seq) return;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* og = reinterpret_cast<float*>(a.o) + (((int64_t)b * a.seq + qpos) * a.hq + h) * D + part * DQ;
#pragma unroll
    for (int t = 0; t < DQ; ++t) og[t] = o[t] * inv;
    if (a.lse && part == 0)
        a.lse[((int64_t)b * a.hq + h) * a.seq + qpos] =
            l_run > 0.0f ? (m_run * c2 + __log2f(l_run)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    const int64_t grid = a.batch * a.hq * a.n_qblk;
    if (a.head_dim == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else if (a.head_dim == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace flux
