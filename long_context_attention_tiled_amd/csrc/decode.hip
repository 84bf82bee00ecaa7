// decode.hip -- single-token GQA decode: split-KV partials + log-sum-exp merge.
//
// One new query per sequence attends to its KV cache.  Decode is bound by HBM
// bandwidth (each cached K/V element is read once and used for G = hq/hkv
// query heads), so the kernel is organised for streaming, not for matrix
// cores: 16-byte coalesced loads, many workgroups in flight, and the
// arithmetic kept on the vector ALUs (bf16 dot2 for q.k, fp32 FMA for p.v).
//
// Split kernel: workgroup = (split, kv head g, batch b), 256 threads.  The
// active keys (dense: all; sparse: sink blocks + window blocks of the query's
// row, the Flux Attention page's KV bypass) are numbered 0..n_active-1 and cut
// into equal 64-aligned chunks; a workgroup walks its chunk 64 keys at a time:
//   scores:   4 lanes per key, each a quarter of the row's 16-byte chunks,
//             dot2 against the G query rows held in registers, quad reduce;
//   softmax:  one wave per query head updates its running max/sum over the 64
//             scores (online softmax of the openads.co.kr newsletter);
//   P.V:      16 (or 32) key slots x 16-byte d chunks; accumulators rescaled by
//             exp(m_old - m_new) per head.
// The chunk's partial (O_s normalised, lse_s natural log) goes to the workspace.
// Combine kernel: LSE = M + ln sum_s exp(lse_s - M), O = sum_s exp(lse_s - LSE) O_s.
#include "flux_internal.h"

#include <mutex>

namespace flux {
namespace {

// Scratch of the no-allocation decode entry point (flux_attn_decode_noalloc): the split partials
// live here instead of in a caller workspace.  One copy per device, held until the process ends.
// Host code never passes this name to a kernel (on the host it is only a stand-in for the symbol);
// it passes the device address decode_scratch() looks up.
static __device__ __align__(256) __attribute__((used)) char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kThreads = 256;
constexpr int kSub = 64;  // keys per step
constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float dot8(uint4 k, uint4 q, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x), __builtin_bit_cast(bf16x2, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y), __builtin_bit_cast(bf16x2, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z), __builtin_bit_cast(bf16x2, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w), __builtin_bit_cast(bf16x2, q.w), acc, false);
    return acc;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// token position of active key idx
__device__ __forceinline__ int64_t token_of(const DecodeArgs& a, int64_t idx) {
    return idx < a.r0_end ? idx : a.r1_begin + (idx - a.r0_end);
}
// cache row holding token t (RING: window-cache layout)
template <bool RING>
__device__ __forceinline__ int64_t row_of(const DecodeArgs& a, int64_t t) {
    if (!RING || t < a.sink_rows) return t;
    const int slot = (int)(t >> 6) % a.ring_blocks;   // t < 2^37, so the block index fits 32 bits
    return a.sink_rows + (int64_t)slot * 64 + (t & 63);
}

template <int D, int G, bool RING>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    constexpr int KCH = D / 8;            // 16-byte chunks per K/V row
    constexpr int KPL = KCH / 4;          // chunks per lane in the score step
    constexpr int DSLOTS = KCH;           // d-chunk owners in the P.V step
    constexpr int KSLOTS = kThreads / DSLOTS;
    constexpr int KPS = kSub / KSLOTS;    // keys per thread in the P.V step
    constexpr int HPW = (G + 3) / 4;      // heads per wave in the softmax step

    __shared__ float s_p[2][kSub][G];
    __shared__ float s_alpha[2][G];
    __shared__ float s_ml[G][2];
    __shared__ float s_red[4][G][D];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t a0 = (int64_t)split * a.split_len;
    const int64_t a1 = min(a0 + a.split_len, a.n_active);
    const int64_t row_stride = (int64_t)a.hkv * D;
    const u16* kg = reinterpret_cast<const u16*>(a.k) + ((int64_t)b * a.kv_cap * a.hkv + g) * D;
    const u16* vg = reinterpret_cast<const u16*>(a.v) + ((int64_t)b * a.kv_cap * a.hkv + g) * D;
    const int h0 = g * G;

    // score-step mapping: key = tid/4, lane part = tid%4 owns chunks part + 4i
    const int sk = tid >> 2, part = tid & 3;
    uint4 qreg[G][KPL];
    const u16* qg = reinterpret_cast<const u16*>(a.q) + ((int64_t)b * a.hq + h0) * D;
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
        for (int i = 0; i < KPL; ++i) qreg[hq][i] = *reinterpret_cast<const uint4*>(qg + hq * D + (part + 4 * i) * 8);

    // P.V mapping: d chunk = tid % DSLOTS, key slot = tid / DSLOTS
    const int dch = tid % DSLOTS, kslot = tid / DSLOTS;
    float o[G][8];
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hq][e] = 0.0f;
    float m_run[HPW], l_run[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        m_run[i] = kNegBig;
        l_run[i] = 0.0f;
    }
    const float c2 = a.scale_log2;

    // K and V of a 64-key step are loaded into registers one step ahead, so that a step's
    // arithmetic overlaps the next step's HBM reads.
    uint4 kcur[KPL], vcur[KPS];
    // A 64-key step never straddles a 64-token block (split starts, the end of the sink range and the
    // start of the window range are all multiples of 64), so its keys sit in consecutive cache rows
    // from a per-step base row.
    auto load_step = [&](int64_t t0, uint4* kr, uint4* vr) {
        const int64_t base = row_of<RING>(a, token_of(a, t0));   // uniform
        const int64_t kidx = min(t0 + sk, a1 - 1);
        const u16* krow = kg + (base + (kidx - t0)) * row_stride;
#pragma unroll
        for (int i = 0; i < KPL; ++i) kr[i] = *reinterpret_cast<const uint4*>(krow + (part + 4 * i) * 8);
#pragma unroll
        for (int i = 0; i < KPS; ++i) {
            const int64_t idx = min(t0 + kslot + i * KSLOTS, a1 - 1);
            vr[i] = *reinterpret_cast<const uint4*>(vg + (base + (idx - t0)) * row_stride + dch * 8);
        }
    };
    if (a0 < a1) load_step(a0, kcur, vcur);

    int buf = 0;
    for (int64_t t0 = a0; t0 < a1; t0 += kSub, buf ^= 1) {
        uint4 knext[KPL], vnext[KPS];
        if (t0 + kSub < a1) load_step(t0 + kSub, knext, vnext);
        uint4 vreg[KPS];
#pragma unroll
        for (int i = 0; i < KPS; ++i) {
            // keys past the chunk end are clamped to its last key above; their V is zeroed here
            vreg[i] = t0 + kslot + i * KSLOTS < a1 ? vcur[i] : make_uint4(0, 0, 0, 0);
        }
        {
            const int64_t idx = t0 + sk;
            const bool valid = idx < a1;
            float sc[G];
#pragma unroll
            for (int hq = 0; hq < G; ++hq) sc[hq] = 0.0f;
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
#pragma unroll
                for (int hq = 0; hq < G; ++hq) sc[hq] = dot8(kcur[i], qreg[hq][i], sc[hq]);
            }
#pragma unroll
            for (int hq = 0; hq < G; ++hq) {
                sc[hq] += __shfl_xor(sc[hq], 1);
                sc[hq] += __shfl_xor(sc[hq], 2);
            }
            if (part == 0) {
#pragma unroll
                for (int hq = 0; hq < G; ++hq) s_p[buf][sk][hq] = valid ? sc[hq] : -INFINITY;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int hq = wave + 4 * i;
            if (hq < G) {
                const float x = s_p[buf][lane][hq];
                const float m_new = fmaxf(m_run[i], wave_max(x));
                const float alpha = __builtin_amdgcn_exp2f((m_run[i] - m_new) * c2);
                const float p = __builtin_amdgcn_exp2f(fmaf(x, c2, -m_new * c2));
                l_run[i] = l_run[i] * alpha + wave_sum(p);
                m_run[i] = m_new;
                s_p[buf][lane][hq] = p;
                if (lane == 0) s_alpha[buf][hq] = alpha;
            }
        }
        __syncthreads();
#pragma unroll
        for (int hq = 0; hq < G; ++hq) {
            const float al = s_alpha[buf][hq];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[hq][e] *= al;
        }
#pragma unroll
        for (int i = 0; i < KPS; ++i) {
            const int kk = kslot + i * KSLOTS;
            const uint4 vx = vreg[i];
            const float vf[8] = {bf_lo(vx.x), bf_hi(vx.x), bf_lo(vx.y), bf_hi(vx.y),
                                 bf_lo(vx.z), bf_hi(vx.z), bf_lo(vx.w), bf_hi(vx.w)};
#pragma unroll
            for (int hq = 0; hq < G; ++hq) {
                const float p = s_p[buf][kk][hq];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hq][e] = fmaf(p, vf[e], o[hq][e]);
            }
        }
        if (t0 + kSub < a1) {
#pragma unroll
            for (int i = 0; i < KPL; ++i) kcur[i] = knext[i];
#pragma unroll
            for (int i = 0; i < KPS; ++i) vcur[i] = vnext[i];
        }
    }

    // reduce o over key slots: slots inside a wave differ by lane / DSLOTS
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[hq][e];
#pragma unroll
            for (int off = DSLOTS; off < 64; off <<= 1) x += __shfl_xor(x, off);
            o[hq][e] = x;
        }
    if (lane < DSLOTS) {
#pragma unroll
        for (int hq = 0; hq < G; ++hq)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_red[wave][hq][dch * 8 + e] = o[hq][e];
    }
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int hq = wave + 4 * i;
        if (hq < G && lane == 0) {
            s_ml[hq][0] = m_run[i];
            s_ml[hq][1] = l_run[i];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int hq = idx / D, d = idx % D;
        const float l = s_ml[hq][1];
        const float sum = s_red[0][hq][d] + s_red[1][hq][d] + s_red[2][hq][d] + s_red[3][hq][d];
        const int64_t row = ((int64_t)b * a.hq + h0 + hq) * a.n_split + split;
        a.part_o[row * D + d] = l > 0.0f ? sum / l : 0.0f;
        if (d == 0) a.part_lse[row] = l > 0.0f ? (s_ml[hq][0] * c2 + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// Stores the new token (position kv_len-1) of every (batch, kv head) into the cache: grid (hkv, B),
// one 16-byte chunk of K or V per thread.  Runs before the split kernel on the same stream.
template <int D, bool RING>
__global__ __launch_bounds__(D / 4) void decode_append_kernel(DecodeArgs a) {
    constexpr int KCH = D / 8;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const bool is_v = tid >= KCH;
    const int c = tid % KCH;
    const int64_t row = row_of<RING>(a, a.kv_len - 1);
    const u16* src = reinterpret_cast<const u16*>(is_v ? a.v_new : a.k_new) + ((int64_t)b * a.hkv + g) * D + c * 8;
    u16* dst = reinterpret_cast<u16*>(const_cast<void*>(is_v ? a.v : a.k)) +
               (((int64_t)b * a.kv_cap + row) * a.hkv + g) * D + c * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// LSE combine of one (batch, query head) row over its splits.  The splits are read in batches of 8
// independent loads and summed in ascending split order: a loop of single loads would wait one memory
// round trip per split (32 of them for a full-cache decode).
constexpr int kCombineBatch = 8;
template <int D, bool OUT_F32>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    const int64_t row = blockIdx.x;  // b * hq + h
    const float* pl = a.part_lse + row * a.n_split;
    const int ns = a.n_split;
    auto weight = [](float l, float mx) { return l == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((l - mx) * kLog2e); };
    float mx = -INFINITY;
    int s = 0;
    for (; s + kCombineBatch <= ns; s += kCombineBatch) {
        float x[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) x[i] = pl[s + i];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) mx = fmaxf(mx, x[i]);
    }
    for (; s < ns; ++s) mx = fmaxf(mx, pl[s]);
    float wsum = 0.0f;
    for (s = 0; s + kCombineBatch <= ns; s += kCombineBatch) {
        float x[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) x[i] = pl[s + i];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) wsum += weight(x[i], mx);
    }
    for (; s < ns; ++s) wsum += weight(pl[s], mx);
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        const float* po = a.part_o + row * a.n_split * D + d;
        float acc = 0.0f;
        for (s = 0; s + kCombineBatch <= ns; s += kCombineBatch) {
            float x[kCombineBatch], o[kCombineBatch];
#pragma unroll
            for (int i = 0; i < kCombineBatch; ++i) {
                x[i] = pl[s + i];
                o[i] = po[(int64_t)(s + i) * D];
            }
#pragma unroll
            for (int i = 0; i < kCombineBatch; ++i) acc = fmaf(weight(x[i], mx), o[i], acc);
        }
        for (; s < ns; ++s) acc = fmaf(weight(pl[s], mx), po[(int64_t)s * D], acc);
        acc *= inv;
        if constexpr (OUT_F32)
            reinterpret_cast<float*>(a.o)[row * D + d] = acc;
        else
            reinterpret_cast<__bf16*>(a.o)[row * D + d] = (__bf16)acc;
    }
    if (a.lse && threadIdx.x == 0) a.lse[row] = wsum > 0.0f ? mx + __logf(wsum) : -INFINITY;
}

template <int D, int G, bool RING>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
    if (a.k_new) {
        hipLaunchKernelGGL((decode_append_kernel<D, RING>), dim3(a.hkv, (unsigned)a.batch), dim3(D / 4), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_split_kernel<D, G, RING>), dim3(a.n_split, a.hkv, (unsigned)a.batch), dim3(kThreads), 0,
                       s, a);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
    hipError_t e = a.ring ? launch_split<D, G, true>(a, s) : launch_split<D, G, false>(a, s);
    if (e != hipSuccess) return e;
    const unsigned rows = (unsigned)(a.batch * a.hq);
    if (a.out_f32)
        hipLaunchKernelGGL((decode_combine_kernel<D, true>), dim3(rows), dim3(D), 0, s, a);
    else
        hipLaunchKernelGGL((decode_combine_kernel<D, false>), dim3(rows), dim3(D), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
    switch (a.hq / a.hkv) {
        case 1: return launch_g<D, 1>(a, s);
        case 2: return launch_g<D, 2>(a, s);
        case 4: return launch_g<D, 4>(a, s);
        case 8: return launch_g<D, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t decode_scratch(void** ptr) {
    // looked up once per device, with that device current (each device holds its own copy)
    static std::mutex mu;
    static void* dev_ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (a.head_dim == 128) return launch_d<128>(a, s);
    if (a.head_dim == 64) return launch_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace flux
