// prefill_bf16.hip -- tiled attention prefill for gfx950, bf16 in, fp32 accumulate.
//
// What it computes: O = softmax(scale * Q K^T + mask) V for every (batch, query
// head), one key tile at a time with the online softmax of the openads.co.kr
// FlashAttention newsletter ("Online Softmax" section): a running row maximum m
// and row sum l, earlier partial outputs rescaled by exp(m_old - m_new) when the
// maximum grows, and the scores never leaving the chip ("FlashAttention: reduce
// memory movement" section).  In block-sparse mode only the key blocks listed in
// the CSR are visited, so K/V of the other blocks are never read (Flux Attention
// page, implementation and architecture paragraphs).
//
// Layout of the work on CDNA4:
//   * workgroup = 256 threads = 4 wave64s, 128 query rows of one (batch, head);
//     each wave owns 32 query rows; key tiles are 64 keys (= one sparse block).
//   * both contractions run on v_mfma_f32_32x32x16_bf16, computing the
//     transposed products S^T = K Q^T and O^T = V^T P^T.  With that orientation a
//     lane's 32x32 accumulator column is one query row, so the softmax statistics
//     (row max, row sum, rescale factor) of a lane's outputs are lane-local: only
//     one cross-lane step (lanes l and l^32) per tile for the max, none for O.
//   * Q stays in registers as the B operand of S^T for the whole kernel.
//   * K tiles are staged row-major in LDS; V tiles are staged transposed (Vt[d][key])
//     with keys permuted inside each 16-key group so that one 16-byte LDS read gives a
//     lane exactly the 8 keys its P registers hold.  The transpose happens in
//     registers between the global load and the LDS store.
//   * two LDS stages: the global loads of tile t+1 are in flight while tile t is
//     computed; one barrier per tile.
//   * exp2 with scale*log2(e) folded into one FMA; the O rescale is skipped when no
//     row maximum grew (exact: the factor would be 1).
//   * workgroup order: kv-head groups are kept on one XCD (blockIdx % 8 picks the
//     XCD) so the 4 query heads sharing K/V hit the same L2, and query tiles are
//     issued longest-first for causal masks.
#include "flux_internal.h"

namespace flux {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBR = 128;       // query rows per workgroup
constexpr int kBC = 64;        // keys per tile
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;  // finite start value of the running max
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
struct Lay {
    static constexpr int KS = D + 8;                       // K row stride in LDS (elements)
    static constexpr int VS = kBC + 8;                     // Vt row stride in LDS (elements)
    static constexpr int K_ELEMS = kBC * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;        // elements per LDS stage
    static constexpr int KCH = D / 8;                      // 16-byte chunks per K row
    static constexpr int K_LOADS = kBC * KCH / kThreads;   // 16-byte K loads per thread
    static constexpr int VG = D / 4;                       // groups of 4 d per V row
    static constexpr int V_KQ = kThreads / VG;             // key quads per V round
    static constexpr int V_ROUNDS = kBC / (4 * V_KQ);
    static_assert(K_LOADS * kThreads == kBC * KCH, "K tile split");
    static_assert(V_ROUNDS * 4 * V_KQ == kBC, "V tile split");
};

// Position of key k (0..63) inside a Vt row: bits 2 and 3 swapped, so that the
// keys a lane holds in its P registers (see kernel) are 8 consecutive entries.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <int D>
struct TileRegs {
    u32x4 k[Lay<D>::K_LOADS];
    u32x2 v[Lay<D>::V_ROUNDS][4];
};

// Global -> registers for key tile kb.  Keys past the end of the sequence are
// clamped to the last row (no branches); their scores are masked to -inf and
// their probabilities are 0, so the duplicated rows never contribute.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const u16* __restrict__ kg, const u16* __restrict__ vg,
                                          uint32_t row_stride, int kb, int last_key, int tid) {
    using L = Lay<D>;
    const int key0 = kb * kBC;
#pragma unroll
    for (int i = 0; i < L::K_LOADS; ++i) {
        const int idx = tid + i * kThreads;
        const int row = idx / L::KCH, ch = idx % L::KCH;
        const uint32_t key = (uint32_t)min(key0 + row, last_key);
        r.k[i] = *reinterpret_cast<const u32x4*>(kg + key * row_stride + ch * 8);
    }
    const int dg = tid % L::VG, kq = tid / L::VG;
#pragma unroll
    for (int rr = 0; rr < L::V_ROUNDS; ++rr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t key = (uint32_t)min(key0 + rr * 4 * L::V_KQ + 4 * kq + e, last_key);
            r.v[rr][e] = *reinterpret_cast<const u32x2*>(vg + key * row_stride + dg * 4);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, u16* ks, u16* vts, int tid) {
    using L = Lay<D>;
#pragma unroll
    for (int i = 0; i < L::K_LOADS; ++i) {
        int idx = tid + i * kThreads;
        int row = idx / L::KCH, ch = idx % L::KCH;
        *reinterpret_cast<u32x4*>(ks + row * L::KS + ch * 8) = r.k[i];
    }
    const int dg = tid % L::VG, kq = tid / L::VG;
#pragma unroll
    for (int rr = 0; rr < L::V_ROUNDS; ++rr) {
        const int pos = vt_pos(rr * 4 * L::V_KQ + 4 * kq);
        const u32x2 x0 = r.v[rr][0], x1 = r.v[rr][1], x2 = r.v[rr][2], x3 = r.v[rr][3];
        // 4 keys x 4 d  ->  4 d x 4 keys (bf16 halves regrouped)
        u32x2 o0, o1, o2, o3;
        o0.x = (x0.x & 0xffffu) | (x1.x << 16);
        o0.y = (x2.x & 0xffffu) | (x3.x << 16);
        o1.x = (x0.x >> 16) | (x1.x & 0xffff0000u);
        o1.y = (x2.x >> 16) | (x3.x & 0xffff0000u);
        o2.x = (x0.y & 0xffffu) | (x1.y << 16);
        o2.y = (x2.y & 0xffffu) | (x3.y << 16);
        o3.x = (x0.y >> 16) | (x1.y & 0xffff0000u);
        o3.y = (x2.y >> 16) | (x3.y & 0xffff0000u);
        u16* base = vts + (4 * dg) * L::VS + pos;
        *reinterpret_cast<u32x2*>(base) = o0;
        *reinterpret_cast<u32x2*>(base + L::VS) = o1;
        *reinterpret_cast<u32x2*>(base + 2 * L::VS) = o2;
        *reinterpret_cast<u32x2*>(base + 3 * L::VS) = o3;
    }
}

// Bijection blockIdx -> logical work id that keeps consecutive logical ids on one
// XCD (workgroups are dealt to the 8 XCDs round-robin by blockIdx).
__device__ __forceinline__ int xcd_remap(int x, int total) {
    constexpr int kXcd = 8;
    const int per = total / kXcd;
    if (x >= per * kXcd) return x;
    return (x % kXcd) * per + x / kXcd;
}

enum Mode { kDenseCausal = 0, kDenseFull = 1, kSparse = 2 };

// Walks the key tiles of a workgroup (query blocks qb0 = 2*qt and qb1 = qb0+1):
// dense -- tiles 0..last; sparse -- the sorted union of the two CSR rows.
template <int MODE>
struct TileWalk {
    int next_kb, last_kb, qb0, qb1;
    int p0, e0, p1, e1;
    const int32_t* ci;

    __device__ void init(int qt, int n_qblk, const int32_t* rp, const int32_t* ci_) {
        qb0 = 2 * qt;
        qb1 = 2 * qt + 1;
        ci = ci_;
        if constexpr (MODE == kSparse) {
            p0 = rp[qb0];
            e0 = rp[qb0 + 1];
            if (qb1 < n_qblk) {
                p1 = rp[qb1];
                e1 = rp[qb1 + 1];
            } else {
                p1 = e1 = 0;
            }
        } else {
            next_kb = 0;
            last_kb = MODE == kDenseCausal ? min(qb1, n_qblk - 1) : n_qblk - 1;
        }
    }

    // Next tile; in0/in1: whether query block qb0/qb1 uses it.
    __device__ bool next(int& kb, bool& in0, bool& in1) {
        if constexpr (MODE == kSparse) {
            const int big = 0x7fffffff;
            int c0 = p0 < e0 ? ci[p0] : big;
            int c1 = p1 < e1 ? ci[p1] : big;
            kb = min(c0, c1);
            if (kb == big) return false;
            in0 = c0 == kb;
            in1 = c1 == kb;
            p0 += in0;
            p1 += in1;
            return true;
        } else {
            if (next_kb > last_kb) return false;
            kb = next_kb++;
            in0 = MODE == kDenseFull || kb <= qb0;
            in1 = MODE == kDenseFull || kb <= qb1;
            return true;
        }
    }
};

template <int D, int MODE, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2))) void
prefill_bf16_kernel(PrefillArgs a) {
    using L = Lay<D>;
    constexpr int NC = D / 16;   // 16-wide d chunks of the S^T contraction
    constexpr int NM = D / 32;   // 32-row d tiles of O^T
    __shared__ __attribute__((aligned(16))) u16 smem[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;     // query column of this lane inside the wave's 32 rows
    const int hh = lane >> 5;    // which half of the k-slots / accumulator rows

    const int nqt = (int)((a.seq + kBR - 1) / kBR);
    const int G = a.hq / a.hkv;
    const int total = (int)(a.batch * a.hq) * nqt;
    int lid = xcd_remap((int)blockIdx.x, total);
    const int j = lid % G;
    lid /= G;
    const int qt_rank = lid % nqt;
    lid /= nqt;
    const int g = lid % a.hkv;
    const int b = lid / a.hkv;
    const int h = g * G + j;
    const int qt = (MODE == kDenseCausal) ? nqt - 1 - qt_rank : qt_rank;

    const uint32_t q_row_stride = (uint32_t)(a.hq * D);
    const uint32_t kv_row_stride = (uint32_t)(a.hkv * D);
    const int seq = (int)a.seq;          // the host guarantees seq * max(hq, hkv) * d < 2^31
    const int last_key = seq - 1;
    const u16* qg = reinterpret_cast<const u16*>(a.q) + ((int64_t)b * a.seq * a.hq + h) * D;
    const u16* kg = reinterpret_cast<const u16*>(a.k) + ((int64_t)b * a.seq * a.hkv + g) * D;
    const u16* vg = reinterpret_cast<const u16*>(a.v) + ((int64_t)b * a.seq * a.hkv + g) * D;

    const int q0 = qt * kBR + wave * 32;       // first query row of this wave
    const int qpos = q0 + n;                   // this lane's query row
    const bool wave_live = q0 < seq;
    const bool wave_in_qb1 = wave >= 2;
    const int my_qb = qt * 2 + (wave_in_qb1 ? 1 : 0);

    // Q rows as the B operand of S^T = K Q^T: lane holds Q[qpos][16c + 8hh .. +7]
    bf16x8 qreg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const uint32_t qrow = (uint32_t)min(qpos, last_key);
        qreg[c] = *reinterpret_cast<const bf16x8*>(qg + qrow * q_row_stride + 16 * c + 8 * hh);
    }
    // wait for Q here: otherwise the wait for Q lands inside the tile loop, where it also
    // waits for the next tile's prefetch (vmcnt counts every outstanding load)
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)

    f32x16 oacc[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) oacc[mt] = f32x16{};
    float m_run = kNegBig, l_run = 0.0f;
    const float c2 = a.scale_log2;

    TileWalk<MODE> walk;
    walk.init(qt, a.n_qblk, a.row_ptr, a.col_idx);
    int kb;
    bool in0, in1;
    bool have = walk.next(kb, in0, in1);
    TileRegs<D> regs;
    if (have) {
        load_tile<D>(regs, kg, vg, kv_row_stride, kb, last_key, tid);
        store_tile<D>(regs, smem, smem + L::K_ELEMS, tid);
    }
    __syncthreads();
    int buf = 0;
    while (have) {
        int kb_n;
        bool in0_n, in1_n;
        const bool have_n = walk.next(kb_n, in0_n, in1_n);
        if (have_n) load_tile<D>(regs, kg, vg, kv_row_stride, kb_n, last_key, tid);

        const bool mine = wave_live && (wave_in_qb1 ? in1 : in0);
        if (mine) {
            const u16* ks = smem + buf * L::STAGE;
            const u16* vts = ks + L::K_ELEMS;
            // ---- S^T = K Q^T : two 32-key halves, two independent accumulation chains
            f32x16 sacc[2] = {f32x16{}, f32x16{}};
            const u16* krow = ks + n * L::KS + 8 * hh;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(krow + 16 * c);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(krow + 32 * L::KS + 16 * c);
                sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[c], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[c], sacc[1], 0, 0, 0);
            }
            // lane holds S[qpos][key], key = kb*64 + 32kh + 8(r/4) + 4hh + (r%4)
            const bool need_mask = (MODE != kDenseFull && kb >= my_qb) || (kb + 1) * kBC > seq;
            if (need_mask) {
                // key = kb*64 + 32kh + 8(r/4) + 4hh + r%4 is masked when key > lim
                const int lim = (MODE != kDenseFull ? min(qpos, last_key) : last_key) - (kb * kBC + 4 * hh);
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * kh + 8 * (r >> 2) + (r & 3) > lim) sacc[kh][r] = -INFINITY;
            }
            float mx = sacc[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
            const float mc = m_new * c2;
            float rs = 0.0f;
            bf16x8 pb[2][2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int aa = 0; aa < 2; ++aa) {
                    float p[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        p[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[kh][8 * aa + jj], c2, -mc));
                        rs += p[jj];
                    }
                    pb[kh][aa] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                                        (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int mt = 0; mt < NM; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[mt][r] *= alpha;
            }
            // ---- O^T += V^T P^T ; P slot jj of step (kh, aa) is key 32kh + 16aa + 8(jj/4) + 4hh + jj%4
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
                const u16* vrow = vts + (32 * mt + n) * L::VS + 8 * hh;
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int aa = 0; aa < 2; ++aa) {
                        bf16x8 av = *reinterpret_cast<const bf16x8*>(vrow + 32 * kh + 16 * aa);
                        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kh][aa], oacc[mt], 0, 0, 0);
                    }
            }
        }
        if (have_n) {
            u16* ks_n = smem + (buf ^ 1) * L::STAGE;
            store_tile<D>(regs, ks_n, ks_n + L::K_ELEMS, tid);
        }
        __syncthreads();
        buf ^= 1;
        kb = kb_n;
        in0 = in0_n;
        in1 = in1_n;
        have = have_n;
    }

    // ---- epilogue: O = O^T / l, lane holds O[qpos][32mt + 8(r/4) + 4hh + r%4]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!wave_live || qpos >= seq) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t orow = ((int64_t)b * seq + qpos) * a.hq + h;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * mt + 8 * r4 + 4 * hh;
            const float v0 = oacc[mt][4 * r4] * inv, v1 = oacc[mt][4 * r4 + 1] * inv;
            const float v2 = oacc[mt][4 * r4 + 2] * inv, v3 = oacc[mt][4 * r4 + 3] * inv;
            if constexpr (OUT_F32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + orow * D + d) = make_float4(v0, v1, v2, v3);
            } else {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 pk = bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                *reinterpret_cast<bf16x4*>(reinterpret_cast<u16*>(a.o) + orow * D + d) = pk;
            }
        }
    if (a.lse && hh == 0) {
        const float lse = l_tot > 0.0f ? (m_run * c2 + __log2f(l_tot)) * kLn2 : -INFINITY;
        a.lse[((int64_t)b * a.hq + h) * a.seq + qpos] = lse;
    }
}

template <int D, int MODE>
hipError_t launch_mode(const PrefillArgs& a, hipStream_t s) {
    const int64_t nqt = (a.seq + kBR - 1) / kBR;
    const int64_t grid = a.batch * a.hq * nqt;
    if (a.out_f32)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const PrefillArgs& a, hipStream_t s) {
    if (a.sparse) return launch_mode<D, kSparse>(a, s);
    if (a.causal) return launch_mode<D, kDenseCausal>(a, s);
    return launch_mode<D, kDenseFull>(a, s);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    if (a.head_dim == 128) return launch_dim<128>(a, s);
    if (a.head_dim == 64) return launch_dim<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace flux
