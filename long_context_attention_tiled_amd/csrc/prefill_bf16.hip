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
//   * both contractions run on v_mfma_f32_32x32x16_bf16 in transposed form,
//     S^T = K Q^T and O^T = V^T P^T.  A lane's 32x32 accumulator column is then one
//     query row, so the softmax statistics (row max, row sum, rescale factor) of a
//     lane's outputs are lane-local: one l <-> l^32 exchange per tile, none for O.
//   * Q stays in registers (B operand of S^T) for the whole kernel.
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4: no
//     staging registers, no LDS store instructions), row-major with an XOR swizzle
//     of the 16-byte chunks of each row so that the operand reads are bank-conflict
//     free.  The V^T operand is read with ds_read_b64_tr_b16, which transposes
//     4x4 blocks of 16-bit elements across lanes: every lane receives 4 keys of its
//     own d column per read, so V never needs a transposed copy.
//   * two LDS stages: the loads of tile t+1 are in flight while tile t is
//     computed; one barrier per tile.
//   * exp2 with scale*log2(e) folded into one FMA.  The running maximum is raised
//     only when some row's new maximum exceeds it by more than 8 (log2 units):
//     until then probabilities up to 2^8 are accumulated against the old
//     reference, which is exact in exact arithmetic (the same reference scales
//     numerator and denominator) and removes most O rescales; the newsletter's
//     FlashAttention-4 section describes the m_new <= m_old special case of this.
//   * the row sum is taken over the bf16-rounded P that enters P.V (v_dot2 against
//     (1, 1)), so O is a convex combination of V rows up to fp32 accumulation.
//   * workgroup order: kv-head groups are kept on one XCD (blockIdx % 8 picks the
//     XCD) so the query heads sharing K/V hit the same L2, and query tiles are
//     issued longest-first for causal masks.
#include "flux_internal.h"

namespace flux {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBR = 128;       // query rows per workgroup
constexpr int kBC = 64;        // keys per tile
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;  // finite start value of the running max
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag the true max

template <int D>
struct Lay {
    static constexpr int ROW_B = D * 2;                    // bytes per K/V row in LDS (no padding)
    static constexpr int CH = ROW_B / 16;                  // 16-byte chunks per row
    static constexpr int TILE_B = kBC * ROW_B;             // bytes per K (or V) tile
    static constexpr int STAGE_B = 2 * TILE_B;             // K tile + V tile
    static constexpr int ROWS_PER_INST = 1024 / ROW_B;     // rows one direct-load instruction fills
    static constexpr int INSTS_PER_WAVE = TILE_B / 1024 / 4;
    static_assert(INSTS_PER_WAVE * 4 * 1024 == TILE_B, "tile split over 4 waves");
};

// Chunk swizzles (physical chunk = logical chunk ^ swizzle(row)).  K rows are read
// 16 (or 8) at a time at one logical chunk by the S^T operand loads; V rows are read
// 8 at a time, 64 bytes each, by the transposing loads.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row ^ (row >> 3)) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
    if constexpr (D == 128) return 4 * (row & 3);
    else return 4 * ((row >> 1) & 1);
}

// 16-byte direct HBM -> LDS load from sbase + voff (sbase wave-uniform, in SGPRs; voff a
// per-lane byte offset): lane l's 16 bytes land at LDS byte lds_base + 16*l (lds_base is
// wave-uniform and goes through M0).  Written as inline asm on purpose: the instruction
// has no destination register, and hiding it from the compiler's wait-count pass stops
// that pass from assuming the in-flight write may alias every later LDS read of the
// other stage (it would then wait for the whole prefetch before the P.V reads).  The
// kernel itself waits for vmcnt(0) before the barrier that publishes a tile.
__device__ __forceinline__ void load_lds_16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

__device__ __forceinline__ i16x4 read_tr16(const char* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
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

// Issue this wave's share of the direct HBM -> LDS loads of key tile kb.  Lane l of
// instruction inst fills LDS bytes [1024*inst + 16*l, +16): row inst*ROWS_PER_INST +
// l/CH, physical chunk l%CH, i.e. logical chunk (l%CH) ^ swizzle(row) of that key.
// Keys past the end of the sequence are clamped to the last one (masked to -inf in
// the scores, probability 0 in P.V).
template <int D>
__device__ __forceinline__ void issue_tile(const u16* __restrict__ kg, const u16* __restrict__ vg,
                                           uint32_t row_stride, int kb, int last_key, char* stage, int wave,
                                           int lane, const uint32_t* koff, const uint32_t* voff) {
    using L = Lay<D>;
    const int key0 = kb * kBC;
    const uint32_t ks = __builtin_amdgcn_readfirstlane(lds_addr(stage));
    const uint32_t vs = ks + L::TILE_B;
    if (key0 + kBC - 1 <= last_key) {
        const u16* kt = kg + (uint32_t)key0 * row_stride;   // uniform
        const u16* vt = vg + (uint32_t)key0 * row_stride;
#pragma unroll
        for (int i = 0; i < L::INSTS_PER_WAVE; ++i) {
            const int inst = wave * L::INSTS_PER_WAVE + i;
            load_lds_16(kt, koff[i], ks + inst * 1024);
            load_lds_16(vt, voff[i], vs + inst * 1024);
        }
    } else {
#pragma unroll
        for (int i = 0; i < L::INSTS_PER_WAVE; ++i) {
            const int inst = wave * L::INSTS_PER_WAVE + i;
            const int row = inst * L::ROWS_PER_INST + lane / L::CH;
            const uint32_t key = (uint32_t)min(key0 + row, last_key);
            const int pch = lane % L::CH;
            load_lds_16(kg, 2 * (key * row_stride + 8 * (pch ^ swz_k<D>(row))), ks + inst * 1024);
            load_lds_16(vg, 2 * (key * row_stride + 8 * (pch ^ swz_v<D>(row))), vs + inst * 1024);
        }
    }
}

template <int D, int MODE, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2))) void
prefill_bf16_kernel(PrefillArgs a) {
    using L = Lay<D>;
    constexpr int NC = D / 16;   // 16-wide d chunks of the S^T contraction
    constexpr int NM = D / 32;   // 32-row d tiles of O^T
    __shared__ __attribute__((aligned(1024))) char smem[2 * L::STAGE_B];

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

    // per-lane byte offsets of the direct loads inside a tile (tile-invariant)
    uint32_t koff[L::INSTS_PER_WAVE], voff[L::INSTS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < L::INSTS_PER_WAVE; ++i) {
        const int row = (wave * L::INSTS_PER_WAVE + i) * L::ROWS_PER_INST + lane / L::CH;
        const int pch = lane % L::CH;
        koff[i] = 2 * (row * kv_row_stride + 8 * (pch ^ swz_k<D>(row)));   // bytes
        voff[i] = 2 * (row * kv_row_stride + 8 * (pch ^ swz_v<D>(row)));
    }

    // Q rows as the B operand of S^T = K Q^T: lane holds Q[qpos][16c + 8hh .. +7]
    bf16x8 qreg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const uint32_t qrow = (uint32_t)min(qpos, last_key);
        qreg[c] = *reinterpret_cast<const bf16x8*>(qg + qrow * q_row_stride + 16 * c + 8 * hh);
    }

    // LDS byte offsets of this lane's operand reads (stage-relative)
    // K: row 32kh + n, logical chunk 2c + hh -> physical (2c + hh) ^ swz_k(n)  (swz_k(32kh+n) = swz_k(n)
    // for d = 128; for d = 64 the 32kh term is added below through the row address only)
    uint32_t kaddr[2][NC];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            kaddr[kh][c] = (32 * kh + n) * L::ROW_B + 16 * ((2 * c + hh) ^ swz_k<D>(32 * kh + n));
    // V (transposing reads): 16-lane group gq = lane/16 -> key quad hh = gq>>1, d half dh = gq&1;
    // lane jj = lane&15 points at key 4hh + (jj>>2) (+ tile offsets), d = 32mt + 16dh + 4(jj&3)
    const int jj = lane & 15, dh = (lane >> 4) & 1;
    const int vkey = 4 * hh + (jj >> 2);
    uint32_t vaddr[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
        const int lch = 4 * mt + 2 * dh + ((jj & 3) >> 1);
        vaddr[mt] = L::TILE_B + vkey * L::ROW_B + 16 * (lch ^ swz_v<D>(vkey)) + 8 * (jj & 1);
    }

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
    if (have) issue_tile<D>(kg, vg, kv_row_stride, kb, last_key, smem, wave, lane, koff, voff);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): Q and tile 0 in place
    __syncthreads();
    int buf = 0;
    while (have) {
        int kb_n;
        bool in0_n, in1_n;
        const bool have_n = walk.next(kb_n, in0_n, in1_n);
        if (have_n)
            issue_tile<D>(kg, vg, kv_row_stride, kb_n, last_key, smem + (buf ^ 1) * L::STAGE_B, wave, lane, koff,
                          voff);

        const bool mine = wave_live && (wave_in_qb1 ? in1 : in0);
        if (mine) {
            const char* st = smem + buf * L::STAGE_B;
            // ---- S^T = K Q^T : two 32-key halves, two independent accumulation chains.  The
            // K operands of step c+1 are read from LDS while step c's MFMAs run, and the wave
            // raises its issue priority for the MFMA phase so that the other wave on the SIMD
            // fills the gaps with its vector work.
            __builtin_amdgcn_s_setprio(2);
            f32x16 sacc[2] = {f32x16{}, f32x16{}};
            bf16x8 ka[2][2];
            ka[0][0] = *reinterpret_cast<const bf16x8*>(st + kaddr[0][0]);
            ka[0][1] = *reinterpret_cast<const bf16x8*>(st + kaddr[1][0]);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if (c + 1 < NC) {
                    ka[(c + 1) & 1][0] = *reinterpret_cast<const bf16x8*>(st + kaddr[0][c + 1]);
                    ka[(c + 1) & 1][1] = *reinterpret_cast<const bf16x8*>(st + kaddr[1][c + 1]);
                }
                sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c & 1][0], qreg[c], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c & 1][1], qreg[c], sacc[1], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            // lane holds S[qpos][key], key = kb*64 + 32kh + 8(r/4) + 4hh + (r%4)
            const bool need_mask = (MODE != kDenseFull && kb >= my_qb) || (kb + 1) * kBC > seq;
            if (need_mask) {
                // key > lim is masked, lim = last allowed key of this lane's row minus the tile/lane base
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
            // raise the reference max only when some row outgrows it by more than the slack
            if (__ballot((mx - m_run) * c2 > kRescaleSlack)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
                l_run *= alpha;
#pragma unroll
                for (int mt = 0; mt < NM; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[mt][r] *= alpha;
                m_run = m_new;
            }
            const float mc = m_run * c2;
            bf16x8 pb[2][2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int aa = 0; aa < 2; ++aa) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kh][8 * aa + e], c2, -mc));
                    pb[kh][aa] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                                        (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
                }
            // row sum over the rounded P (exactly what P.V uses)
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int aa = 0; aa < 2; ++aa) {
                    const bf16x8 v = pb[kh][aa];
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, ones, l_run, false);
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, ones, l_run, false);
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[4], v[5]}, ones, l_run, false);
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[6], v[7]}, ones, l_run, false);
                }
            // ---- O^T += V^T P^T ; P slot e' of step (kh, aa) is key 32kh + 16aa + 8(e'/4) + 4hh + e'%4.
            // Two transposing reads per step: keys +0..3 and +8..11 of the lane group's 4-key block.
            // the V operand of step i+1 is read while step i's MFMA runs
            __builtin_amdgcn_s_setprio(2);
            auto vread = [&](int i) {
                const int mt = i >> 2, kh = (i >> 1) & 1, aa = i & 1;
                const char* vp = st + vaddr[mt] + (32 * kh + 16 * aa) * L::ROW_B;
                const i16x4 lo = read_tr16(vp);
                const i16x4 hi = read_tr16(vp + 8 * L::ROW_B);
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            bf16x8 va[2];
            va[0] = vread(0);
#pragma unroll
            for (int i = 0; i < 4 * NM; ++i) {
                if (i + 1 < 4 * NM) va[(i + 1) & 1] = vread(i + 1);
                const int mt = i >> 2, kh = (i >> 1) & 1, aa = i & 1;
                oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i & 1], pb[kh][aa], oacc[mt], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's share of tile t+1 has landed
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
