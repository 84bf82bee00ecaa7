// backward.hip -- gradients of tiled attention on gfx950 (bf16 inputs, head_dim 128, fp32 gradients).
//
// With P the probabilities of one attention row (rebuilt from Q, K and the row log-sum-exp the
// forward pass keeps), the chain rule through the softmax gives, per (batch, query head):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D = rowsum(dO * O) = rowsum(P * dP),
//   dQ = scale dS K,  dK = scale dS^T Q
// -- the softmax Jacobian diag(p) - p p^T applied row by row to the attention definition of the
// FlashAttention newsletter ("Softmax is not a simple function").  It is what training the layer
// router of the Flux Attention page over a frozen backbone needs.  As in the forward pass, the
// score matrix never reaches HBM: it is rebuilt tile by tile over the same key sets (causal,
// all keys, or the sink + local window of 64-token blocks, whose other blocks are never read).
//
// Kernels, in stream order:
//   bwd_rowstat_kernel    D and -LSE*log2(e) per query row, in 64-row tiles (rows past the end get
//                         (-inf, 0), so they weigh nothing); clears the two work-queue heads.
//   bwd_dkdv_kernel       one work unit = 128 keys (4 waves x 32) and one query head; walks the
//                         64-query tiles that see those keys: S = Q K^T and dP = dO V^T with K, V
//                         held in registers (keys in lanes), then dV^T += dO^T P and dK^T += Q^T dS
//                         with the Q and dO tiles read transposed from LDS.
//   bwd_dq_kernel         one work unit = 128 queries (4 waves x 32) of one query head; walks the
//                         visible 64-key tiles: S^T = K Q^T and dP^T = V dO^T with Q, dO in
//                         registers (queries in lanes), then dQ^T += K^T dS^T.
//   bwd_group_sum_kernel  grouped-query attention: adds the per-query-head dK/dV of each group, in
//                         head order, into dK/dV.
// Computing dQ apart from dK/dV rebuilds S and dP once more (7 matrix products instead of 5) but
// needs no atomics: every gradient element is written once, summed in a fixed order.
//
// P and dS enter the gradient products as a bf16 pair hi + lo (hi = x truncated to bf16, lo =
// bf16(x - hi)):
// the sums over up to seq rows of bf16-rounded P or dS alone would carry a relative error of
// 2^-9 per term, about 1e-2 absolute on gradients of size 5; the pair brings it near 2^-16 at the
// cost of a second MFMA on the same A operand.
//
// Both main kernels are persistent (one workgroup per CU, 1 wave per SIMD) and take units from a
// device counter, longest first.  Two LDS slots: the tile in use and the next one in flight.
#include "flux_internal.h"
#include "tile_common.h"

namespace flux {
namespace {

using namespace tile;

constexpr int kD = 128;
constexpr int kNC = kD / 16;          // 16-wide d chunks: contraction steps of S and dP
constexpr int kNM = kD / 32;          // 32-row d tiles of the transposed gradients
constexpr int kRowB = kD * 2;         // bytes of one bf16 row
constexpr int kTileB = 64 * kRowB;    // one 64-row tile
constexpr int kStatB = 512;           // a tile's row statistics: 64 x -LSE*log2(e), then 64 x D
constexpr int kSlotB = 2 * kTileB + kStatB;
constexpr int kSlots = 2;            // the tile in use and the next one in flight
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

// One chunk swizzle for row reads (16 aligned rows at one logical chunk: 16 distinct physical
// chunks) and transposing reads (4 aligned rows x 4 aligned chunks): swapping the two 2-bit halves
// of row & 15 is a bijection on 16 rows and gives 4 aligned rows 4 distinct high halves.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// 4-byte direct HBM -> LDS load (see load_lds_16): lane l's dword lands at lds_base + 4*l.
__device__ __forceinline__ void load_lds_4(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory", "m0");
}

// 64 rows of kD bf16 (row r at base + r * row_stride elements, rows past last_row clamped to it)
// into one LDS tile: row r at r * kRowB, 16-byte chunks swizzled.  16 loads of 1 KB (4 rows each),
// 4 per wave.
__device__ __forceinline__ void load_tile(const u16* base, uint32_t row_stride, int r0, int last_row, uint32_t lds,
                                          int wave, int lane) {
    const u16* sb = uniform_ptr(base);
    const int pch = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int inst = wave * 4 + i;
        const int row = inst * 4 + (lane >> 4);
        const uint32_t grow = (uint32_t)min(r0 + row, last_row);
        load_lds_16(sb, 2u * (grow * row_stride + 8u * (uint32_t)(pch ^ swz(row))), lds + inst * 1024);
    }
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
    return bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                  (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lane geometry of the MFMA operands (v_mfma_f32_32x32x16_bf16: lane l feeds row/column l % 32 with
// k-slots 8(l/32) .. +7; the accumulator's register r of lane l is row 8(r/4) + 4(l/32) + r%4).
struct Lanes {
    int lane, n, hh, jj, dh;
    uint32_t rd[kNC];          // row read: row n, logical chunk 2c + hh (add 32 rows: + 32 * kRowB)
    uint32_t trl[kNM], trh[kNM];  // transposing reads of k-step 0: rows 4hh + jj/4 (lo) and + 8 (hi)
    __device__ __forceinline__ void init(int l) {
        lane = l;
        n = l & 31;
        hh = l >> 5;
        jj = l & 15;
        dh = (l >> 4) & 1;
#pragma unroll
        for (int c = 0; c < kNC; ++c) rd[c] = n * kRowB + 16 * ((2 * c + hh) ^ swz(n));
        const int rlo = 4 * hh + (jj >> 2), rhi = rlo + 8;
#pragma unroll
        for (int mt = 0; mt < kNM; ++mt) {
            const int lch = 4 * mt + 2 * dh + ((jj & 3) >> 1);
            trl[mt] = rlo * kRowB + 16 * (lch ^ swz(rlo)) + 8 * (jj & 1);
            trh[mt] = rhi * kRowB + 16 * (lch ^ swz(rhi)) + 8 * (jj & 1);
        }
    }
    // A operand X^T[32mt + l%32][16kk + k-slots] of a 64-row tile X (k-slot e of lane half hh is
    // row 16kk + 8(e/4) + 4hh + e%4, matching the accumulator layout of the B operand).
    __device__ __forceinline__ bf16x8 tr(const char* tile, int kk, int mt) const {
        const i16x4 lo = read_tr16(tile + kk * 16 * kRowB + trl[mt]);
        const i16x4 hi = read_tr16(tile + kk * 16 * kRowB + trh[mt]);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // A operand X[32half + l%32][16c + 8(l/32) .. +7] of a 64-row tile X
    __device__ __forceinline__ bf16x8 row(const char* tile, int half, int c) const {
        return *reinterpret_cast<const bf16x8*>(tile + half * 32 * kRowB + rd[c]);
    }
};

// Work queue: thread 0 takes the next unit; two LDS cells alternate so that the value read at the
// end of one unit is not overwritten before every thread has read it.
struct Queue {
    int* counter;
    int* cell;   // LDS [2]
    int it;
    __device__ __forceinline__ int first() {
        if (threadIdx.x == 0) cell[0] = atomicAdd(counter, 1);
        __syncthreads();
        it = 0;
        return __builtin_amdgcn_readfirstlane(cell[0]);
    }
    __device__ __forceinline__ void prefetch() {
        if (threadIdx.x == 0) cell[(it + 1) & 1] = atomicAdd(counter, 1);
    }
    __device__ __forceinline__ int next() {   // after a __syncthreads that follows prefetch()
        ++it;
        return __builtin_amdgcn_readfirstlane(cell[it & 1]);
    }
};

// ------------------------------------------------------------------ row statistics
__global__ void __launch_bounds__(256) bwd_rowstat_kernel(BackwardArgs a) {
    if (blockIdx.x == 0 && threadIdx.x < 2) a.counters[threadIdx.x] = 0;
    const int padded = a.n_qblk * 64;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (row >= a.batch * padded * a.hq) return;   // all 16 lanes of a row leave together
    const int h = (int)(row % a.hq);
    const int64_t rest = row / a.hq;
    const int i = (int)(rest % padded);
    const int64_t b = rest / padded;
    float acc = 0.0f;
    if (i < a.seq) {
        const int64_t off = ((b * a.seq + i) * a.hq + h) * kD + 8 * c;
        const uint4 g4 = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(a.d_o) + off);
        float o[8];
        if (a.o_f32) {
            const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.o) + off);
            const float4 y = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.o) + off + 4);
            o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w; o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(a.o) + off);
            o[0] = bf16_lo(x.x); o[1] = bf16_hi(x.x); o[2] = bf16_lo(x.y); o[3] = bf16_hi(x.y);
            o[4] = bf16_lo(x.z); o[5] = bf16_hi(x.z); o[6] = bf16_lo(x.w); o[7] = bf16_hi(x.w);
        }
        acc = o[0] * bf16_lo(g4.x) + o[1] * bf16_hi(g4.x);
        acc += o[2] * bf16_lo(g4.y) + o[3] * bf16_hi(g4.y);
        acc += o[4] * bf16_lo(g4.z) + o[5] * bf16_hi(g4.z);
        acc += o[6] * bf16_lo(g4.w) + o[7] * bf16_hi(g4.w);
    }
    acc += __shfl_xor(acc, 8, 16);
    acc += __shfl_xor(acc, 4, 16);
    acc += __shfl_xor(acc, 2, 16);
    acc += __shfl_xor(acc, 1, 16);
    if (c == 0) {
        float* st = a.stat + ((b * a.hq + h) * a.n_qblk + i / 64) * 128 + i % 64;
        const bool live = i < a.seq;
        st[0] = live ? -a.lse[(b * a.hq + h) * a.seq + i] * kLog2e : -INFINITY;
        st[64] = live ? acc : 0.0f;
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// (x0, x1) = hi + lo per element, hi = x with its low 16 bits cleared (exact in bf16), lo = bf16(x - hi):
// two bf16 MFMA operands whose products sum to x * y with a relative error near 2^-16 instead of
// bf16's 2^-9.  Packed as bf16 pairs (element 2i in the low half of word i).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const float h0 = __uint_as_float(__float_as_uint(x0) & 0xffff0000u);
    const float h1 = __uint_as_float(__float_as_uint(x1) & 0xffff0000u);
    hi = pack2(h0, h1);
    lo = pack2(x0 - h0, x1 - h1);
}

__device__ __forceinline__ bf16x8 as_op(const uint32_t* w) {
    return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

__device__ __forceinline__ float comp(const float4& v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)

// ------------------------------------------------------------------ dK, dV
//
// One 64-query tile for a wave (32 keys) is 96 MFMAs: 32 for S and dP (16 rows at a time from the Q
// and dO tiles, K and V rows in registers), then 16 groups of 4 for dV^T and dK^T (each group one
// transposed dO operand and one transposed Q operand, times P hi, dS hi, P lo, dS lo).  The vector
// work of the tile is spread over the MFMA steps once its inputs are complete (exp of S half 0
// during S half 1, of half 1 during dP, dS during dP half 1 and the first gradient groups), and
// every LDS operand is read a few MFMAs ahead; sched_barrier pins that order.
__global__ void __launch_bounds__(kThreads, 1) bwd_dkdv_kernel(BackwardArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSlots * kSlotB];
    __shared__ int qcell[2];
    Lanes L;
    L.init(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = L.lane, n = L.n, hh = L.hh;

    const int seq = (int)a.seq, nqb = a.n_qblk, G = a.hq / a.hkv;
    const int bh_total = (int)a.batch * a.hq;
    const int total = ((nqb + 1) / 2) * bh_total;
    const uint32_t q_stride = (uint32_t)a.hq * kD;
    const float c2 = a.scale_log2;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    Queue queue{a.counters + 0, qcell, 0};
    int u = queue.first();
    while (u < total) {
        queue.prefetch();
        const int m = u / bh_total, bh = u % bh_total;   // key pair m: longest query range first
        const int b = bh / a.hq, h = bh % a.hq, g = h / G;
        const int kb = 2 * m + (wave >> 1);               // this wave's key block
        const int key = 128 * m + 32 * wave + n;          // this lane's key
        int lo = 0, hi = nqb - 1;
        if (a.causal) {
            lo = 2 * m;
            if (a.sparse && 2 * m >= a.sink_blocks) hi = min(hi, 2 * m + a.window_blocks);
        }
        const int nt = hi - lo + 1;

        const u16* qg = reinterpret_cast<const u16*>(a.q) + ((int64_t)b * a.seq * a.hq + h) * kD;
        const u16* dog = reinterpret_cast<const u16*>(a.d_o) + ((int64_t)b * a.seq * a.hq + h) * kD;
        const float* stg = a.stat + ((int64_t)b * a.hq + h) * nqb * 128;
        auto issue = [&](int t, int slot) {
            const uint32_t base = lds0 + slot * kSlotB;
            load_tile(qg, q_stride, 64 * t, seq - 1, base, wave, lane);
            load_tile(dog, q_stride, 64 * t, seq - 1, base + kTileB, wave, lane);
            if (wave == 0) {
                const u16* sp = uniform_ptr(reinterpret_cast<const u16*>(stg + t * 128));
                load_lds_4(sp, 4u * lane, base + 2 * kTileB);
                load_lds_4(sp, 256u + 4u * lane, base + 2 * kTileB + 256);
            }
        };
        issue(lo, 0);

        // K and V rows of this lane's key as B operands (k-slots = d)
        bf16x8 kreg[kNC], vreg[kNC];
        {
            const int kc = min(key, seq - 1);
            const int64_t off = (((int64_t)b * a.seq + kc) * a.hkv + g) * kD + 8 * hh;
            const u16* kp = reinterpret_cast<const u16*>(a.k) + off;
            const u16* vp = reinterpret_cast<const u16*>(a.v) + off;
#pragma unroll
            for (int c = 0; c < kNC; ++c) {
                kreg[c] = *reinterpret_cast<const bf16x8*>(kp + 16 * c);
                vreg[c] = *reinterpret_cast<const bf16x8*>(vp + 16 * c);
            }
        }

        f32x16 dv[kNM], dk[kNM];
#pragma unroll
        for (int mt = 0; mt < kNM; ++mt) {
            dv[mt] = f32x16{};
            dk[mt] = f32x16{};
        }

        // One tile.  MASK: apply the per-element mask (C < lim, C = query - 64t - 4hh); tiles where no
        // element of the workgroup can be masked skip it.
        auto tile = [&](auto mask_tag, const char* qt, int lim) {
            constexpr bool MASK = decltype(mask_tag)::value;
            const char* dot = qt + kTileB;
            const char* st = qt + 2 * kTileB;
            f32x16 s[2], dp[2];
            float pf[2][16], df[2][16];
            uint32_t ph[4][4], pl[4][4], dh[4][4], dl[4][4];   // [k-step][word]: P and dS, hi and lo
            float4 nl4[2][4], dd4[2][4];

            auto E = [&](int hf, int r) {   // P element
                float p = __builtin_amdgcn_exp2f(fmaf(s[hf][r], c2, comp(nl4[hf][r >> 2], r & 3)));
                if (MASK) p = (32 * hf + 8 * (r >> 2) + (r & 3) < lim) ? 0.0f : p;
                pf[hf][r] = p;
            };
            auto Dd = [&](int hf, int r) { df[hf][r] = pf[hf][r] * (dp[hf][r] - comp(dd4[hf][r >> 2], r & 3)); };
            auto SP = [&](int hf, int pr) {   // pair pr of P half hf -> k-step 2hf + pr/4, word pr%4
                split2(pf[hf][2 * pr], pf[hf][2 * pr + 1], ph[2 * hf + (pr >> 2)][pr & 3], pl[2 * hf + (pr >> 2)][pr & 3]);
            };
            auto SD = [&](int hf, int pr) {
                split2(df[hf][2 * pr], df[hf][2 * pr + 1], dh[2 * hf + (pr >> 2)][pr & 3], dl[2 * hf + (pr >> 2)][pr & 3]);
            };
            auto rowA = [&](int j) -> bf16x8 { return L.row(j < 16 ? qt : dot, (j >> 3) & 1, j & 7); };
            auto trop = [&](int gidx, int which) -> bf16x8 {   // group gidx = 4kk + mt; which 0: dO, 1: Q
                return L.tr(which ? qt : dot, gidx >> 2, gidx & 3);
            };

            // ---- S (steps 0..15) and dP (16..31), operands read 4 steps ahead
            bf16x8 ra[4];
            bf16x8 rc[3][2];   // transposed operands of gradient groups, read 2 groups ahead
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = rowA(j);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const bf16x8 op = ra[j & 3];
                if (j + 4 < 32) ra[j & 3] = rowA(j + 4);
                if (j == 30 || j == 31) {
                    rc[j - 30][0] = trop(j - 30, 0);
                    rc[j - 30][1] = trop(j - 30, 1);
                }
                if (j < 16) {
                    const int hf = j >> 3, c = j & 7;
                    s[hf] = MFMA(op, kreg[c], c ? s[hf] : f32x16{});
                } else {
                    const int hf = (j - 16) >> 3, c = j & 7;
                    dp[hf] = MFMA(op, vreg[c], c ? dp[hf] : f32x16{});
                }
                if (j < 8) {
                    nl4[j >> 2][j & 3] = *reinterpret_cast<const float4*>(st + 4 * (32 * (j >> 2) + 8 * (j & 3) + 4 * hh));
                    dd4[j >> 2][j & 3] =
                        *reinterpret_cast<const float4*>(st + 256 + 4 * (32 * (j >> 2) + 8 * (j & 3) + 4 * hh));
                } else if (j < 16) {
                    E(0, 2 * (j - 8));
                    E(0, 2 * (j - 8) + 1);
                } else if (j < 24) {
                    E(1, 2 * (j - 16));
                    E(1, 2 * (j - 16) + 1);
                    SP(0, j - 16);
                } else {
                    Dd(0, 2 * (j - 24));
                    Dd(0, 2 * (j - 24) + 1);
                    if (j >= 28) SD(0, j - 28);
                }
                __builtin_amdgcn_sched_barrier(0);
            }

            // ---- dV^T += dO^T P and dK^T += Q^T dS: group gi = (kk, mt), operands 2 groups ahead
#pragma unroll
            for (int gi = 0; gi < 16; ++gi) {
                const int kk = gi >> 2, mt = gi & 3;
                const bf16x8 ado = rc[gi % 3][0], aq = rc[gi % 3][1];
                if (gi + 2 < 16) {
                    rc[(gi + 2) % 3][0] = trop(gi + 2, 0);
                    rc[(gi + 2) % 3][1] = trop(gi + 2, 1);
                }
                dv[mt] = MFMA(ado, as_op(ph[kk]), dv[mt]);
                dk[mt] = MFMA(aq, as_op(dh[kk]), dk[mt]);
                dv[mt] = MFMA(ado, as_op(pl[kk]), dv[mt]);
                dk[mt] = MFMA(aq, as_op(dl[kk]), dk[mt]);
                if (gi < 4) {
                    Dd(1, 4 * gi);
                    Dd(1, 4 * gi + 1);
                    Dd(1, 4 * gi + 2);
                    Dd(1, 4 * gi + 3);
                    SD(0, 4 + gi);
                } else if (gi < 12) {
                    SP(1, gi - 4);
                    SD(1, gi - 4);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        int slot = 0;
        for (int i = 0; i < nt; ++i) {
            const int t = lo + i;
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's share of tile t landed
            __syncthreads();                       // tile t complete; every wave is done with tile t-1
            if (i + 1 < nt) issue(t + 1, slot ^ 1);
            const char* qt = smem + slot * kSlotB;
            // masked iff query < key, i.e. C < lim with C = query - 64t - 4hh
            int lim = key - 64 * t - 4 * hh;
            if (!a.causal) lim = -1000;
            else if (a.sparse && kb >= a.sink_blocks && t - kb >= a.window_blocks) lim = 1000;
            // some wave of the workgroup masks something: the diagonal tiles, or a tile the sparse
            // pattern hides from one of the two key blocks
            const bool any_mask = a.causal && (t < 2 * m + 2 ||
                                               (a.sparse && ((2 * m >= a.sink_blocks && t - 2 * m >= a.window_blocks) ||
                                                             (2 * m + 1 >= a.sink_blocks &&
                                                              t - 2 * m - 1 >= a.window_blocks))));
            if (any_mask) tile(Flag<true>{}, qt, lim);
            else tile(Flag<false>{}, qt, lim);
            slot ^= 1;
        }

        // lane holds column key, rows d = 32mt + 8(r/4) + 4hh + r%4
        if (key < seq) {
            float* dkp;
            float* dvp;
            if (G == 1) {
                const int64_t off = (((int64_t)b * a.seq + key) * a.hkv + g) * kD;
                dkp = a.dk + off;
                dvp = a.dv + off;
            } else {
                const int64_t off = (((int64_t)b * a.seq + key) * a.hq + h) * kD;
                dkp = a.dk_part + off;
                dvp = a.dv_part + off;
            }
#pragma unroll
            for (int mt = 0; mt < kNM; ++mt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * mt + 8 * g4 + 4 * hh;
                    *reinterpret_cast<float4*>(dkp + d) =
                        float4{a.scale * dk[mt][4 * g4], a.scale * dk[mt][4 * g4 + 1], a.scale * dk[mt][4 * g4 + 2],
                               a.scale * dk[mt][4 * g4 + 3]};
                    *reinterpret_cast<float4*>(dvp + d) =
                        float4{dv[mt][4 * g4], dv[mt][4 * g4 + 1], dv[mt][4 * g4 + 2], dv[mt][4 * g4 + 3]};
                }
        }
        __syncthreads();   // every wave is done with the slots before the next unit loads into them
        u = queue.next();
    }
}

// ------------------------------------------------------------------ dQ
//
// One 64-key tile for a wave (32 queries) is 64 MFMAs: 32 for S^T and dP^T (K and V rows from LDS,
// Q and dO rows in registers), then 4 groups of 8 for dQ^T (four transposed K operands times dS hi,
// then times dS lo).  The vector work is spread over the MFMA steps as in the dK/dV kernel.
__global__ void __launch_bounds__(kThreads, 1) bwd_dq_kernel(BackwardArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSlots * 2 * kTileB];
    __shared__ int qcell[2];
    Lanes L;
    L.init(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = L.lane, n = L.n, hh = L.hh;

    const int seq = (int)a.seq, nqb = a.n_qblk, G = a.hq / a.hkv;
    const int npair = (nqb + 1) / 2;
    const int bh_total = (int)a.batch * a.hq;
    const int total = npair * bh_total;
    const uint32_t kv_stride = (uint32_t)a.hkv * kD;
    const float c2 = a.scale_log2;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    Queue queue{a.counters + 1, qcell, 0};
    int u = queue.first();
    while (u < total) {
        queue.prefetch();
        const int rank = u / bh_total, bh = u % bh_total;
        const int tp = a.causal ? npair - 1 - rank : rank;   // query-tile pair: causal longest first
        const int b = bh / a.hq, h = bh % a.hq, g = h / G;
        const int qb = 2 * tp + (wave >> 1);                  // this wave's query block
        const int qpos = 128 * tp + 32 * wave + n;            // this lane's query

        // visible key blocks of the pair: [0, e0) then [w0, hi]
        int hi = nqb - 1, e0 = 0, w0 = 0;
        if (a.causal) {
            hi = min(hi, 2 * tp + 1);
            if (a.sparse) {
                e0 = min(a.sink_blocks, hi + 1);
                w0 = max(e0, 2 * tp - a.window_blocks + 1);
            }
        }
        const int nt = e0 + (hi - w0 + 1);

        const u16* kg = reinterpret_cast<const u16*>(a.k) + ((int64_t)b * a.seq * a.hkv + g) * kD;
        const u16* vg = reinterpret_cast<const u16*>(a.v) + ((int64_t)b * a.seq * a.hkv + g) * kD;
        auto kb_of = [&](int i) { return i < e0 ? i : w0 + (i - e0); };
        auto issue = [&](int kb, int slot) {
            const uint32_t base = lds0 + slot * 2 * kTileB;
            load_tile(kg, kv_stride, 64 * kb, seq - 1, base, wave, lane);
            load_tile(vg, kv_stride, 64 * kb, seq - 1, base + kTileB, wave, lane);
        };
        issue(kb_of(0), 0);

        // Q and dO rows of this lane's query as B operands; the row statistics as scalars
        bf16x8 qreg[kNC], doreg[kNC];
        float nl = -INFINITY, dd = 0.0f;
        {
            const int qc = min(qpos, seq - 1);
            const int64_t off = (((int64_t)b * a.seq + qc) * a.hq + h) * kD + 8 * hh;
            const u16* qp = reinterpret_cast<const u16*>(a.q) + off;
            const u16* dop = reinterpret_cast<const u16*>(a.d_o) + off;
#pragma unroll
            for (int c = 0; c < kNC; ++c) {
                qreg[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
                doreg[c] = *reinterpret_cast<const bf16x8*>(dop + 16 * c);
            }
            if (qpos < seq) {
                const float* sp = a.stat + (((int64_t)b * a.hq + h) * nqb + qpos / 64) * 128 + qpos % 64;
                nl = sp[0];
                dd = sp[64];
            }
        }

        f32x16 dq[kNM];
#pragma unroll
        for (int mt = 0; mt < kNM; ++mt) dq[mt] = f32x16{};

        // One tile.  MASK: apply the per-element mask (C > lim, C = key - 64kb - 4hh).
        auto tile = [&](auto mask_tag, const char* kt, int lim) {
            constexpr bool MASK = decltype(mask_tag)::value;
            const char* vt = kt + kTileB;
            f32x16 s[2], dp[2];
            float pf[2][16], df[2][16];
            uint32_t dh[4][4], dl[4][4];

            auto E = [&](int kh, int r) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kh][r], c2, nl));
                if (MASK) p = (32 * kh + 8 * (r >> 2) + (r & 3) > lim) ? 0.0f : p;
                pf[kh][r] = p;
            };
            auto Dd = [&](int kh, int r) { df[kh][r] = pf[kh][r] * (dp[kh][r] - dd); };
            auto SD = [&](int kh, int pr) {
                split2(df[kh][2 * pr], df[kh][2 * pr + 1], dh[2 * kh + (pr >> 2)][pr & 3], dl[2 * kh + (pr >> 2)][pr & 3]);
            };
            auto rowA = [&](int j) -> bf16x8 { return L.row(j < 16 ? kt : vt, (j >> 3) & 1, j & 7); };

            bf16x8 ra[4];
            bf16x8 rc[2][kNM];   // transposed K operands of k-steps kk, kk + 1
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = rowA(j);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const bf16x8 op = ra[j & 3];
                if (j + 4 < 32) ra[j & 3] = rowA(j + 4);
                if (j >= 28) rc[0][j - 28] = L.tr(kt, 0, j - 28);
                if (j < 16) {
                    const int kh = j >> 3, c = j & 7;
                    s[kh] = MFMA(op, qreg[c], c ? s[kh] : f32x16{});
                } else {
                    const int kh = (j - 16) >> 3, c = j & 7;
                    dp[kh] = MFMA(op, doreg[c], c ? dp[kh] : f32x16{});
                }
                if (j >= 8 && j < 16) {
                    E(0, 2 * (j - 8));
                    E(0, 2 * (j - 8) + 1);
                } else if (j >= 16 && j < 24) {
                    E(1, 2 * (j - 16));
                    E(1, 2 * (j - 16) + 1);
                } else if (j >= 24) {
                    Dd(0, 2 * (j - 24));
                    Dd(0, 2 * (j - 24) + 1);
                    if (j >= 28) SD(0, j - 28);
                }
                __builtin_amdgcn_sched_barrier(0);
            }

            // ---- dQ^T += K^T dS^T, k-step kk: 4 operands, times dS hi then dS lo
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int mt = x & 3;
                    const bf16x8 ak = rc[kk & 1][mt];
                    dq[mt] = MFMA(ak, as_op(x < 4 ? dh[kk] : dl[kk]), dq[mt]);
                    if (x >= 4 && kk + 1 < 4) rc[(kk + 1) & 1][x - 4] = L.tr(kt, kk + 1, x - 4);
                    if (kk == 0) {
                        Dd(1, 2 * x);
                        Dd(1, 2 * x + 1);
                        if (x < 4) SD(0, 4 + x);
                    } else if (kk == 1) {
                        SD(1, x);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        int slot = 0;
        for (int i = 0; i < nt; ++i) {
            const int kb = kb_of(i);
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            __syncthreads();
            if (i + 1 < nt) issue(kb_of(i + 1), slot ^ 1);
            const char* kt = smem + slot * 2 * kTileB;
            // masked iff C > lim, C = key - 64kb - 4hh
            int lim = qpos - 64 * kb - 4 * hh;                                     // causal
            if (!a.causal) lim = seq - 1 - 64 * kb - 4 * hh;                       // keys past the end
            else if (a.sparse && kb >= a.sink_blocks && qb - kb >= a.window_blocks) lim = -1000;
            const bool any_mask = a.causal ? (kb >= 2 * tp || (a.sparse && kb >= a.sink_blocks &&
                                                              2 * tp + 1 - kb >= a.window_blocks))
                                           : 64 * (kb + 1) > seq;
            if (any_mask) tile(Flag<true>{}, kt, lim);
            else tile(Flag<false>{}, kt, lim);
            slot ^= 1;
        }

        // lane holds column query, rows d = 32mt + 8(r/4) + 4hh + r%4
        if (qpos < seq) {
            float* dqp = a.dq + (((int64_t)b * a.seq + qpos) * a.hq + h) * kD;
#pragma unroll
            for (int mt = 0; mt < kNM; ++mt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *reinterpret_cast<float4*>(dqp + 32 * mt + 8 * g4 + 4 * hh) =
                        float4{a.scale * dq[mt][4 * g4], a.scale * dq[mt][4 * g4 + 1], a.scale * dq[mt][4 * g4 + 2],
                               a.scale * dq[mt][4 * g4 + 3]};
        }
        __syncthreads();
        u = queue.next();
    }
}

#undef MFMA

// ------------------------------------------------------------------ grouped-query sum
// out[b, s, g, :] = sum over j < G of part[b, s, g*G + j, :], j ascending; blockIdx.y picks dK / dV.
__global__ void __launch_bounds__(256) bwd_group_sum_kernel(BackwardArgs a) {
    const int G = a.hq / a.hkv;
    const float* part = blockIdx.y == 0 ? a.dk_part : a.dv_part;
    float* out = blockIdx.y == 0 ? a.dk : a.dv;
    const int64_t n4 = a.batch * a.seq * a.hkv * (kD / 4);
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const int d4 = (int)(i % (kD / 4));
    const int64_t rg = i / (kD / 4);          // (b, s, g)
    const int g = (int)(rg % a.hkv);
    const int64_t bs = rg / a.hkv;
    const float4* src = reinterpret_cast<const float4*>(part + (bs * a.hq + (int64_t)g * G) * kD) + d4;
    float4 acc = src[0];
    for (int j = 1; j < G; ++j) {
        const float4 x = src[j * (kD / 4)];
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
    }
    reinterpret_cast<float4*>(out)[i] = acc;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
    if (a.head_dim != kD) return hipErrorInvalidValue;
    const int64_t rows = a.batch * (int64_t)a.n_qblk * 64 * a.hq;
    hipLaunchKernelGGL(bwd_rowstat_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
    const int64_t units = ((a.n_qblk + 1) / 2) * a.batch * (int64_t)a.hq;
    const int cu = a.num_cu > 0 ? a.num_cu : 256;
    const unsigned grid = (unsigned)(units < cu ? units : cu);
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    if (a.hq != a.hkv) {
        const int64_t n4 = a.batch * a.seq * a.hkv * (kD / 4);
        hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((n4 + 255) / 256), 2), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace flux
