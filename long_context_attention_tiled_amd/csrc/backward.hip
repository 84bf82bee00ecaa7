// backward.hip -- gradients of tiled attention on gfx950 (bf16 inputs, head_dim 64 or 128, fp32 gradients).
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
//   bwd_absmax_kernel     partial maxima of |x| of Q, K, V, dO per (batch, KV head) over token chunks
//                         (one launch for the four tensors).
//   bwd_convert_kernel    fp16 copies of Q, K, V scaled by 2^-e per (batch, KV head) and tensor, e
//                         chosen from those maxima so the largest magnitude lands in [2^14, 2^15); also
//                         stores dO's e.
//   bwd_rowstat_kernel    D and -LSE*log2(e) per query row, in 64-row tiles (rows past the end get
//                         (-inf, 0), so they weigh nothing), and the fp16 copy of dO; clears the two
//                         work-queue heads.  It also serves the float32 kernels of backward_f32.hip.
//   bwd_dkdv_kernel       one work unit = 128 keys (4 groups of 32) of one KV head with its query heads
//                         taken in turn (a single query head for the sink key pairs of block-sparse
//                         GQA), 8 waves: per key group one wave accumulates dV, one dK; they walk the
//                         64-query tiles that see those keys: S = Q K^T (dV wave, K in registers, keys in lanes;
//                         P goes to the dK wave through LDS) and dP = dO V^T (dK wave, V in
//                         registers), then dV^T += dO^T P or dK^T += Q^T dS with the dO or Q tile
//                         read transposed from LDS.
//   bwd_dq_kernel         one work unit = 128 queries (4 waves x 32) of one query head; walks the
//                         visible 64-key tiles: S^T = K Q^T and dP^T = V dO^T with Q, dO in
//                         registers (queries in lanes), then dQ^T += K^T dS^T.
//   bwd_group_sum_kernel  block-sparse grouped-query attention: adds the per-query-head dK/dV of the
//                         sink keys, in head order, into dK/dV.
// Computing dQ apart from dK/dV rebuilds S and dP once more (7 matrix products instead of 5) but
// needs no atomics: every gradient element is written once, summed in a fixed order.  Both kernels
// write their fp32 gradient rows through a per-wave LDS stage (in their tile slots, after a barrier),
// 256 contiguous bytes of 4 rows per store.
//
// Precision.  Every product runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation.  The bf16 inputs
// convert to fp16 exactly once scaled into fp16's range (a bf16 value has 8 significant bits, fp16
// 11), so S and dP are the bf16 products.  P and dS, which the kernels form in fp32, enter the
// gradient products rounded once to fp16 (relative 2^-12): rounded to bf16 (2^-9) they would put
// errors of ~1e-2 on the dV of sink keys that 2^16 query rows sum into.  Scales, all powers of two:
//   Q16 = Q 2^-eQ, K16 = K 2^-eK, V16 = V 2^-eV, dO16 = dO 2^-eDO   (per batch and KV head)
//   S   = 2^(eQ + eK) (Q16 K16^T),  dP = 2^(eDO + eV) (dO16 V16^T)
//   P16 = P 2^14 (P <= 1, so small probabilities stay normal fp16 numbers)
//   dS16 = dS 2^-eS with eS = 23 + eDO + eV: |dP| <= d * 2^30 * 2^(eDO + eV) <= 2^(37 + eDO + eV) and
//        |dS| <= 2 max|dP|, so |dS16| < 2^15 always; formed as P16 (dP16 2^-37 - D 2^-(37 + eDO + eV))
//   dV = 2^(eDO - 14) sum P16 dO16,  dK = scale 2^(eS + eQ) sum dS16 Q16,  dQ = scale 2^(eS + eK) sum dS16 K16
// Values below 2^-29 of their group's maximum are subnormal in fp16 and may lose bits or be flushed
// (absolute error below 2^-29 of that maximum); likewise probabilities below 2^-28 and dS below 2^-29 of
// its bound.  The scale factors stay within fp32's range as long as the largest |Q| times the largest
// |K| of a KV head, and the largest |dO| times the largest |V|, lie between 2^-90 and 2^150.
//
// Both main kernels are persistent, run two waves per SIMD, and take units from a device counter,
// longest first.  Two LDS slots: the tile in use and the next one in flight.
#include "flux_internal.h"
#include "tile_common.h"

namespace flux {
namespace {

using namespace tile;

constexpr int kStatB = 512;           // a tile's row statistics: 64 x -LSE*log2(e), then 64 x D
constexpr int kSlots = 2;             // the tile in use and the next one in flight
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

// Tile geometry for head dimension D (64 or 128).
template <int D>
struct Geo {
    static constexpr int NC = D / 16;                 // 16-wide d chunks: contraction steps of S and dP
    static constexpr int NM = D / 32;                 // 32-row d tiles of the transposed gradients
    static constexpr int ROW_B = 2 * D;               // bytes of one bf16 row
    static constexpr int CH = ROW_B / 16;             // 16-byte chunks per row
    static constexpr int TILE_B = 64 * ROW_B;         // one 64-row tile
    static constexpr int SLOT_B = 2 * TILE_B + kStatB;
    static constexpr int ROWS_PER_INST = 1024 / ROW_B;  // rows one 1 KB direct load fills
    static constexpr int INSTS_PER_WAVE = TILE_B / 1024 / 4;   // a tile's loads, spread over 4 waves
};

// One chunk swizzle for row reads (16 aligned rows at one logical chunk: 16 distinct 16-byte bank
// groups) and transposing reads (4 aligned rows x 4 aligned chunks).  D = 128 (16 chunks per row):
// swap the two 2-bit halves of row & 15.  D = 64 (8 chunks, two rows per 256 bytes): rows of one
// parity get the 8 values ((r >> 1) & 1) << 2 | ((r >> 2) & 3), and rows 4q, 4q + 2 differ in bit 2.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// 4-byte direct HBM -> LDS load (see load_lds_16, same M0 handling): lane l's dword lands
// at lds_base + 4*l.
__device__ __forceinline__ void load_lds_4(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory");
}

// 64 rows of D bf16 (row r at base + r * row_stride elements, rows past last_row clamped to it) into
// one LDS tile: row r at r * ROW_B, 16-byte chunks swizzled.  TILE_B / 1 KB direct loads, a quarter of
// them from each of the 4 waves `wave` indexes.
template <int D>
__device__ __forceinline__ void load_tile(const u16* base, uint32_t row_stride, int r0, int last_row, uint32_t lds,
                                          int wave, int lane) {
    using Gm = Geo<D>;
    const u16* sb = uniform_ptr(base);
    const int pch = lane % Gm::CH;
#pragma unroll
    for (int i = 0; i < Gm::INSTS_PER_WAVE; ++i) {
        const int inst = wave * Gm::INSTS_PER_WAVE + i;
        const int row = inst * Gm::ROWS_PER_INST + lane / Gm::CH;
        const uint32_t grow = (uint32_t)min(r0 + row, last_row);
        load_lds_16(sb, 2u * (grow * row_stride + 8u * (uint32_t)(pch ^ swz<D>(row))), lds + inst * 1024);
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Lane geometry of the MFMA operands (v_mfma_f32_32x32x16_f16: lane l feeds row/column l % 32 with
// k-slots 8(l/32) .. +7; the accumulator's register r of lane l is row 8(r/4) + 4(l/32) + r%4).
template <int D>
struct Lanes {
    using Gm = Geo<D>;
    int lane, n, hh, jj, dh;
    uint32_t rd[Gm::NC];                // row read: row n, logical chunk 2c + hh (add 32 rows: + 32 * ROW_B)
    uint32_t trl[Gm::NM], trh[Gm::NM];  // transposing reads of k-step 0: rows 4hh + jj/4 (lo) and + 8 (hi)
    __device__ __forceinline__ void init(int l) {
        lane = l;
        n = l & 31;
        hh = l >> 5;
        jj = l & 15;
        dh = (l >> 4) & 1;
#pragma unroll
        for (int c = 0; c < Gm::NC; ++c) rd[c] = n * Gm::ROW_B + 16 * ((2 * c + hh) ^ swz<D>(n));
        const int rlo = 4 * hh + (jj >> 2), rhi = rlo + 8;
#pragma unroll
        for (int mt = 0; mt < Gm::NM; ++mt) {
            const int lch = 4 * mt + 2 * dh + ((jj & 3) >> 1);
            trl[mt] = rlo * Gm::ROW_B + 16 * (lch ^ swz<D>(rlo)) + 8 * (jj & 1);
            trh[mt] = rhi * Gm::ROW_B + 16 * (lch ^ swz<D>(rhi)) + 8 * (jj & 1);
        }
    }
    // A operand X^T[32mt + l%32][16kk + k-slots] of a 64-row tile X (k-slot e of lane half hh is
    // row 16kk + 8(e/4) + 4hh + e%4, matching the accumulator layout of the B operand).
    __device__ __forceinline__ f16x8 tr(const char* tile, int kk, int mt) const {
        const i16x4 lo = read_tr16(tile + kk * 16 * Gm::ROW_B + trl[mt]);
        const i16x4 hi = read_tr16(tile + kk * 16 * Gm::ROW_B + trh[mt]);
        return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // A operand X[32half + l%32][16c + 8(l/32) .. +7] of a 64-row tile X
    __device__ __forceinline__ f16x8 row(const char* tile, int half, int c) const {
        return *reinterpret_cast<const f16x8*>(tile + half * 32 * Gm::ROW_B + rd[c]);
    }
};

// Work queue: thread 0 takes the next unit during the current unit's last step (taking it earlier would
// fix each workgroup's next unit at the start of the current one and undo the balancing of a dynamic
// queue when units are few and long); two LDS cells alternate so that the value read at the end of one
// unit is not overwritten before every thread has read it.
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

// ------------------------------------------------------------------ fp16 copies of the inputs
//
// Tensor t of (Q, K, V, dO) = (0, 1, 2, 3) restricted to one (batch b, KV head g): tokens s in [0, seq),
// heads [h0, h0 + nh) contiguous per token (Q, dO: the G query heads of g; K, V: head g).
struct Slice {
    const u16* src;
    u16* dst;
    int64_t heads;   // heads per token of the tensor
    int64_t off;     // element offset of (b, token 0, h0)
    int run;         // 16-byte vectors per token of the slice
};

// The tensor is a template parameter (each a compile-time instance), so no pointer is picked at run time.
template <int D, int T>
__device__ __forceinline__ Slice slice_of(const BackwardArgs& a, int bg) {
    const int G = a.hq / a.hkv, b = bg / a.hkv, g = bg % a.hkv;
    constexpr bool qside = T == 0 || T == 3;
    Slice sl;
    if constexpr (T == 0) { sl.src = reinterpret_cast<const u16*>(a.q);   sl.dst = reinterpret_cast<u16*>(a.q16); }
    if constexpr (T == 1) { sl.src = reinterpret_cast<const u16*>(a.k);   sl.dst = reinterpret_cast<u16*>(a.k16); }
    if constexpr (T == 2) { sl.src = reinterpret_cast<const u16*>(a.v);   sl.dst = reinterpret_cast<u16*>(a.v16); }
    if constexpr (T == 3) { sl.src = reinterpret_cast<const u16*>(a.d_o); sl.dst = reinterpret_cast<u16*>(a.do16); }
    sl.heads = qside ? a.hq : a.hkv;
    sl.off = ((int64_t)b * a.seq * sl.heads + (qside ? (int64_t)g * G : g)) * D;
    sl.run = (qside ? G : 1) * (D / 8);
    return sl;
}

__device__ __forceinline__ uint32_t absmax_bits(uint4 x) {   // largest |x| of 8 bf16 as its bit pattern
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
    return m;
}

// e with max * 2^-e in [2^14, 2^15) for the bf16 bit pattern of the maximum (0 for an all-zero slice)
__device__ __forceinline__ int scale_exp(uint32_t m) {
    if (m == 0) return 0;
    const int E = (int)((m >> 7) & 0xffu);
    return (E > 1 ? E : 1) - 141;
}

// One 16-byte vector of 8 bf16 as 8 fp16 of x 2^-e (round to nearest even), element order kept.
__device__ __forceinline__ uint4 to_f16_scaled(uint4 x, int e) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        y[q] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)ldexpf(bf16_lo(w[q]), -e), (_Float16)ldexpf(bf16_hi(w[q]), -e)});
    return uint4{y[0], y[1], y[2], y[3]};
}

// Vector i of a slice (16 bytes, 8 elements): token i / run, vector i % run of that token.  A slice holds
// at most seq * hq * d / 8 < 2^28 vectors, so 32-bit indices suffice.
__device__ __forceinline__ int64_t vec_off(const Slice& sl, uint32_t i, int d) {
    const uint32_t s = i / (uint32_t)sl.run, r = i - s * (uint32_t)sl.run;
    return sl.off + (int64_t)s * sl.heads * d + 8 * r;
}

// Maximum over the 256 threads of a block (4 waves).
__device__ __forceinline__ uint32_t block_max(uint32_t m) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    __shared__ uint32_t wm[4];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    return max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

// Block (c, bg) of tensor T reduces the vectors of tokens [c seq / chunks, (c + 1) seq / chunks) of its
// slice, four independent 16-byte loads in flight per thread.
template <int D, int T>
__device__ __forceinline__ void absmax_slice(const BackwardArgs& a, int c, int bg) {
    const Slice sl = slice_of<D, T>(a, bg);
    const uint32_t n0 = (uint32_t)(a.seq * c / kAbsmaxChunks) * sl.run;
    const uint32_t n1 = (uint32_t)(a.seq * (c + 1) / kAbsmaxChunks) * sl.run;
    uint32_t m = 0;
    for (uint32_t i = n0 + threadIdx.x; i < n1; i += 4 * 256) {
        uint4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[j] = i + 256 * j < n1 ? *reinterpret_cast<const uint4*>(sl.src + vec_off(sl, i + 256 * j, D))
                                    : uint4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, absmax_bits(x[j]));
    }
    m = block_max(m);
    if (threadIdx.x == 0) a.amax[((int64_t)T * gridDim.y + bg) * kAbsmaxChunks + c] = m;
}

// grid (kAbsmaxChunks, B * Hkv, 4): blockIdx.z is the tensor (Q, K, V, dO), each case its own
// compile-time instance, so no tensor pointer is picked by a run-time index.
template <int D>
__global__ void __launch_bounds__(256) bwd_absmax_kernel(BackwardArgs a) {
    const int c = blockIdx.x, bg = blockIdx.y;
    switch (blockIdx.z) {
        case 0: absmax_slice<D, 0>(a, c, bg); break;
        case 1: absmax_slice<D, 1>(a, c, bg); break;
        case 2: absmax_slice<D, 2>(a, c, bg); break;
        default: absmax_slice<D, 3>(a, c, bg); break;
    }
}

// The scale exponent of tensor T for (batch, KV head) bg from its chunk maxima (every thread gets it).
template <int T>
__device__ __forceinline__ int slice_exp(const BackwardArgs& a, int bg) {
    static_assert(kAbsmaxChunks <= 256, "one chunk maximum per thread");
    return scale_exp(block_max(threadIdx.x < kAbsmaxChunks
                                   ? a.amax[((int64_t)T * gridDim.y + bg) * kAbsmaxChunks + threadIdx.x]
                                   : 0u));
}

// Converts block (c, bg)'s tokens of tensor T (Q, K or V) to fp16 scaled by 2^-e.
template <int D, int T>
__device__ __forceinline__ void convert_slice(const BackwardArgs& a, int c, int bg) {
    const Slice sl = slice_of<D, T>(a, bg);
    const int e = slice_exp<T>(a, bg);
    if (c == 0 && threadIdx.x == 0) a.exps[T * gridDim.y + bg] = e;
    const uint32_t n0 = (uint32_t)(a.seq * c / kAbsmaxChunks) * sl.run;
    const uint32_t n1 = (uint32_t)(a.seq * (c + 1) / kAbsmaxChunks) * sl.run;
    for (uint32_t i = n0 + threadIdx.x; i < n1; i += 4 * 256) {
        uint4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + 256 * j < n1) x[j] = *reinterpret_cast<const uint4*>(sl.src + vec_off(sl, i + 256 * j, D));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i + 256 * j >= n1) break;
            *reinterpret_cast<uint4*>(sl.dst + vec_off(sl, i + 256 * j, D)) = to_f16_scaled(x[j], e);
        }
    }
}

// Same grid: Q, K and V are converted here; dO is converted by the row statistics kernel, which reads it
// anyway, so the blocks of z = 3 only store dO's exponent.
template <int D>
__global__ void __launch_bounds__(256) bwd_convert_kernel(BackwardArgs a) {
    const int c = blockIdx.x, bg = blockIdx.y;
    switch (blockIdx.z) {
        case 0: convert_slice<D, 0>(a, c, bg); break;
        case 1: convert_slice<D, 1>(a, c, bg); break;
        case 2: convert_slice<D, 2>(a, c, bg); break;
        default:
            if (c == 0) {
                const int e = slice_exp<3>(a, bg);
                if (threadIdx.x == 0) a.exps[3 * gridDim.y + bg] = e;
            }
            break;
    }
}

// ------------------------------------------------------------------ row statistics
//
// bf16 inputs (the fp16 matrix-core kernels): the row statistics are stored pre-scaled for them,
// -LSE*log2(e) + 14 (P16 = P 2^14) and D 2^-(37 + eDO + eV) (so dS16 = P16 (dP16 2^-37 - D')), and the
// kernel writes the fp16 copy of dO, which it reads for D anyway.
template <int D>
__global__ void __launch_bounds__(256) bwd_rowstat_kernel(BackwardArgs a) {
    constexpr int LPR = D / 8;            // lanes per row, 8 elements (16 bytes) each
    constexpr int RPB = 256 / LPR;        // rows per block
    if (blockIdx.x == 0 && threadIdx.x < 2) a.counters[threadIdx.x] = 0;
    const int padded = a.n_qblk * 64;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    if (row >= a.batch * padded * a.hq) return;   // all lanes of a row leave together
    const int h = (int)(row % a.hq);
    const int64_t rest = row / a.hq;
    const int i = (int)(rest % padded);
    const int64_t b = rest / padded;
    float acc = 0.0f;
    if (i < a.seq) {
        const int64_t off = ((b * a.seq + i) * a.hq + h) * D + 8 * c;
        float gv[8];
        if (a.in_f32) {
            const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.d_o) + off);
            const float4 y = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.d_o) + off + 4);
            gv[0] = x.x; gv[1] = x.y; gv[2] = x.z; gv[3] = x.w; gv[4] = y.x; gv[5] = y.y; gv[6] = y.z; gv[7] = y.w;
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(a.d_o) + off);
            gv[0] = bf16_lo(x.x); gv[1] = bf16_hi(x.x); gv[2] = bf16_lo(x.y); gv[3] = bf16_hi(x.y);
            gv[4] = bf16_lo(x.z); gv[5] = bf16_hi(x.z); gv[6] = bf16_lo(x.w); gv[7] = bf16_hi(x.w);
            // the fp16 copy of dO (the matrix-core kernels' operand) from the same load
            const int bg = (int)b * a.hkv + h / (a.hq / a.hkv), nbg = (int)a.batch * a.hkv;
            *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(a.do16) + off) = to_f16_scaled(x, a.exps[3 * nbg + bg]);
        }
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
        acc = o[0] * gv[0] + o[1] * gv[1];
        acc += o[2] * gv[2] + o[3] * gv[3];
        acc += o[4] * gv[4] + o[5] * gv[5];
        acc += o[6] * gv[6] + o[7] * gv[7];
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, LPR);
    if (c == 0) {
        float* st = a.stat + ((b * a.hq + h) * a.n_qblk + i / 64) * 128 + i % 64;
        const bool live = i < a.seq;
        float nl = live ? -a.lse[(b * a.hq + h) * a.seq + i] * kLog2e : -INFINITY;
        if (!a.in_f32) {
            const int bg = (int)b * a.hkv + h / (a.hq / a.hkv), nbg = (int)a.batch * a.hkv;
            nl += 14.0f;
            acc = ldexpf(acc, -(37 + a.exps[3 * nbg + bg] + a.exps[2 * nbg + bg]));
        }
        st[0] = nl;
        st[64] = live ? acc : 0.0f;
    }
}

// 16 accumulator values of one 32x32 block -> fp16 operands (round to nearest even) of its two 16-wide
// k-steps (element 2i in the low half of word i)
__device__ __forceinline__ void to_f16(const float* x, f16x8* y) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        uint32_t h[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            h[w] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)x[8 * q + 2 * w], (_Float16)x[8 * q + 2 * w + 1]});
        y[q] = __builtin_bit_cast(f16x8, u32x4{h[0], h[1], h[2], h[3]});
    }
}

__device__ __forceinline__ float comp(const float4& v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_f16((a), (b), (c), 0, 0, 0)

// NS MFMA steps whose A operands come from LDS: operand(i) is read kAhead steps before step(i, op)
// uses it, and sched_barrier keeps that order (left alone, the scheduler reuses one register and
// waits for each read right before its MFMA).
constexpr int kAhead = 3;
template <int NS, typename Operand, typename Step>
__device__ __forceinline__ void mfma_seq(Operand operand, Step step) {
    __builtin_amdgcn_s_setprio(1);   // the other wave of the SIMD fills the MFMA shadow with its vector work
    f16x8 ring[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
        if (i < NS) ring[i] = operand(i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const f16x8 op = ring[i % kAhead];
        if (i + kAhead < NS) ring[i % kAhead] = operand(i + kAhead);
        step(i, op);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
}

// acc[mt] += X^T[mt, k-steps kk0, kk0 + 1] * x16: the transposed operand of (kk0 + 1, mt) is read into
// the register the MFMA of (kk0, mt) frees.
template <int D>
__device__ __forceinline__ void grad_product(const Lanes<D>& L, const char* xt, int kk0, const f16x8* x16,
                                             f32x16* acc) {
    constexpr int kNM = Geo<D>::NM;
    __builtin_amdgcn_s_setprio(1);
    f16x8 ax[kNM];
#pragma unroll
    for (int mt = 0; mt < kNM; ++mt) ax[mt] = L.tr(xt, kk0, mt);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int mt = 0; mt < kNM; ++mt) {
            acc[mt] = MFMA(ax[mt], x16[q], acc[mt]);
            if (q == 0) ax[mt] = L.tr(xt, kk0 + 1, mt);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// Epilogue store of the fp32 gradient rows a wave holds in the transposed accumulator layout (lane l: row
// l % 32 of the wave's 32 rows; acc[mt][4 g4 + e] is d = 32 mt + 8 g4 + 4 (l / 32) + e), each value
// f * acc * 2^ex, through the wave's own LDS stage: 64 d values (256 bytes) of every row at a time, rows
// padded to 272 bytes so that the 16-byte writes and reads both spread over the banks.  Each store then
// writes 256 contiguous bytes of each of 4 rows, where the accumulator layout gives 16 bytes of each of
// 32 rows.  One v_permlane32_swap per dword gives every lane 32 contiguous bytes of its row for the stage
// writes.  dst(r) is row r's destination, nullptr for a row not stored.  Every lane of the wave takes
// part; the caller has made the stage memory free for the whole workgroup.
constexpr int kStageRowB = 256 + 16;
template <int D, typename Dst>
__device__ __forceinline__ void store_rows_staged(const f32x16* acc, float f, int ex, char* stage, int lane,
                                                  Dst dst) {
    constexpr int kNM = Geo<D>::NM;
    const int n = lane & 31, hh = lane >> 5;
    const int c = lane & 15, r0 = lane >> 4;
#pragma unroll
    for (int p = 0; p < kNM / 2; ++p) {   // d values 64p .. 64p + 63
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // lane half 0 gets its own then its partner's 4 values of g4 = 2j, half 1 its partner's
                // then its own of g4 = 2j + 1: d = 32 (2p + m) + 16j + 8hh .. + 7 either way
                const f32x16& x = acc[2 * p + m];
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ldexpf(f * x[8 * j + k], ex)),
                                                                     __float_as_uint(ldexpf(f * x[8 * j + 4 + k], ex)),
                                                                     false, false);
                    lo[k] = sw[0];
                    hi[k] = sw[1];
                }
                char* sp = stage + n * kStageRowB + 128 * m + 64 * j + 32 * hh;
                *reinterpret_cast<uint4*>(sp) = uint4{lo[0], lo[1], lo[2], lo[3]};
                *reinterpret_cast<uint4*>(sp + 16) = uint4{hi[0], hi[1], hi[2], hi[3]};
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the stage writes done
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + r0;
            const uint4 v = *reinterpret_cast<const uint4*>(stage + r * kStageRowB + 16 * c);
            float* d = dst(r);
            if (d) *reinterpret_cast<uint4*>(d + 64 * p + 4 * c) = v;
            __builtin_amdgcn_sched_barrier(0);   // one read, one store: no stage registers held
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the stage reads done before it is written again
    }
}

// Key pairs (128 keys) that hold sink blocks when the pattern is block-sparse and query heads are grouped:
// every query sees them, so they are split by query head (one unit per head, partial dK/dV summed by
// bwd_group_sum_kernel) rather than taking a KV head's G heads in one unit, which would make them the
// longest units by a factor of G.
__host__ __device__ __forceinline__ int dkdv_sink_pairs(const BackwardArgs& a) {
    if (!a.sparse || !a.causal || a.hq == a.hkv) return 0;
    const int npk = (a.n_qblk + 1) / 2;
    const int sp = (a.sink_blocks + 1) / 2;
    return sp < npk ? sp : npk;
}

// ------------------------------------------------------------------ dK, dV
//
// 8 waves, two per SIMD, on 128 keys: waves w and w + 4 own the same 32 keys; wave w accumulates
// dV^T, wave w + 4 dK^T.  Each takes a 64-query tile in two 32-query halves: wave w computes S (D/16
// MFMAs) and P and hands P to wave w + 4 through LDS, which meanwhile computes dP (as many MFMAs) and
// then dS; each runs the 2 * D/32 MFMAs of its gradient product, the dK wave one half late (at the start
// of the next half, before its dP), so that the matrix core has the dK wave's product to run while the
// dV wave computes exp2.  At D = 128 that is 32 + 32 MFMAs per SIMD and tile, S is computed once per
// key group, and the two roles are compiled as separate code paths (191 registers at D = 128).
constexpr int kKvWaves = 8;
// Q/dO tile slots of the dK/dV pass: the tile in use, the next one in flight, and the previous one, whose
// Q the dK waves still read during the current tile's first half (their gradient product runs one half late).
constexpr int kKvSlots = 3;
template <int D>
__global__ void __launch_bounds__(64 * kKvWaves, 2) bwd_dkdv_kernel(BackwardArgs a) {
    using Gm = Geo<D>;
    constexpr int kNC = Gm::NC, kNM = Gm::NM, kTileB = Gm::TILE_B, kSlotB = Gm::SLOT_B;
    // the Q/dO tile slots, which also hold the epilogue's output stage
    constexpr int kSmemB = kKvSlots * kSlotB > kKvWaves * 32 * kStageRowB ? kKvSlots * kSlotB : kKvWaves * 32 * kStageRowB;
    __shared__ __attribute__((aligned(1024))) char smem[kSmemB];
    // P of one 32-query half, handed from the dV wave to the dK wave of each key group: two halves in
    // flight, [parity][key group][accumulator quad][lane] (lane-contiguous float4: conflict-free)
    __shared__ float4 pbuf[2][4][4][64];
    __shared__ int qcell[2];
    Lanes<D> L;
    L.init(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = L.lane, n = L.n, hh = L.hh;
    const int ks = wave & 3;          // 32-key group
    const bool is_dk = wave >= 4;     // role: dK (true) or dV (false)
    int par = 0;                      // parity of the P buffer of the next half

    const int seq = (int)a.seq, nqb = a.n_qblk, G = a.hq / a.hkv;
    const int bh_total = (int)a.batch * a.hq, bg_total = (int)a.batch * a.hkv;
    const int n_sp = dkdv_sink_pairs(a);
    const int ph_units = n_sp * bh_total;
    const int total = ph_units + ((nqb + 1) / 2 - n_sp) * bg_total;
    const uint32_t q_stride = (uint32_t)a.hq * D;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    Queue queue{a.counters + 0, qcell, 0};
    int u = queue.first();
    while (u < total) {
        // Units, longest query range first: a key pair holding sink blocks (every query sees it) with one
        // query head, its dK/dV going to per-head partials; any other key pair with all G query heads of
        // one KV head in turn, summed in registers in head order and written to dK/dV directly.
        int m, b, h0, nh;
        if (u < ph_units) {
            m = u / bh_total;
            const int bh = u % bh_total;
            b = bh / a.hq;
            h0 = bh % a.hq;
            nh = 1;
        } else {
            const int v = u - ph_units;
            m = n_sp + v / bg_total;
            const int bg = v % bg_total;
            b = bg / a.hkv;
            h0 = (bg % a.hkv) * G;
            nh = G;
        }
        const bool partial = nh < G;
        const int g = h0 / G;
        const int bg = b * a.hkv + g;
        const int eQ = a.exps[bg], eK = a.exps[bg_total + bg], eV = a.exps[2 * bg_total + bg];
        const int eDO = a.exps[3 * bg_total + bg];
        const float c2 = ldexpf(a.scale_log2, eQ + eK);   // exp2 argument per unit of Q16 K16^T
        const int kb = 2 * m + (ks >> 1);                 // this wave's key block
        const int key = 128 * m + 32 * ks + n;            // this lane's key
        int lo = 0, hi = nqb - 1;
        if (a.causal) {
            lo = 2 * m;
            if (a.sparse && 2 * m >= a.sink_blocks) hi = min(hi, 2 * m + a.window_blocks);
        }
        const int nt = hi - lo + 1;
        const int nsteps = nh * nt;   // the unit's steps: its heads in order, each over tiles lo .. hi

        // a tile is 32 loads of 1 KB (Q by waves 0-3, dO by waves 4-7) plus 2 of row statistics
        auto issue = [&](int h, int t, int slot) {
            const u16* qg = reinterpret_cast<const u16*>(a.q16) + ((int64_t)b * a.seq * a.hq + h) * D;
            const u16* dog = reinterpret_cast<const u16*>(a.do16) + ((int64_t)b * a.seq * a.hq + h) * D;
            const float* stg = a.stat + ((int64_t)b * a.hq + h) * nqb * 128;
            const uint32_t base = lds0 + slot * kSlotB;
            if (wave < 4) load_tile<D>(qg, q_stride, 64 * t, seq - 1, base, wave, lane);
            else load_tile<D>(dog, q_stride, 64 * t, seq - 1, base + kTileB, wave - 4, lane);
            if (wave == 0) {
                const u16* sp = uniform_ptr(reinterpret_cast<const u16*>(stg + t * 128));
                load_lds_4(sp, 4u * lane, base + 2 * kTileB);
                load_lds_4(sp, 256u + 4u * lane, base + 2 * kTileB + 256);
            }
        };
        issue(h0, lo, 0);

        // The rest of the unit, compiled once per role (dV: DK false, dK: DK true), so that each role's
        // registers are allocated for its own code path.
        auto role_body = [&](auto dk_tag) {
            constexpr bool DK = decltype(dk_tag)::value;
            // this lane's key row as the B operand (k-slots = d): K for the dV wave (S = Q K^T), V for the
            // dK wave (dP = dO V^T)
            f16x8 breg[kNC];
            {
                const int kc = min(key, seq - 1);
                const int64_t off = (((int64_t)b * a.seq + kc) * a.hkv + g) * D + 8 * hh;
                const u16* bp = reinterpret_cast<const u16*>(DK ? a.v16 : a.k16) + off;
#pragma unroll
                for (int c = 0; c < kNC; ++c) breg[c] = *reinterpret_cast<const f16x8*>(bp + 16 * c);
            }

            f32x16 acc[kNM];   // dV^T or dK^T: lane = key, rows d = 32mt + 8(r/4) + 4hh + r%4
#pragma unroll
            for (int mt = 0; mt < kNM; ++mt) acc[mt] = f32x16{};
            // dK wave: dS16 of the previous half, whose gradient product runs at the start of the next half
            // (beside the dV wave's S and exp2 rather than after the dV wave's product), with its Q tile
            f16x8 dk_pend[2];
            const char* pend_xt = smem;   // the Q tile of a pending second half
            bool pend = false;            // a second half is pending (from the previous tile)

            // One tile, in two 32-query halves.  The dV wave computes S, P16 = P 2^14 (exp2 of the scaled
            // score minus the row's LSE, plus 14; zero where masked) and publishes it in LDS; the dK wave
            // computes dP meanwhile, and after the barrier forms dS16 = P16 (dP16 2^-37 - D') from the
            // published P16.  Then the dV wave runs its gradient product beside the dK wave's dS; the dK
            // wave's product of that half runs at the start of the next half, beside the dV wave's S and
            // exp2 (the unit's last one after its last tile).  Elements with C < lim are masked
            // (C = query - 64t - 4hh).
            auto tile = [&](const char* qt, int lim, bool need_mask) {
                const char* dot = qt + kTileB;
                const char* st = qt + 2 * kTileB;
                const char* xt = DK ? qt : dot;   // tile read transposed for the gradient product
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    if constexpr (DK) {
                        if (hf == 1) grad_product(L, xt, 0, dk_pend, acc);   // this tile's first half
                        else if (pend) grad_product(L, pend_xt, 2, dk_pend, acc);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    f32x16 sd = f32x16{};   // S (dV wave) or dP (dK wave)
                    mfma_seq<kNC>([&](int i) { return L.row(DK ? dot : qt, hf, i); },
                                  [&](int i, f16x8 op) { sd = MFMA(op, breg[i], sd); });
                    float x[16];   // P16, then dS16 for the dK wave
                    if constexpr (!DK) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const float4 nl = *reinterpret_cast<const float4*>(st + 4 * (32 * hf + 8 * g4 + 4 * hh));
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                x[4 * g4 + e] = __builtin_amdgcn_exp2f(fmaf(sd[4 * g4 + e], c2, comp(nl, e)));
                        }
                        if (need_mask) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) x[r] = (32 * hf + 8 * (r >> 2) + (r & 3) < lim) ? 0.0f : x[r];
                        }
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
                            pbuf[par][ks][g4][lane] = float4{x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]};
                    }
                    __syncthreads();   // P of this half published
                    if constexpr (DK) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const float4 p = pbuf[par][ks][g4][lane];
                            const float4 dd = *reinterpret_cast<const float4*>(st + 256 + 4 * (32 * hf + 8 * g4 + 4 * hh));
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                x[4 * g4 + e] = comp(p, e) * fmaf(sd[4 * g4 + e], 0x1p-37f, -comp(dd, e));
                        }
                    }
                    par ^= 1;
                    if constexpr (!DK) {
                        f16x8 x16[2];
                        to_f16(x, x16);
                        grad_product(L, xt, 2 * hf, x16, acc);
                    } else {
                        to_f16(x, dk_pend);
                        if (hf == 1) {
                            pend_xt = xt;
                            pend = true;
                        }
                    }
                }
            };

            int slot = 0, t = lo, h = h0;
            for (int i = 0; i < nsteps; ++i) {
                const int t_next = t < hi ? t + 1 : lo, h_next = t < hi ? h : h + 1;
                const int slot_next = slot == kKvSlots - 1 ? 0 : slot + 1;
                __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's share of tile t landed
                __syncthreads();   // tile t complete; every wave is done with tile t-2 (the dK waves with t-1)
                if (i + 1 < nsteps) issue(h_next, t_next, slot_next);
                else queue.prefetch();   // the next unit is taken when this one ends (keeps the queue dynamic)
                const char* qt = smem + slot * kSlotB;
                // masked iff query < key, i.e. C < lim with C = query - 64t - 4hh
                int lim = key - 64 * t - 4 * hh;
                if (!a.causal) lim = -1000;
                else if (a.sparse && kb >= a.sink_blocks && t - kb >= a.window_blocks) lim = 1000;
                // this wave masks something only on its diagonal tile, on tiles before it, and on tiles the
                // sparse pattern hides from its key block
                const bool need_mask = a.causal && (t <= kb || lim == 1000);
                tile(qt, lim, need_mask);
                slot = slot_next;
                t = t_next;
                h = h_next;
            }
            if constexpr (DK)
                if (pend) grad_product(L, pend_xt, 2, dk_pend, acc);   // the unit's last half

            // lane holds column key, rows d = 32mt + 8(r/4) + 4hh + r%4
            __syncthreads();   // every wave is done with the tile slots: they hold the output stage now
            {
                // dK = scale 2^(eS + eQ) acc with eS = 23 + eDO + eV; dV = 2^(eDO - 14) acc
                const float f = DK ? a.scale : 1.0f;
                const int ex = DK ? 23 + eDO + eV + eQ : eDO - 14;
                const int key0 = 128 * m + 32 * ks;
                int ln = lane;
                asm volatile("" : "+v"(ln));   // stage addresses formed here, not hoisted out of the unit loop
                store_rows_staged<D>(acc, f, ex, smem + wave * 32 * kStageRowB, ln, [&](int r) -> float* {
                    const int k = key0 + r;
                    if (k >= seq) return nullptr;
                    if (!partial) return (DK ? a.dk : a.dv) + (((int64_t)b * a.seq + k) * a.hkv + g) * D;
                    return (DK ? a.dk_part : a.dv_part) + (((int64_t)b * a.part_keys + k) * a.hq + h0) * D;
                });
            }
        };
        if (is_dk) role_body(BoolTag<true>{});
        else role_body(BoolTag<false>{});
        __syncthreads();   // every wave is done with the slots before the next unit loads into them
        u = queue.next();
    }
}

// ------------------------------------------------------------------ dQ
//
// 4 waves of 32 queries, two workgroups per CU (two waves per SIMD).  A 64-key tile is taken in two
// 32-key halves: S^T and dP^T (D/8 MFMAs, K and V rows from LDS, Q and dO rows in registers), the
// vector work, then 2 * D/32 MFMAs of dQ^T += K^T dS^T; the first half's product runs after the second
// half's S^T and dP^T, beside its vector work (0.8% faster than in order).
template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_kernel(BackwardArgs a) {
    using Gm = Geo<D>;
    constexpr int kNC = Gm::NC, kNM = Gm::NM, kTileB = Gm::TILE_B;
    // the K/V tile slots, which also hold the epilogue's output stage
    constexpr int kSmemB = kSlots * 2 * kTileB > 4 * 32 * kStageRowB ? kSlots * 2 * kTileB : 4 * 32 * kStageRowB;
    __shared__ __attribute__((aligned(1024))) char smem[kSmemB];
    __shared__ int qcell[2];
    Lanes<D> L;
    L.init(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = L.lane, n = L.n, hh = L.hh;

    const int seq = (int)a.seq, nqb = a.n_qblk, G = a.hq / a.hkv;
    const int npair = (nqb + 1) / 2;
    const int bh_total = (int)a.batch * a.hq;
    const int total = npair * bh_total;
    const uint32_t kv_stride = (uint32_t)a.hkv * D;
    const int bg_total = (int)a.batch * a.hkv;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    Queue queue{a.counters + 1, qcell, 0};
    int u = queue.first();
    while (u < total) {
        const int rank = u / bh_total, bh = u % bh_total;
        const int tp = a.causal ? npair - 1 - rank : rank;   // query-tile pair: causal longest first
        const int b = bh / a.hq, h = bh % a.hq, g = h / G;
        const int bg = b * a.hkv + g;
        const int eQ = a.exps[bg], eK = a.exps[bg_total + bg], eV = a.exps[2 * bg_total + bg];
        const int eDO = a.exps[3 * bg_total + bg];
        const float c2 = ldexpf(a.scale_log2, eQ + eK);   // exp2 argument per unit of K16 Q16^T
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

        const u16* kg = reinterpret_cast<const u16*>(a.k16) + ((int64_t)b * a.seq * a.hkv + g) * D;
        const u16* vg = reinterpret_cast<const u16*>(a.v16) + ((int64_t)b * a.seq * a.hkv + g) * D;
        auto kb_of = [&](int i) { return i < e0 ? i : w0 + (i - e0); };
        auto issue = [&](int kb, int slot) {
            const uint32_t base = lds0 + slot * 2 * kTileB;
            load_tile<D>(kg, kv_stride, 64 * kb, seq - 1, base, wave, lane);
            load_tile<D>(vg, kv_stride, 64 * kb, seq - 1, base + kTileB, wave, lane);
        };
        issue(kb_of(0), 0);

        // Q and dO rows of this lane's query as B operands; the row statistics as scalars
        f16x8 qreg[kNC], doreg[kNC];
        float nl = -INFINITY, dd = 0.0f;
        {
            const int qc = min(qpos, seq - 1);
            const int64_t off = (((int64_t)b * a.seq + qc) * a.hq + h) * D + 8 * hh;
            const u16* qp = reinterpret_cast<const u16*>(a.q16) + off;
            const u16* dop = reinterpret_cast<const u16*>(a.do16) + off;
#pragma unroll
            for (int c = 0; c < kNC; ++c) {
                qreg[c] = *reinterpret_cast<const f16x8*>(qp + 16 * c);
                doreg[c] = *reinterpret_cast<const f16x8*>(dop + 16 * c);
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

        // One tile: elements with C > lim are masked (C = key - 64kb - 4hh).  One body for masked and
        // unmasked tiles (the mask is a short branch): two bodies would cost registers and spill.
        auto tile = [&](const char* kt, int lim, bool need_mask) {
            const char* vt = kt + kTileB;
            f16x8 pend16[2];   // dS16 of the first half: its product runs beside the second half's vector work
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                // S^T = K Q^T, dP^T = V dO^T: lane = query n, registers = keys 32kh + 8(r/4) + 4hh + r%4
                f32x16 s = f32x16{}, dp = f32x16{};
                mfma_seq<2 * kNC>([&](int i) { return L.row(i < kNC ? kt : vt, kh, i % kNC); }, [&](int i, f16x8 op) {
                    if (i < kNC) s = MFMA(op, qreg[i], s);
                    else dp = MFMA(op, doreg[i - kNC], dp);
                });
                if (kh == 1) grad_product(L, kt, 0, pend16, dq);
                float x[16];   // P16 = P 2^14, then dS16 = P16 (dP16 2^-37 - D')
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, nl));
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[r] = (32 * kh + 8 * (r >> 2) + (r & 3) > lim) ? 0.0f : x[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] *= fmaf(dp[r], 0x1p-37f, -dd);
                if (kh == 0) {
                    to_f16(x, pend16);
                } else {
                    f16x8 x16[2];
                    to_f16(x, x16);
                    grad_product(L, kt, 2, x16, dq);   // dQ^T += K^T dS16^T
                }
            }
        };

        int slot = 0;
        for (int i = 0; i < nt; ++i) {
            const int kb = kb_of(i);
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            __syncthreads();
            if (i + 1 < nt) issue(kb_of(i + 1), slot ^ 1);
            else queue.prefetch();   // the next unit is taken when this one ends (keeps the queue dynamic)
            const char* kt = smem + slot * 2 * kTileB;
            // masked iff C > lim, C = key - 64kb - 4hh
            int lim = qpos - 64 * kb - 4 * hh;                                     // causal
            if (!a.causal) lim = seq - 1 - 64 * kb - 4 * hh;                       // keys past the end
            else if (a.sparse && kb >= a.sink_blocks && qb - kb >= a.window_blocks) lim = -1000;
            // this wave masks something only on its diagonal tile, on tiles after it, on tiles the
            // sparse pattern hides from its query block, and (all keys visible) on a ragged last tile
            const bool need_mask = a.causal ? (kb >= qb || lim == -1000) : 64 * (kb + 1) > seq;
            tile(kt, lim, need_mask);
            slot ^= 1;
        }

        // lane holds column query, rows d = 32mt + 8(r/4) + 4hh + r%4
        __syncthreads();   // every wave is done with the K/V slots: they hold the output stage now
        {
            const int ex = 23 + eDO + eV + eK;   // dQ = scale 2^(eS + eK) acc
            const int q0 = 128 * tp + 32 * wave;
            int ln = lane;
            asm volatile("" : "+v"(ln));   // stage addresses formed here, not hoisted out of the unit loop
            store_rows_staged<D>(dq, a.scale, ex, smem + wave * 32 * kStageRowB, ln, [&](int r) -> float* {
                const int q = q0 + r;
                return q < seq ? a.dq + (((int64_t)b * a.seq + q) * a.hq + h) * D : nullptr;
            });
        }
        __syncthreads();
        u = queue.next();
    }
}

#undef MFMA


// ------------------------------------------------------------------ grouped-query sum
// out[b, s, g, :] = sum over j < G of part[b, s, g*G + j, :], j ascending, for the keys s < part_keys of
// the per-head units (the sink key pairs); blockIdx.y picks dK / dV.
template <int D>
__global__ void __launch_bounds__(256) bwd_group_sum_kernel(BackwardArgs a) {
    const int G = a.hq / a.hkv;
    const int64_t nkeys = a.part_keys;
    const float* part = blockIdx.y == 0 ? a.dk_part : a.dv_part;
    float* out = blockIdx.y == 0 ? a.dk : a.dv;
    const int64_t n4 = a.batch * nkeys * a.hkv * (D / 4);
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const int d4 = (int)(i % (D / 4));
    const int64_t rg = i / (D / 4);          // (b, s, g), s < nkeys
    const int g = (int)(rg % a.hkv);
    const int64_t bk = rg / a.hkv;           // b * nkeys + s
    const int64_t bs = (bk / nkeys) * a.seq + bk % nkeys;
    const float4* src = reinterpret_cast<const float4*>(part + (bk * a.hq + (int64_t)g * G) * D) + d4;
    float4 acc = src[0];
    for (int j = 1; j < G; ++j) {
        const float4 x = src[j * (D / 4)];
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
    }
    reinterpret_cast<float4*>(out + (bs * a.hkv + g) * D)[d4] = acc;
}

}  // namespace

namespace {

template <int D>
hipError_t launch_backward_d(const BackwardArgs& a, hipStream_t s) {
    const int64_t npk = (a.n_qblk + 1) / 2;
    const int64_t n_sp = dkdv_sink_pairs(a);
    // the per-head partial buffers must hold exactly the sink key pairs' keys (checked before any launch)
    if (!a.in_f32 && n_sp > 0 &&
        (a.part_keys != (128 * n_sp < a.seq ? 128 * n_sp : a.seq) || !a.dk_part || !a.dv_part))
        return hipErrorInvalidValue;
    const int64_t rows = a.batch * (int64_t)a.n_qblk * 64 * a.hq;
    constexpr int rpb = 256 / (D / 8);
    if (!a.in_f32) {   // fp16 copies for the matrix-core kernels; the row statistics read their scales
        const dim3 grid(kAbsmaxChunks, (unsigned)(a.batch * a.hkv), 4);   // z: Q, K, V, dO
        hipLaunchKernelGGL(bwd_absmax_kernel<D>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(bwd_convert_kernel<D>, grid, dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(bwd_rowstat_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, s, a);
    if (a.in_f32) return launch_backward_f32(a, s);   // float32 inputs: vector-ALU kernels
    const int64_t units_kv = n_sp * a.batch * a.hq + (npk - n_sp) * a.batch * a.hkv;
    const int64_t units_q = npk * a.batch * (int64_t)a.hq;
    const int cu = a.num_cu > 0 ? a.num_cu : 256;
    const unsigned grid_kv = (unsigned)(units_kv < cu ? units_kv : cu);          // one 8-wave group per CU
    const unsigned grid_q = (unsigned)(units_q < 2 * cu ? units_q : 2 * cu);     // two 4-wave groups per CU
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(grid_kv), dim3(64 * kKvWaves), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(grid_q), dim3(kThreads), 0, s, a);
    if (n_sp > 0) {
        const int64_t n4 = a.batch * a.part_keys * a.hkv * (D / 4);
        hipLaunchKernelGGL(bwd_group_sum_kernel<D>, dim3((unsigned)((n4 + 255) / 256), 2), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
    if (a.head_dim == 128) return launch_backward_d<128>(a, s);
    if (a.head_dim == 64) return launch_backward_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace flux
