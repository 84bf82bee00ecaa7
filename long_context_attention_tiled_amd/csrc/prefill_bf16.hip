// prefill_bf16.hip -- tiled attention prefill for gfx950, bf16 in, fp32 accumulate.
//
// What it computes: O = softmax(scale * Q K^T + mask) V for every (batch, query
// head), one key tile at a time with the online softmax of the openads.co.kr
// FlashAttention newsletter ("Online Softmax" section): a running row maximum m
// and row sum l, earlier partial outputs rescaled by exp(m_old - m_new) when the
// maximum grows, and the scores never leaving the chip ("FlashAttention: reduce
// memory movement" section).  In block-sparse mode only the key blocks listed in
// the CSR are visited, so K/V of the other blocks are never read (Flux Attention
// page, implementation and architecture paragraphs); without a CSR the same blocks
// (the sink blocks, then the window blocks up to the diagonal) are derived from
// the sink and window sizes with integer arithmetic, which saves the per-tile
// scalar index loads of the CSR walk (4-5% of a block-sparse launch).
//
// Layout of the work on CDNA4:
//   * workgroup = 512 threads = 8 wave64s in two groups of 4.  A group owns 128
//     query rows of one query head (32 rows per wave); the two groups of a
//     workgroup share every K/V tile in LDS: with an even number of query heads per
//     KV head they are two heads of the same KV head over the same rows, otherwise
//     two consecutive 128-row tiles of one head.  Key tiles are 64 keys (= one
//     sparse block).
//   * both contractions run on v_mfma_f32_32x32x16_bf16 in transposed form,
//     S^T = K Q^T and O^T = V^T P^T.  A lane's 32x32 accumulator column is then one
//     query row, so the softmax statistics of a lane's outputs are lane-local: one
//     lane <-> lane^32 exchange per tile (v_permlane32_swap), none for O.
//   * ping-pong between the groups: every step has two phases separated by
//     workgroup barriers.  In each phase one group issues matrix work (P.V of the
//     previous tile, then S of the current tile: 32 MFMAs per wave) while the other
//     group runs the vector work of the softmax (max, exp2, bf16 packing, row sum)
//     of the tile it has just scored; the roles swap every phase.  The two waves
//     sharing a SIMD therefore keep the matrix core and the vector ALU busy at the
//     same time instead of taking turns.
//   * Q stays in registers (B operand of S^T) for the whole kernel.
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4: no
//     staging registers, no LDS store instructions), row-major with an XOR swizzle
//     of the 16-byte chunks of each row so that the operand reads are bank-conflict
//     free.  The V^T operand is read with ds_read_b64_tr_b16, which transposes
//     4x4 blocks of 16-bit elements across lanes: every lane receives 4 keys of its
//     own d column per read, so V never needs a transposed copy.
//   * two LDS slots for K and two for V; K runs one tile ahead of V: at the start of
//     step u the loads of K(u+1) and V(u) are issued (each wave's share of a tile as
//     one run of loads with M0 set once) and they only have to land by the end of
//     step u (two phases later).  The tile loop runs two steps per pass, so that each
//     copy of the step has its slots as constants.
//   * exp2 with scale*log2(e) folded into one FMA.  The running maximum is raised
//     only when some row's new maximum exceeds it by more than 8 (log2 units):
//     until then probabilities up to 2^8 are accumulated against the old
//     reference, which is exact in exact arithmetic (the same reference scales
//     numerator and denominator) and removes most O rescales; the newsletter's
//     FlashAttention-4 section describes the m_new <= m_old special case of this.
//   * P enters P.V rounded to bf16; the row sum is accumulated in fp32 from the
//     unrounded probabilities.
//   * epilogue: bf16 outputs pass through a per-wave LDS stage placed after the K/V
//     slots and leave as 16-byte stores of whole rows, 4 rows per instruction (the
//     accumulator layout alone would put 8 bytes into each of 32 rows per store).
//   * workgroup order: kv-head groups are kept on one XCD (blockIdx % 8 picks the
//     XCD) so the query heads sharing K/V hit the same L2, and query tiles are
//     issued longest-first for causal masks.
//   * soft routing (the Flux Attention page's training-time mix of both modes) is
//     one dense-causal pass whose walk visits each row's sink and window tiles
//     first: where a row's window ends its running O / l is exactly the
//     block-sparse output, which goes to an fp32 scratch buffer; the epilogue
//     writes w_FA * dense + w_SA * sparse.
#include "flux_internal.h"
#include "tile_common.h"

namespace flux {
namespace {

using namespace tile;

constexpr int kBR = 128;       // query rows per wave group
constexpr int kBC = 64;        // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1.0e30f;  // finite start value of the running max
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag the true max

template <int D>
struct Lay {
    static constexpr int ROW_B = D * 2;                    // bytes per K/V row in LDS (no padding)
    static constexpr int CH = ROW_B / 16;                  // 16-byte chunks per row
    static constexpr int TILE_B = kBC * ROW_B;             // bytes per K (or V) tile
    static constexpr int K_BASE = 0;                       // two K slots
    static constexpr int V_BASE = 2 * TILE_B;              // two V slots
    static constexpr int STAGE_BASE = 4 * TILE_B;          // bf16 output stage: 32 rows per wave,
    static constexpr int STAGE_ROW_B = ROW_B + 16;         // each padded by one chunk (bank spread)
    static constexpr int STAGE_B = kWaves * 32 * STAGE_ROW_B;
    static constexpr int SMEM_B = 4 * TILE_B + STAGE_B;
    static constexpr int ROWS_PER_INST = 1024 / ROW_B;     // rows one direct-load instruction fills
    static constexpr int INSTS_PER_WAVE = TILE_B / 1024 / kWaves;
    static_assert(INSTS_PER_WAVE * kWaves * 1024 == TILE_B, "tile split over the waves");
};

// kRouted: causal, dense or sparse as the layer's device-resident mode says (read at start).
// kSoft: dense causal with the key tiles ordered sink, window (descending), then the rest, so that every
// row's block-sparse set is a prefix of its walk: the row's sparse output is taken where its window
// ends and both outputs come from one pass (soft routing).
// kSparseArith: the block-sparse key set derived from (sink, window) with integer arithmetic, the same
// blocks the CSR of flux_build_block_mask lists (kSparse walks that CSR with scalar loads each step).
enum Mode { kDenseCausal = 0, kDenseFull = 1, kSparse = 2, kRouted = 3, kSoft = 4, kSparseArith = 5 };


// Walks the key tiles of a workgroup, whose query rows span the 64-row query blocks
// qb_base .. qb_base + nrows - 1 (nrows = 2 or 4): dense -- tiles 0..last; sparse -- the
// sorted union of those blocks' CSR rows.  next() also returns which of the query
// blocks use the tile (bit r: block qb_base + r).
// Row bits [lo, 4) (lo <= 4) and [0, hi) (hi >= 0) of a 4-row mask: integer arithmetic on workgroup-
// uniform values, which stays on the scalar unit (a bool turned into a bit costs a vector select per
// row, and a clamp from both sides is selected as a vector med3).
__device__ __forceinline__ uint32_t rows_from(int lo) { return (0xFu << max(lo, 0)) & 0xFu; }
__device__ __forceinline__ uint32_t rows_below(int hi) { return (1u << min(hi, 4)) - 1u; }

template <int MODE>
struct TileWalk {
    int next_kb, last_kb, qb_base, nvalid;
    uint32_t valid;   // rows of the workgroup inside the sequence: bits [0, nvalid)
    int p0, p1, p2, p3, e0, e1, e2, e3;   // CSR cursors and ends of the (up to 4) query blocks
    int n_sink, desc_lo, sink_b, win_b;   // kSoft / kSparseArith: sink tiles, lowest window tile, sink and
                                          // window blocks
    const int32_t* ci;
    static constexpr bool sparse = MODE == kSparse;

    __device__ void init(int qb_base_, int nrows, int n_qblk, const int32_t* rp, const int32_t* ci_, int sb = 0,
                         int wb = 0) {
        qb_base = qb_base_;
        nvalid = max(0, min(nrows, n_qblk - qb_base));
        valid = rows_below(nvalid);
        ci = ci_;
        next_kb = 0;
        last_kb = MODE == kDenseFull ? n_qblk - 1 : qb_base + nvalid - 1;
        if constexpr (MODE == kSoft) {
            // walk: sink [0, n_sink), window [desc_lo, last_kb] from the top down, then [sb, desc_lo)
            sink_b = sb;
            n_sink = min(sb, last_kb + 1);
            desc_lo = max(sb, qb_base - wb + 1);
        }
        if constexpr (MODE == kSparseArith) {
            // the union over the rows' blocks I of [0, min(sb, I+1)) and [max(sb, I-wb+1), I]: the sink
            // tiles [0, n_sink), then the window tiles [desc_lo, last_kb] (desc_lo >= n_sink)
            sink_b = sb;
            win_b = wb;
            n_sink = min(sb, last_kb + 1);
            desc_lo = max(n_sink, qb_base - wb + 1);
        }
        if constexpr (sparse) {
            p0 = p1 = p2 = p3 = e0 = e1 = e2 = e3 = 0;
            if (nvalid > 0) p0 = rp[qb_base], e0 = rp[qb_base + 1];
            if (nvalid > 1) p1 = rp[qb_base + 1], e1 = rp[qb_base + 2];
            if (nvalid > 2) p2 = rp[qb_base + 2], e2 = rp[qb_base + 3];
            if (nvalid > 3) p3 = rp[qb_base + 3], e3 = rp[qb_base + 4];
        }
    }

    __device__ int next(int& kb, uint32_t& in) {   // 1: kb and in hold the next tile; 0: the walk is over
        if constexpr (sparse) {
            const int big = 0x7fffffff;
            const int c0 = p0 < e0 ? ci[p0] : big;
            const int c1 = p1 < e1 ? ci[p1] : big;
            const int c2 = p2 < e2 ? ci[p2] : big;
            const int c3 = p3 < e3 ? ci[p3] : big;
            kb = min(min(c0, c1), min(c2, c3));
            if (kb == big) return false;
            const bool h0 = c0 == kb, h1 = c1 == kb, h2 = c2 == kb, h3 = c3 == kb;
            p0 += h0;
            p1 += h1;
            p2 += h2;
            p3 += h3;
            in = (uint32_t)h0 | ((uint32_t)h1 << 1) | ((uint32_t)h2 << 2) | ((uint32_t)h3 << 3);
            return true;
        } else if constexpr (MODE == kSparseArith) {
            kb = next_kb < n_sink ? next_kb : max(next_kb, desc_lo);
            // branch-free on scalars (an early return would make the result a lane mask): have = kb <= last_kb
            const int have = (int)(((uint32_t)(last_kb - kb) >> 31) ^ 1u);
            next_kb = have ? kb + 1 : next_kb;
            // query block I = qb_base + r of the workgroup uses the tile iff kb <= I and (kb is a sink
            // block or I - kb < win_b): rows r >= kb - qb_base, and r < kb - qb_base + win_b unless sink
            const int d = have ? kb - qb_base : 4;   // kb - qb_base <= 3 when the tile exists
            in = valid & rows_from(d) & (kb < sink_b ? 0xFu : rows_below(d + win_b));
            return have;
        } else {
            if constexpr (MODE == kSoft) {
                const int i = next_kb;   // position in the walk
                const int n_desc = max(0, last_kb - desc_lo + 1);
                if (i < n_sink) kb = i;
                else if (i < n_sink + n_desc) kb = last_kb - (i - n_sink);
                else kb = sink_b + (i - n_sink - n_desc);
                if (i >= n_sink + n_desc && kb >= min(desc_lo, last_kb + 1)) return false;
                ++next_kb;
                in = MODE == kDenseFull ? valid : valid & rows_from(kb - qb_base);
                return true;
            } else {
                // branch-free on scalars (an early return would make the result a lane mask)
                kb = next_kb;
                const int have = (int)(((uint32_t)(last_kb - kb) >> 31) ^ 1u);   // kb <= last_kb
                next_kb += have;
                // causal: rows r >= kb - qb_base (<= nvalid <= 4 even one past the last tile)
                in = MODE == kDenseFull ? valid : valid & rows_from(kb - qb_base);
                return have;
            }
        }
    }
};

// Issue this wave's share of the direct HBM -> LDS loads of one K (or V) tile kb into
// the LDS slot at byte address slot.  Lane l of instruction inst fills bytes
// [1024*inst + 16*l, +16) of the slot: row inst*ROWS_PER_INST + l/CH, physical chunk
// l%CH, i.e. logical chunk (l%CH) ^ swizzle(row) of that key.  Keys past the end of
// the sequence are clamped to the last one (masked to -inf in the scores,
// probability 0 in P.V).
template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile(const u16* __restrict__ gbase, uint32_t row_stride, int kb, int last_key,
                                           uint32_t slot, int wave, int lane, const uint32_t* off) {
    using L = Lay<D>;
    const int key0 = kb * kBC;
    if (key0 + kBC - 1 <= last_key) {
        load_lds_run<L::INSTS_PER_WAVE>(uniform_ptr(gbase + (uint32_t)key0 * row_stride), off,
                                        slot + wave * L::INSTS_PER_WAVE * 1024);
    } else {
#pragma unroll
        for (int i = 0; i < L::INSTS_PER_WAVE; ++i) {
            const int inst = wave * L::INSTS_PER_WAVE + i;
            const int row = inst * L::ROWS_PER_INST + lane / L::CH;
            const uint32_t key = (uint32_t)min(key0 + row, last_key);
            const int pch = lane % L::CH;
            const int sw = IS_V ? swz_v<D>(row) : swz_k<D>(row);
            load_lds_16(uniform_ptr(gbase), 2 * (key * row_stride + 8 * (pch ^ sw)), slot + inst * 1024);
        }
    }
}

// The K-tile loads of one wave: NI direct-load instructions of the tile, starting at instruction `first`
// (the K tile's instructions are not split evenly over the waves; see prefill_body).
template <int D, int NI>
__device__ __forceinline__ void issue_k(const u16* __restrict__ gbase, uint32_t row_stride, int kb, int last_key,
                                        uint32_t slot, int first, int lane, const uint32_t* off) {
    using L = Lay<D>;
    const int key0 = kb * kBC;
    if (key0 + kBC - 1 <= last_key) {
        if constexpr (NI > 0) load_lds_run<NI>(uniform_ptr(gbase + (uint32_t)key0 * row_stride), off, slot + first * 1024);
    } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int inst = first + i;
            const int row = inst * L::ROWS_PER_INST + lane / L::CH;
            const uint32_t key = (uint32_t)min(key0 + row, last_key);
            const int pch = lane % L::CH;
            load_lds_16(uniform_ptr(gbase), 2 * (key * row_stride + 8 * (pch ^ swz_k<D>(row))), slot + inst * 1024);
        }
    }
}

template <int D, int MODE, bool OUT_F32>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, char* smem) {
    using L = Lay<D>;
    constexpr int NC = D / 16;   // 16-wide d chunks of the S^T contraction
    constexpr int NM = D / 32;   // 32-row d tiles of O^T

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;   // wave group
    const int wq = wave & 3;     // wave inside its group
    const int n = lane & 31;     // query column of this lane inside the wave's 32 rows
    const int hh = lane >> 5;    // which half of the k-slots / accumulator rows

    // ---- work units: (batch, kv head g, two slots of 128 query rows).  A unit's logical id comes
    // from a virtual block index through xcd_remap, so the units of one kv head share an XCD.
    const int seq = (int)a.seq;          // the host guarantees seq * max(hq, hkv) * d < 2^31
    const int nqt = (seq + kBR - 1) / kBR;
    const int G = a.hq / a.hkv;
    const bool pair_heads = (G & 1) == 0;
    const int per_g = pair_heads ? (G / 2) * nqt : G * ((nqt + 1) / 2);
    const int total = (int)a.batch * a.hkv * per_g;
    // Persistent schedule when the grid is smaller than the unit count (the grid is then a multiple
    // of 8): workgroup w stays on XCD w % 8 and takes that XCD's units in snake order over rounds of
    // gridDim/8 (longest-first units in even rounds, shortest-first in odd ones), which balances the
    // causal triangle; otherwise one unit per workgroup.
    const bool persistent = (int)gridDim.x < total;
    const int xcd = (int)blockIdx.x & 7, wi = (int)blockIdx.x >> 3, nper = (int)gridDim.x >> 3;
    auto vb_at = [&](int k) -> int {
        if (!persistent) return k == 0 ? (int)blockIdx.x : total;
        const int t = k * nper + ((k & 1) ? nper - 1 - wi : wi);
        return t * 8 + xcd;
    };

    const uint32_t q_row_stride = (uint32_t)(a.hq * D);
    const uint32_t kv_row_stride = (uint32_t)(a.hkv * D);
    const int last_key = seq - 1;

    // per-lane byte offsets of the direct loads inside a tile (tile-invariant)
    uint32_t koff[4], voff[L::INSTS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < L::INSTS_PER_WAVE; ++i) {
        const int row = (wave * L::INSTS_PER_WAVE + i) * L::ROWS_PER_INST + lane / L::CH;
        const int pch = lane % L::CH;
        voff[i] = 2 * (row * kv_row_stride + 8 * (pch ^ swz_v<D>(row))) - 1024 * i;   // see load_lds_run
    }
    // Each step opens with every wave issuing its share of the next tiles' direct loads (one run per tile,
    // ~60 cycles per instruction and wave when all eight waves issue together), and group 1 then runs the
    // softmax phase, the longer of the two first phases: at head_dim 128 the waves of group 0 take 3 of
    // the K tile's 16 instructions each and those of group 1 take 1 (0.6-0.7% faster at seq 131072 dense
    // than 2 and 2 when each load set and restored M0 itself; within noise with the runs).
    constexpr int KI = L::TILE_B / 1024;          // K-tile instructions per workgroup
    constexpr int KA = D == 128 ? 3 : KI / 8;     // per wave of group 0 (matrix work first)
    constexpr int KB = (KI - 4 * KA) / 4;         // per wave of group 1
    static_assert(4 * KA + 4 * KB == KI && KA <= 4, "K tile split over the waves");
    const int kfirst = grp == 0 ? KA * wq : 4 * KA + KB * wq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (kfirst + i) * L::ROWS_PER_INST + lane / L::CH;
        const int pch = lane % L::CH;
        koff[i] = 2 * (row * kv_row_stride + 8 * (pch ^ swz_k<D>(row))) - 1024 * i;   // see load_lds_run
    }
    const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // state of the current unit
    int b = 0, h = 0, qb_base = 0, my_r = 0, my_qb = 0, qpos = 0;
    bool wave_live = false;
    const u16* kg = nullptr;
    const u16* vg = nullptr;
    auto issue_ktile = [&](int kb, uint32_t slot) {
        if (grp == 0) issue_k<D, KA>(kg, kv_row_stride, kb, last_key, slot, kfirst, lane, koff);
        else issue_k<D, KB>(kg, kv_row_stride, kb, last_key, slot, kfirst, lane, koff);
    };
    bf16x8 qreg[NC];   // Q rows as the B operand of S^T = K Q^T: lane holds Q[qpos][16c + 8hh .. +7]
    TileWalk<MODE> walk;
    uint32_t in;
    int kb_p = 0, kb_c = 0, kb_n = 0;
    bool mine_p = false, mine_c = false, mine_n = false, have_any = false;
    int have_n = 0;   // an int rather than a bool, kept on the scalar unit across the loop's blocks

    // Set up unit vb and issue its first loads (K of its first tile into K slot 0, its Q rows into
    // registers).  Called before the first unit and, for the next unit, after the current unit's
    // last S (Q and both K slots are free then).
    auto begin_unit = [&](int vb) {
        int lid = xcd_remap(vb, total);
        const int unit = lid % per_g;
        lid /= per_g;
        const int g = lid % a.hkv;
        b = lid / a.hkv;
        int qt, nrows;
        if (pair_heads) {                    // groups = query heads 2jp, 2jp+1 of g, same rows
            const int jp = unit % (G / 2);
            const int rank = unit / (G / 2);
            qt = (MODE != kDenseFull) ? nqt - 1 - rank : rank;   // causal: longest first
            h = g * G + 2 * jp + grp;
            qb_base = 2 * qt;
            my_r = wq >> 1;
            nrows = 2;
        } else {                             // groups = query tiles 2qp, 2qp+1 of one head
            const int npq = (nqt + 1) / 2;
            const int j = unit % G;
            const int rank = unit / G;
            const int qp = (MODE != kDenseFull) ? npq - 1 - rank : rank;
            h = g * G + j;
            qt = 2 * qp + grp;
            qb_base = 4 * qp;
            my_r = 2 * grp + (wq >> 1);
            nrows = 4;
        }
        kg = reinterpret_cast<const u16*>(a.k) + ((int64_t)b * a.seq * a.hkv + g) * D;
        vg = reinterpret_cast<const u16*>(a.v) + ((int64_t)b * a.seq * a.hkv + g) * D;
        const int q0 = qt * kBR + wq * 32;   // first query row of this wave
        qpos = q0 + n;                       // this lane's query row
        wave_live = q0 < seq;
        my_qb = qb_base + my_r;
        walk.init(qb_base, nrows, a.n_qblk, a.row_ptr, a.col_idx, a.sink_blocks, a.window_blocks);
        have_any = walk.next(kb_c, in);      // uniform over the workgroup; true for every valid launch
        mine_c = have_any && wave_live && ((in >> my_r) & 1);
        have_n = have_any ? walk.next(kb_n, in) : 0;
        mine_n = have_n && wave_live && ((in >> my_r) & 1);
        mine_p = false;
        if (have_any) issue_ktile(kb_c, smem_lds + L::K_BASE);
        const u16* qg = reinterpret_cast<const u16*>(a.q) + ((int64_t)b * a.seq * a.hq + h) * D;
        const uint32_t qrow = (uint32_t)min(qpos, last_key);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qreg[c] = *reinterpret_cast<const bf16x8*>(qg + qrow * q_row_stride + 16 * c + 8 * hh);
    };

    // LDS byte offsets of this lane's operand reads (slot-relative)
    // K: row 32kh + n, logical chunk 2c + hh -> physical (2c + hh) ^ swz_k(32kh + n)
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
        vaddr[mt] = vkey * L::ROW_B + 16 * (lch ^ swz_v<D>(vkey)) + 8 * (jj & 1);
    }

    f32x16 oacc[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) oacc[mt] = f32x16{};
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    bf16x8 pb[2][2];
    float m_run = kNegBig, l_run = 0.0f;
    const float c2 = a.scale_log2;
    const float slack_s = kRescaleSlack / c2;   // the slack in score units
    float m_thr = kNegBig;                       // m_run + slack_s (kNegBig absorbs the slack)
    bool snapped = false;   // kSoft: this wave's block-sparse output has been written to soft_ws

    // kSoft: the rows' block-sparse output O / l over the tiles accumulated so far (the row's sink and
    // window tiles), to soft_ws in fp32.  Wave-uniform call (the half-row sums are exchanged).
    auto snapshot = [&]() {
        const float l_tot = sum_halves(l_run);
        if (!wave_live || qpos >= seq) return;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float* dst = a.soft_ws + (((int64_t)b * seq + qpos) * a.hq + h) * D;
#pragma unroll
        for (int mt = 0; mt < NM; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<float4*>(dst + 32 * mt + 8 * r4 + 4 * hh) =
                    make_float4(oacc[mt][4 * r4] * inv, oacc[mt][4 * r4 + 1] * inv, oacc[mt][4 * r4 + 2] * inv,
                                oacc[mt][4 * r4 + 3] * inv);
    };

    // ---- matrix work of one phase: O^T += V^T P^T for the previous tile (V slot vs), then
    // S^T = K Q^T for the current tile (K slot ks), as one sequence of up to 32 MFMAs whose
    // LDS operands are read kPrefetch MFMAs ahead (one 32x32x16 MFMA runs 32 cycles, an LDS
    // read under load takes several times that).  The wave raises its issue priority so
    // that the vector work of the other group fills the MFMA shadow rather than delaying
    // the next MFMA.
    constexpr int kPrefetch = 6;
    auto mseq = [&](auto pv_tag, auto s_tag, int vs, int ks) {
        constexpr bool PV = decltype(pv_tag)::value;
        constexpr bool S = decltype(s_tag)::value;
        constexpr int NPV = PV ? 4 * NM : 0;    // P.V steps: (kh, aa) major, d tile mt minor
        constexpr int NT = NPV + (S ? 2 * NC : 0);
        const char* vt = smem + L::V_BASE + vs * L::TILE_B;
        const char* kt = smem + L::K_BASE + ks * L::TILE_B;
        // operand of step i.  P.V step (kh, aa, mt): P slot e' is key 32kh + 16aa + 8(e'/4) +
        // 4hh + e'%4, so two transposing reads (keys +0..3 and +8..11 of the lane group's 4-key
        // block).  S step (c, kh): K rows 32kh + n, d chunk c.
        auto operand = [&](int i) -> bf16x8 {
            if (i < NPV) {
                const int kk = i / NM, mt = i % NM;
                const char* vp = vt + vaddr[mt] + (32 * (kk >> 1) + 16 * (kk & 1)) * L::ROW_B;
                const i16x4 lo = read_tr16(vp);
                const i16x4 hi = read_tr16(vp + 8 * L::ROW_B);
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            const int j = i - NPV;
            return *reinterpret_cast<const bf16x8*>(kt + kaddr[j & 1][j >> 1]);
        };
        bf16x8 ring[kPrefetch];
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i)
            if (i < NT) ring[i] = operand(i);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const bf16x8 op = ring[i % kPrefetch];
            if (i + kPrefetch < NT) ring[i % kPrefetch] = operand(i + kPrefetch);
            if (i < NPV) {
                const int kk = i / NM, mt = i % NM;
                oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pb[kk >> 1][kk & 1], oacc[mt], 0, 0, 0);
            } else {
                const int j = i - NPV;   // two independent chains: 32-key halves kh = j & 1
                const f32x16 acc = j < 2 ? f32x16{} : sacc[j & 1];
                sacc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[j >> 1], acc, 0, 0, 0);
            }
            // keep the written order (read i+kPrefetch, MFMA i): the scheduler would otherwise
            // hoist every read of the phase and run out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto mwork = [&](auto pv_tag, auto s_tag, int vs, int ks) {
        __builtin_amdgcn_s_setprio(2);
        mseq(pv_tag, s_tag, vs, ks);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- vector work: online softmax of the scores of key tile kb -> P (bf16) in pb.
    // Lane holds S[qpos][key], key = kb*64 + 32kh + 8(r/4) + 4hh + (r%4).
    auto vwork = [&](bool mine, int kb) {
        if constexpr (MODE == kSoft) {
            // first tile of this wave's rows outside their sink and window: every earlier P.V is in O
            // (the matrix phase before this one added the previous tile), l counts exactly those tiles
            if (mine && !snapped && kb >= a.sink_blocks && my_qb - kb >= a.window_blocks) {
                snapshot();
                snapped = true;
            }
        }
        if (!mine) {   // tile not used by this wave's rows: its P.V adds exact zeros
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int aa = 0; aa < 2; ++aa) pb[kh][aa] = bf16x8{};
            return;
        }
        const bool need_mask = (MODE != kDenseFull && kb >= my_qb) || (kb + 1) * kBC > seq;
        if (need_mask) {
            // key > lim is masked, lim = last allowed key of this lane's row minus the tile/lane base
            const int lim = (MODE != kDenseFull ? min(qpos, last_key) : last_key) - (kb * kBC + 4 * hh);
            // one compare/select pair at a time: hoisting all 32 compares would hold 32 lane masks
            // in scalar registers and push other scalars out to spill slots for the whole kernel
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (32 * kh + 8 * (r >> 2) + (r & 3) > lim) sacc[kh][r] = -INFINITY;
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        // row max as a chain of v_maximum3_f32 (the IEEE maximum needs no canonicalising of the MFMA
        // results, which fmaxf's maxnum does; the scores are finite or -inf, where the two agree)
        float mx = sacc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sacc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sacc[1][r]);
        mx = max_halves(mx);
        // raise the reference max only when some row outgrows it by more than the slack, i.e. exceeds
        // m_thr = m_run + slack / c2 (c2 > 0)
        if (__ballot(mx > m_thr)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < NM; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[mt][r] *= alpha;
            m_run = m_new;
            m_thr = m_new + slack_s;
        }
        const float mc = m_run * c2;
        float lsum[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int aa = 0; aa < 2; ++aa) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kh][8 * aa + e], c2, -mc));
                pb[kh][aa] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                                    (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
                lsum[kh][aa] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            }
        // row sum in fp32 over the unrounded probabilities (plain adds: cheaper than bf16 dot
        // products in this phase)
        l_run += (lsum[0][0] + lsum[0][1]) + (lsum[1][0] + lsum[1][1]);
    };

    // ---- epilogue of the current unit: O = O^T / l, lane holds O[qpos][32mt + 8(r/4) + 4hh + r%4].
    // bf16 outputs (but the soft form's) pass through the wave's own LDS stage (32 rows, each padded by 16
    // bytes so that the 16-byte row-wise writes and the chunk-wise reads both spread over the banks, with
    // constant offsets) and leave as 16-byte stores of whole rows, 4 rows (1 KB) per instruction at
    // head_dim 128, where the lane layout would give 8-byte stores to 32 rows per instruction.
    auto finish_unit = [&]() {
        // the soft form writes directly: its mixing reads leave no registers for the stage
        constexpr bool kStaged = !OUT_F32 && MODE != kSoft;
        const float l_tot = sum_halves(l_run);
        if (!wave_live) return;   // wave-uniform
        const bool row_ok = qpos < seq;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int64_t orow = ((int64_t)b * seq + qpos) * a.hq + h;
        const int64_t orow_in = ((int64_t)b * seq + min(qpos, seq - 1)) * a.hq + h;
        // the stage addresses are formed here from an opaque copy of the lane index: hoisted out of the
        // unit loop they would hold registers across the whole tile loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int sn = ln & 31, shh = ln >> 5;
        char* stage = smem + L::STAGE_BASE + wave * 32 * L::STAGE_ROW_B;
        uint32_t pa0 = 0, pa1 = 0;   // packed bf16 of the even r4 of a pair, until its odd partner
#pragma unroll
        for (int mt = 0; mt < NM; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * mt + 8 * r4 + 4 * hh;
                float v0 = oacc[mt][4 * r4] * inv, v1 = oacc[mt][4 * r4 + 1] * inv;
                float v2 = oacc[mt][4 * r4 + 2] * inv, v3 = oacc[mt][4 * r4 + 3] * inv;
                if constexpr (MODE == kSoft) {   // w_FA * dense + w_SA * block-sparse
                    const float w0 = a.mix_w[0], w1 = a.mix_w[1];
                    if (snapped) {
                        // rows past seq (never stored) read the last row instead: in bounds, no select
                        const float4 f = *reinterpret_cast<const float4*>(a.soft_ws + orow_in * D + d);
                        v0 = fmaf(w1, f.x, w0 * v0);
                        v1 = fmaf(w1, f.y, w0 * v1);
                        v2 = fmaf(w1, f.z, w0 * v2);
                        v3 = fmaf(w1, f.w, w0 * v3);
                    } else {   // the row's sparse set is all of its keys
                        const float w = w0 + w1;
                        v0 *= w;
                        v1 *= w;
                        v2 *= w;
                        v3 *= w;
                    }
                }
                if constexpr (OUT_F32) {
                    if (row_ok)
                        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + orow * D + d) =
                            make_float4(v0, v1, v2, v3);
                } else if constexpr (!kStaged) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    if (row_ok)
                        *reinterpret_cast<bf16x4*>(reinterpret_cast<u16*>(a.o) + orow * D + d) =
                            bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                } else {
                    // r4 pairs (2j, 2j + 1): one v_permlane32_swap per dword hands each lane 16 contiguous
                    // bytes of its row (lanes 0-31 the pair's first 8 d values, lanes 32-63 its last 8), so
                    // that the stage takes 16-byte writes, 16 rows per bank sweep
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    const uint32_t w0 = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v0, (__bf16)v1});
                    const uint32_t w1 = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v2, (__bf16)v3});
                    if ((r4 & 1) == 0) {
                        pa0 = w0;
                        pa1 = w1;
                    } else {
                        const auto x = __builtin_amdgcn_permlane32_swap(pa0, w0, false, false);
                        const auto y = __builtin_amdgcn_permlane32_swap(pa1, w1, false, false);
                        *reinterpret_cast<uint4*>(stage + sn * L::STAGE_ROW_B + 16 * (4 * mt + (r4 & 2) + shh)) =
                            uint4{x[0], y[0], x[1], y[1]};
                    }
                }
            }
        if constexpr (kStaged) {
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's stage writes done
            constexpr int kRowsPerRead = 64 / L::CH;   // rows one 1 KB read covers
            const int c = ln % L::CH;
            const int r0 = ln / L::CH;
            const int rows_left = seq - (qpos - n) - r0;   // rows of this lane's column still inside seq
            const int64_t step = (int64_t)kRowsPerRead * a.hq * D;
            u16* op = reinterpret_cast<u16*>(a.o) + (((int64_t)b * seq + qpos - n + r0) * a.hq + h) * D + 8 * c;
            const char* sp = stage + r0 * L::STAGE_ROW_B + 16 * c;
#pragma unroll
            for (int i = 0; i < 32 / kRowsPerRead; ++i) {
                const uint4 val = *reinterpret_cast<const uint4*>(sp + i * kRowsPerRead * L::STAGE_ROW_B);
                if (i * kRowsPerRead < rows_left) *reinterpret_cast<uint4*>(op) = val;
                op += step;
                __builtin_amdgcn_sched_barrier(0);   // one read, one store: no stage registers held
            }
        }
        if (a.lse && hh == 0 && row_ok) {
            const float lse = l_tot > 0.0f ? (m_run * c2 + __log2f(l_tot)) * kLn2 : -INFINITY;
            a.lse[((int64_t)b * a.hq + h) * a.seq + qpos] = lse;
        }
    };

    // ---- tile pipeline.  Tile t's K goes to K slot t&1, its V to V slot t&1.  Step u (one per
    // tile, plus a final one) issues the loads of K(u+1) and V(u), then runs two phases:
    //   phase A: group 0 matrix work (P.V of tile u-1, S of tile u) | group 1 softmax of tile u-1
    //   phase B: group 0 softmax of tile u | group 1 matrix work (P.V of tile u-1, S of tile u)
    // The first step has no P.V and the final step no S; every wave of a group issues the
    // same MFMAs (a wave whose rows skip a tile multiplies zero probabilities), so the
    // loop body has a single form.  After the final step's S-free phase each group writes its
    // outputs and starts the loads of its next unit.
    constexpr BoolTag<true> kOn{};
    constexpr BoolTag<false> kOff{};
    begin_unit(vb_at(0));
    auto run = [&](auto group_tag) {
        constexpr bool kG1 = decltype(group_tag)::value;
        for (int k = 1;; ++k) {
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): Q and K of the unit's first tile in place
            __syncthreads();
            if (have_any) {
                // step 0
                if (have_n)
                    issue_ktile(kb_n, smem_lds + L::K_BASE + L::TILE_B);
                issue_tile<D, true>(vg, kv_row_stride, kb_c, last_key, smem_lds + L::V_BASE, wave, lane, voff);
                if constexpr (!kG1) mwork(kOff, kOn, 0, 0);
                __syncthreads();
                if constexpr (!kG1) vwork(mine_c, kb_c);
                else mwork(kOff, kOn, 0, 0);
                __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's loads of K(1), V(0) landed
                __syncthreads();
                // steps 1 .. T-1: step u reads K slot u&1 and V slot (u-1)&1 and loads into the others.
                // Two steps per pass of the loop, so that each copy has its slots as constants and the
                // branch back to the loop head comes once per two steps.
                auto step = [&](auto slot_tag) {
                    constexpr int sl = decltype(slot_tag)::value;
                    kb_p = kb_c;
                    mine_p = mine_c;
                    kb_c = kb_n;
                    mine_c = mine_n;
                    have_n = walk.next(kb_n, in);
                    mine_n = have_n && wave_live && ((in >> my_r) & 1);
                    if (have_n)
                        issue_ktile(kb_n, smem_lds + L::K_BASE + (sl ^ 1) * L::TILE_B);
                    issue_tile<D, true>(vg, kv_row_stride, kb_c, last_key, smem_lds + L::V_BASE + sl * L::TILE_B,
                                        wave, lane, voff);
                    if constexpr (!kG1) mwork(kOn, kOn, sl ^ 1, sl);
                    else vwork(mine_p, kb_p);
                    __syncthreads();
                    if constexpr (!kG1) vwork(mine_c, kb_c);
                    else mwork(kOn, kOn, sl ^ 1, sl);
                    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's loads of K(u+1), V(u) landed
                    __syncthreads();
                };
                int sl = 1;   // the slot the next step's V goes to
                while (have_n) {
                    step(IntTag<1>{});
                    if (!have_n) {
                        sl = 0;
                        break;
                    }
                    step(IntTag<0>{});
                }
                // final step: P.V of the last tile (its V is in slot sl ^ 1)
                if constexpr (!kG1) mwork(kOn, kOff, sl ^ 1, 0);
                else vwork(mine_c, kb_c);
                __syncthreads();
                if constexpr (kG1) mwork(kOn, kOff, sl ^ 1, 0);
            }
            finish_unit();
            const int vb = vb_at(k);
            if (vb >= total) break;
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) oacc[mt] = f32x16{};
            m_run = kNegBig;
            m_thr = kNegBig;
            l_run = 0.0f;
            snapped = false;
            begin_unit(vb);
        }
    };
    if (grp == 0)
        run(BoolTag<false>{});
    else
        run(BoolTag<true>{});
}

// kRouted: one launch whose workgroups read the layer's mode and run the dense-causal or the
// block-sparse body (two complete code paths, so neither carries the other's state).
template <int D, int MODE, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2))) void
prefill_bf16_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[Lay<D>::SMEM_B];
    if constexpr (MODE == kRouted) {
        if (a.mode_dev[0] == 0)
            prefill_body<D, kDenseCausal, OUT_F32>(a, smem);
        else if (a.row_ptr)
            prefill_body<D, kSparse, OUT_F32>(a, smem);
        else
            prefill_body<D, kSparseArith, OUT_F32>(a, smem);
    } else {
        prefill_body<D, MODE, OUT_F32>(a, smem);
    }
}

template <int D, int MODE>
hipError_t launch_mode(const PrefillArgs& a, hipStream_t s) {
    const int64_t nqt = (a.seq + kBR - 1) / kBR;
    const int64_t G = a.hq / a.hkv;
    const int64_t per_g = (G % 2 == 0) ? (G / 2) * nqt : G * ((nqt + 1) / 2);
    const int64_t total = a.batch * a.hkv * per_g;
    // one resident workgroup per CU; persistent when there are at least two units per CU
    const int64_t persist = (int64_t)(a.num_cu / 8) * 8;
    const int64_t grid = (persist >= 8 && total >= 2 * persist) ? persist : total;
    if (a.out_f32)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const PrefillArgs& a, hipStream_t s) {
    if (a.soft_ws) return launch_mode<D, kSoft>(a, s);
    if (a.mode_dev) return launch_mode<D, kRouted>(a, s);
    if (a.sparse) return a.row_ptr ? launch_mode<D, kSparse>(a, s) : launch_mode<D, kSparseArith>(a, s);
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
