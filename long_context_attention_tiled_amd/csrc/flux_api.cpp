// flux_api.cpp -- host side of the C ABI declared in include/flux_attn.h:
// argument validation (before any HIP call), the block-mask builder, launch
// configuration, per-layer dispatch and status reporting.
#include "../../include/flux_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "flux_internal.h"

namespace {

thread_local char g_detail[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_detail[0] = '\0';
    return FLUX_OK;
}

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    return fail(FLUX_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- block mask
struct MaskSpec {
    int64_t seq_q, seq_k, block;
    int64_t sink_blocks, window_blocks;
    bool causal, sparse;
};

int check_mask_spec(int64_t seq_q, int64_t seq_k, int32_t block, int32_t sink, int32_t window,
                    int32_t causal, int32_t mode, MaskSpec* ms) {
    if (seq_q < 1 || seq_k < 1) return fail(FLUX_ERR_INVALID_ARG, "seq_q/seq_k must be >= 1");
    if (block < 1) return fail(FLUX_ERR_INVALID_ARG, "block must be >= 1");
    if (mode != FLUX_MODE_DENSE && mode != FLUX_MODE_SPARSE)
        return fail(FLUX_ERR_INVALID_ARG, "mode must be FLUX_MODE_DENSE or FLUX_MODE_SPARSE");
    if (causal != 0 && causal != 1) return fail(FLUX_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (ceil_div(seq_q, block) > INT32_MAX - 1 || ceil_div(seq_k, block) > INT32_MAX - 1)
        return fail(FLUX_ERR_INVALID_ARG, "too many blocks for int32 indices");
    ms->seq_q = seq_q;
    ms->seq_k = seq_k;
    ms->block = block;
    ms->causal = causal != 0;
    ms->sparse = mode == FLUX_MODE_SPARSE;
    ms->sink_blocks = 0;
    ms->window_blocks = 0;
    if (ms->sparse) {
        if (!causal) return fail(FLUX_ERR_INVALID_ARG, "sparse mode requires causal == 1");
        if (sink < 0 || sink % block != 0)
            return fail(FLUX_ERR_INVALID_ARG, "sink_tokens (%d) must be >= 0 and a multiple of block (%d)", sink,
                        block);
        if (window < block || window % block != 0)
            return fail(FLUX_ERR_INVALID_ARG, "window_tokens (%d) must be >= block and a multiple of block (%d)",
                        window, block);
        ms->sink_blocks = sink / block;
        ms->window_blocks = window / block;
    }
    return FLUX_OK;
}

// Active key blocks of query block I: [0, lo_end) U [hi_begin, hi_end], ascending, disjoint.
void row_ranges(const MaskSpec& ms, int64_t I, int64_t* lo_end, int64_t* hi_begin, int64_t* hi_end) {
    int64_t nbk = ceil_div(ms.seq_k, ms.block);
    int64_t last = ms.causal ? std::min(I, nbk - 1) : nbk - 1;
    if (!ms.sparse) {
        *lo_end = last + 1;
        *hi_begin = last + 1;
        *hi_end = last;
        return;
    }
    int64_t sink_end = std::min(ms.sink_blocks, last + 1);
    int64_t win_begin = std::max(I - ms.window_blocks + 1, sink_end);
    *lo_end = sink_end;
    *hi_begin = win_begin;
    *hi_end = last;
}

int64_t mask_nnz(const MaskSpec& ms) {
    int64_t nbq = ceil_div(ms.seq_q, ms.block), nnz = 0;
    for (int64_t I = 0; I < nbq; ++I) {
        int64_t lo, hb, he;
        row_ranges(ms, I, &lo, &hb, &he);
        nnz += lo + (he >= hb ? he - hb + 1 : 0);
    }
    return nnz;
}

// ---------------------------------------------------------------- prefill validation
int check_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int32_t in_dtype,
                  int32_t out_dtype, int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                  float scale, int32_t causal, int32_t mode, int32_t block, int32_t sink, int32_t window,
                  const int32_t* rp, const int32_t* ci, int64_t nnz, flux::PrefillArgs* a) {
    if (!q || !k || !v || !o) return fail(FLUX_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(FLUX_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(FLUX_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (batch < 1 || seq < 1) return fail(FLUX_ERR_INVALID_ARG, "batch and seq must be >= 1");
    if (hq < 1 || hkv < 1 || hq % hkv != 0)
        return fail(FLUX_ERR_INVALID_ARG, "hq (%d) must be a positive multiple of hkv (%d)", hq, hkv);
    if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(FLUX_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (in_dtype != FLUX_DTYPE_BF16 && in_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "in_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    if (out_dtype != FLUX_DTYPE_BF16 && out_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "out_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    MaskSpec ms;
    int st = check_mask_spec(seq, seq, block, sink, window, causal, mode, &ms);
    if (st != FLUX_OK) return st;
    if (head_dim != 64 && head_dim != 128)
        return fail(FLUX_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
    if (block != flux::kBlock) return fail(FLUX_ERR_UNSUPPORTED, "block %d not supported (64)", block);
    if (in_dtype == FLUX_DTYPE_F32 && out_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_UNSUPPORTED, "float32 input requires float32 output");
    if (batch * (int64_t)hq * ceil_div(seq, 64) > INT32_MAX)
        return fail(FLUX_ERR_UNSUPPORTED, "batch * hq * ceil(seq/64) exceeds the launch grid");
    if (seq * (int64_t)std::max(hq, hkv) * head_dim > INT32_MAX)
        return fail(FLUX_ERR_UNSUPPORTED, "seq * max(hq, hkv) * head_dim must stay below 2^31 elements");
    if (ms.sparse && (rp || ci)) {   // the CSR walk; without a CSR the kernels derive the same blocks
        if (!rp || !ci) return fail(FLUX_ERR_INVALID_ARG, "blk_row_ptr and blk_col_idx must both be given or both NULL");
        int64_t want = mask_nnz(ms);
        if (nnz != want)
            return fail(FLUX_ERR_INVALID_ARG, "blk_nnz %lld does not match the sparse pattern (%lld)",
                        (long long)nnz, (long long)want);
    }
    a->q = q;
    a->k = k;
    a->v = v;
    a->o = o;
    a->lse = lse;
    a->batch = batch;
    a->seq = seq;
    a->hq = hq;
    a->hkv = hkv;
    a->head_dim = head_dim;
    a->scale = scale;
    a->scale_log2 = scale * 1.4426950408889634f;
    a->causal = causal;
    a->sparse = ms.sparse ? 1 : 0;
    a->out_f32 = out_dtype == FLUX_DTYPE_F32;
    a->n_qblk = (int)ceil_div(seq, 64);
    a->row_ptr = ms.sparse ? rp : nullptr;
    a->col_idx = ms.sparse ? ci : nullptr;
    a->mode_dev = nullptr;
    a->num_cu = 0;
    a->mix_w = nullptr;
    a->soft_ws = nullptr;
    a->sink_blocks = ms.sparse ? (int)(sink / block) : 0;
    a->window_blocks = ms.sparse ? (int)(window / block) : 0;
    return FLUX_OK;
}

// Compute units of the current device (cached per device id; 0 if the query fails, which makes the
// prefill launch fall back to one workgroup per unit).
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cached[dev] = v;
    }
    return cached[dev];
}

int launch_prefill(const flux::PrefillArgs& args, int32_t in_dtype, hipStream_t s) {
    flux::PrefillArgs a = args;
    a.num_cu = device_cu_count();
    hipError_t e = in_dtype == FLUX_DTYPE_BF16 ? flux::launch_prefill_bf16(a, s) : flux::launch_prefill_f32(a, s);
    if (e == hipSuccess) e = hipGetLastError();
    return hip_status(e, "prefill launch");
}

// ---------------------------------------------------------------- decode planning
struct DecodePlan {
    int64_t r0_end, r1_begin, n_active;
    int n_split;
    int64_t split_len;
    size_t ws_bytes;
};

constexpr int kDecodeTargetGroups = 2048;  // workgroups the automatic split count aims for
constexpr int64_t kDecodeMinSplit = 192;   // keys per split at least (12 splits for a sink + window row)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int plan_decode(int64_t batch, int32_t hq, int32_t hkv, int64_t kv_len, int32_t head_dim, int32_t mode,
                int32_t block, int32_t sink, int32_t window, int32_t num_splits, DecodePlan* p) {
    if (batch < 1 || kv_len < 1) return fail(FLUX_ERR_INVALID_ARG, "batch and kv_len must be >= 1");
    if (hq < 1 || hkv < 1 || hq % hkv != 0)
        return fail(FLUX_ERR_INVALID_ARG, "hq (%d) must be a positive multiple of hkv (%d)", hq, hkv);
    if (num_splits < 0) return fail(FLUX_ERR_INVALID_ARG, "num_splits must be >= 0");
    MaskSpec ms;
    int st = check_mask_spec(kv_len, kv_len, block, sink, window, 1, mode, &ms);
    if (st != FLUX_OK) return st;
    if (head_dim != 64 && head_dim != 128)
        return fail(FLUX_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
    if (block != flux::kBlock) return fail(FLUX_ERR_UNSUPPORTED, "block %d not supported (64)", block);
    int g = hq / hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(FLUX_ERR_UNSUPPORTED, "hq/hkv = %d not supported (1, 2, 4 or 8)", g);
    // keys of prefill row kv_len-1, as token ranges
    int64_t qb = (kv_len - 1) / block, lo, hb, he;
    row_ranges(ms, qb, &lo, &hb, &he);
    p->r0_end = std::min(lo * block, kv_len);
    p->r1_begin = he >= hb ? std::max(hb * block, p->r0_end) : kv_len;
    if (p->r1_begin > kv_len) p->r1_begin = kv_len;
    p->n_active = p->r0_end + (kv_len - p->r1_begin);
    int64_t max_split = std::max<int64_t>(1, ceil_div(p->n_active, kDecodeMinSplit));
    int64_t n = num_splits;
    if (n == 0) {
        int64_t groups = batch * hkv;
        n = std::max<int64_t>(1, ceil_div(kDecodeTargetGroups, groups));
        n = std::min(n, max_split);
    }
    n = std::min<int64_t>(n, ceil_div(p->n_active, 64));
    if (n > 65535) return fail(FLUX_ERR_UNSUPPORTED, "too many splits");
    p->split_len = ceil_div(ceil_div(p->n_active, n), 64) * 64;
    p->n_split = (int)ceil_div(p->n_active, p->split_len);
    if (num_splits > 0 && p->n_split < num_splits) {
        // keep the caller's split count (some splits end up empty and are weighted 0)
        p->n_split = num_splits;
    }
    size_t rows = (size_t)batch * hq * p->n_split;
    p->ws_bytes = align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
    return FLUX_OK;
}

// ---------------------------------------------------------------- device attributes
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Validation and launch of one decode call.  k_new / v_new non-NULL: the token at kv_len-1 is taken
// from them and stored into the cache by the same launch.  layout FLUX_KV_WINDOW: the cache holds the
// sink rows and a ring of window blocks (see flux_attn.h).
int run_decode(const void* q, const void* k_cache, const void* v_cache, const void* k_new, const void* v_new, void* o,
               float* lse, int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t kv_len, int64_t cache_rows,
               int32_t layout, int32_t hq, int32_t hkv, int32_t head_dim, float scale, int32_t mode, int32_t block,
               int32_t sink_tokens, int32_t window_tokens, int32_t num_splits, void* workspace,
               size_t workspace_bytes, void* hip_stream, bool launch = true) {
    if (!q || !k_cache || !v_cache || !o) return fail(FLUX_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be non-NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return fail(FLUX_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(FLUX_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(FLUX_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (in_dtype != FLUX_DTYPE_BF16 && in_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "in_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    if (out_dtype != FLUX_DTYPE_BF16 && out_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "out_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    DecodePlan p;
    int st = plan_decode(batch, hq, hkv, kv_len, head_dim, mode, block, sink_tokens, window_tokens, num_splits, &p);
    if (st != FLUX_OK) return st;
    if (in_dtype != FLUX_DTYPE_BF16) return fail(FLUX_ERR_UNSUPPORTED, "decode supports bfloat16 inputs only");
    if (!workspace || workspace_bytes < p.ws_bytes)
        return fail(FLUX_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(FLUX_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (!launch) return FLUX_OK;
    flux::DecodeArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.o = o;
    a.lse = lse;
    size_t rows = (size_t)batch * hq * p.n_split;
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                          align256(rows * head_dim * sizeof(float)));
    a.batch = batch;
    a.kv_len = kv_len;
    a.kv_cap = cache_rows;
    a.hq = hq;
    a.hkv = hkv;
    a.head_dim = head_dim;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out_f32 = out_dtype == FLUX_DTYPE_F32;
    a.r0_end = p.r0_end;
    a.r1_begin = p.r1_begin;
    a.n_active = p.n_active;
    a.n_split = p.n_split;
    a.split_len = p.split_len;
    a.ring = layout == FLUX_KV_WINDOW;
    a.sink_rows = sink_tokens;
    a.ring_blocks = window_tokens / flux::kBlock;
    a.k_new = k_new;
    a.v_new = v_new;
    hipError_t e = flux::launch_decode(a, as_stream(hip_stream));
    if (e == hipSuccess) e = hipGetLastError();
    return hip_status(e, "decode launch");
}

int check_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* o,
                      float* lse, int32_t out_dtype, int64_t batch, int64_t pos, int64_t cache_rows, int32_t layout,
                      int32_t hq, int32_t hkv, int32_t head_dim, float scale, int32_t mode, int32_t block,
                      int32_t sink_tokens, int32_t window_tokens, void* workspace, size_t workspace_bytes) {
    if (!k_new || !v_new) return fail(FLUX_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
    if (pos < 0) return fail(FLUX_ERR_INVALID_ARG, "pos must be >= 0");
    if (layout == FLUX_KV_FULL && cache_rows <= pos)
        return fail(FLUX_ERR_CAPACITY, "cache_rows %lld must exceed pos %lld", (long long)cache_rows, (long long)pos);
    if (layout == FLUX_KV_WINDOW && cache_rows == 0)
        return fail(FLUX_ERR_INVALID_ARG, "invalid block / sink / window for the window cache");
    return run_decode(q, k_cache, v_cache, k_new, v_new, o, lse, FLUX_DTYPE_BF16, out_dtype, batch, pos + 1,
                      cache_rows, layout, hq, hkv, head_dim, scale, mode, block, sink_tokens, window_tokens, 0,
                      workspace, workspace_bytes, nullptr, false);
}

}  // namespace

extern "C" {

const char* flux_status_string(int status) {
    switch (status) {
        case FLUX_OK: return "FLUX_OK";
        case FLUX_ERR_INVALID_ARG: return "FLUX_ERR_INVALID_ARG: an argument is outside its documented range";
        case FLUX_ERR_UNSUPPORTED: return "FLUX_ERR_UNSUPPORTED: shape or dtype not handled by this build";
        case FLUX_ERR_CAPACITY: return "FLUX_ERR_CAPACITY: output array too small";
        case FLUX_ERR_WORKSPACE: return "FLUX_ERR_WORKSPACE: workspace missing or too small";
        case FLUX_ERR_HIP: return "FLUX_ERR_HIP: HIP runtime or launch failure";
        default: return "unknown flux status";
    }
}

const char* flux_last_error_detail(void) { return g_detail; }

int flux_version(void) { return 100; }

int flux_build_block_mask(int64_t seq_q, int64_t seq_k, int32_t block, int32_t sink_tokens, int32_t window_tokens,
                          int32_t causal, int32_t mode, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          int64_t* nnz_out) {
    if (!nnz_out) return fail(FLUX_ERR_INVALID_ARG, "nnz_out must be non-NULL");
    MaskSpec ms;
    int st = check_mask_spec(seq_q, seq_k, block, sink_tokens, window_tokens, causal, mode, &ms);
    if (st != FLUX_OK) return st;
    int64_t nnz = mask_nnz(ms);
    if (nnz > INT32_MAX) return fail(FLUX_ERR_UNSUPPORTED, "mask has more than 2^31-1 active blocks");
    *nnz_out = nnz;
    if (!col_idx) {
        if (col_capacity != 0) return fail(FLUX_ERR_INVALID_ARG, "col_idx is NULL but col_capacity != 0");
        return ok();
    }
    if (!row_ptr) return fail(FLUX_ERR_INVALID_ARG, "row_ptr must be non-NULL when col_idx is given");
    if (col_capacity < nnz)
        return fail(FLUX_ERR_CAPACITY, "col_capacity %lld < nnz %lld", (long long)col_capacity, (long long)nnz);
    int64_t nbq = ceil_div(seq_q, block), pos = 0;
    for (int64_t I = 0; I < nbq; ++I) {
        row_ptr[I] = (int32_t)pos;
        int64_t lo, hb, he;
        row_ranges(ms, I, &lo, &hb, &he);
        for (int64_t J = 0; J < lo; ++J) col_idx[pos++] = (int32_t)J;
        for (int64_t J = hb; J <= he; ++J) col_idx[pos++] = (int32_t)J;
    }
    row_ptr[nbq] = (int32_t)pos;
    return ok();
}

int flux_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int32_t in_dtype,
                      int32_t out_dtype, int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                      float scale, int32_t causal, int32_t mode, int32_t block, int32_t sink_tokens,
                      int32_t window_tokens, const int32_t* blk_row_ptr, const int32_t* blk_col_idx, int64_t blk_nnz,
                      void* hip_stream) {
    flux::PrefillArgs a;
    int st = check_prefill(q, k, v, o, lse, in_dtype, out_dtype, batch, seq, hq, hkv, head_dim, scale, causal, mode,
                           block, sink_tokens, window_tokens, blk_row_ptr, blk_col_idx, blk_nnz, &a);
    if (st != FLUX_OK) return st;
    return launch_prefill(a, in_dtype, as_stream(hip_stream));
}

int flux_attn_prefill_layers(int32_t n_layers, const int32_t* modes_host, const void* const* q, const void* const* k,
                             const void* const* v, void* const* o, float* const* lse, int32_t in_dtype,
                             int32_t out_dtype, int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                             float scale, int32_t block, int32_t sink_tokens, int32_t window_tokens,
                             const int32_t* blk_row_ptr, const int32_t* blk_col_idx, int64_t blk_nnz,
                             void* hip_stream) {
    if (n_layers < 1) return fail(FLUX_ERR_INVALID_ARG, "n_layers must be >= 1");
    if (!modes_host || !q || !k || !v || !o) return fail(FLUX_ERR_INVALID_ARG, "layer arrays must be non-NULL");
    for (int32_t l = 0; l < n_layers; ++l) {
        flux::PrefillArgs a;
        int st = check_prefill(q[l], k[l], v[l], o[l], lse ? lse[l] : nullptr, in_dtype, out_dtype, batch, seq, hq,
                               hkv, head_dim, scale, 1, modes_host[l], block, sink_tokens, window_tokens, blk_row_ptr,
                               blk_col_idx, blk_nnz, &a);
        if (st != FLUX_OK) {
            char tmp[512];
            snprintf(tmp, sizeof tmp, "layer %d: %s", l, g_detail);
            return fail(st, "%s", tmp);
        }
    }
    for (int32_t l = 0; l < n_layers; ++l) {
        flux::PrefillArgs a;
        check_prefill(q[l], k[l], v[l], o[l], lse ? lse[l] : nullptr, in_dtype, out_dtype, batch, seq, hq, hkv,
                      head_dim, scale, 1, modes_host[l], block, sink_tokens, window_tokens, blk_row_ptr, blk_col_idx,
                      blk_nnz, &a);
        int st = launch_prefill(a, in_dtype, as_stream(hip_stream));
        if (st != FLUX_OK) return st;
    }
    return ok();
}

int flux_attn_prefill_layers_routed(int32_t n_layers, const int32_t* modes_device, const void* const* q,
                                    const void* const* k, const void* const* v, void* const* o, float* const* lse,
                                    int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t seq, int32_t hq,
                                    int32_t hkv, int32_t head_dim, float scale, int32_t block, int32_t sink_tokens,
                                    int32_t window_tokens, const int32_t* blk_row_ptr, const int32_t* blk_col_idx,
                                    int64_t blk_nnz, void* hip_stream) {
    if (n_layers < 1) return fail(FLUX_ERR_INVALID_ARG, "n_layers must be >= 1");
    if (!modes_device || !q || !k || !v || !o) return fail(FLUX_ERR_INVALID_ARG, "layer arrays must be non-NULL");
    if (reinterpret_cast<uintptr_t>(modes_device) & 3u)
        return fail(FLUX_ERR_INVALID_ARG, "modes_device must be 4-byte aligned");
    // every layer is validated as block-sparse (the stricter case: it needs the CSR); the
    // kernels read the layer's mode from modes_device[l] when they start
    for (int32_t l = 0; l < n_layers; ++l) {
        flux::PrefillArgs a;
        int st = check_prefill(q[l], k[l], v[l], o[l], lse ? lse[l] : nullptr, in_dtype, out_dtype, batch, seq, hq,
                               hkv, head_dim, scale, 1, FLUX_MODE_SPARSE, block, sink_tokens, window_tokens,
                               blk_row_ptr, blk_col_idx, blk_nnz, &a);
        if (st != FLUX_OK) {
            char tmp[512];
            snprintf(tmp, sizeof tmp, "layer %d: %s", l, g_detail);
            return fail(st, "%s", tmp);
        }
    }
    for (int32_t l = 0; l < n_layers; ++l) {
        flux::PrefillArgs a;
        check_prefill(q[l], k[l], v[l], o[l], lse ? lse[l] : nullptr, in_dtype, out_dtype, batch, seq, hq, hkv,
                      head_dim, scale, 1, FLUX_MODE_SPARSE, block, sink_tokens, window_tokens, blk_row_ptr,
                      blk_col_idx, blk_nnz, &a);
        a.mode_dev = modes_device + l;
        int st = launch_prefill(a, in_dtype, as_stream(hip_stream));
        if (st != FLUX_OK) return st;
    }
    return ok();
}

size_t flux_prefill_soft_workspace_size(int64_t batch, int64_t seq, int32_t hq, int32_t head_dim) {
    if (batch < 1 || seq < 1 || hq < 1 || head_dim < 1) return 0;
    return (size_t)batch * seq * hq * head_dim * sizeof(float);
}

int flux_attn_prefill_soft(const void* q, const void* k, const void* v, void* o, int32_t in_dtype, int32_t out_dtype,
                           int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                           int32_t block, int32_t sink_tokens, int32_t window_tokens, const int32_t* blk_row_ptr,
                           const int32_t* blk_col_idx, int64_t blk_nnz, const float* weights_device,
                           void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!weights_device || (reinterpret_cast<uintptr_t>(weights_device) & 3u))
        return fail(FLUX_ERR_INVALID_ARG, "weights_device must be a 4-byte aligned device pointer");
    if (in_dtype != FLUX_DTYPE_BF16) return fail(FLUX_ERR_UNSUPPORTED, "soft routing takes bfloat16 inputs");
    if (!workspace || !aligned16(workspace)) return fail(FLUX_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    // the CSR is optional here (the fused kernel walks the pattern from sink and window); when given it is
    // checked as in sparse mode
    flux::PrefillArgs a;
    int st;
    if (blk_row_ptr || blk_col_idx) {
        st = check_prefill(q, k, v, o, nullptr, in_dtype, out_dtype, batch, seq, hq, hkv, head_dim, scale, 1,
                           FLUX_MODE_SPARSE, block, sink_tokens, window_tokens, blk_row_ptr, blk_col_idx, blk_nnz, &a);
    } else {
        MaskSpec ms;
        st = check_mask_spec(seq, seq, block, sink_tokens, window_tokens, 1, FLUX_MODE_SPARSE, &ms);
        if (st == FLUX_OK)
            st = check_prefill(q, k, v, o, nullptr, in_dtype, out_dtype, batch, seq, hq, hkv, head_dim, scale, 1,
                               FLUX_MODE_DENSE, block, 0, 0, nullptr, nullptr, 0, &a);
        a.sink_blocks = sink_tokens / block;
        a.window_blocks = window_tokens / block;
    }
    if (st != FLUX_OK) return st;
    const size_t need = flux_prefill_soft_workspace_size(batch, seq, hq, head_dim);
    if (workspace_bytes < need)
        return fail(FLUX_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (workspace == o) return fail(FLUX_ERR_INVALID_ARG, "workspace must not alias o");
    // one launch: dense-causal walk ordered sink, window (descending), then the other blocks; each row's
    // block-sparse output is taken when its window ends, the mixture written at the end
    a.sparse = 0;
    a.row_ptr = nullptr;
    a.col_idx = nullptr;
    a.soft_ws = reinterpret_cast<float*>(workspace);
    a.mix_w = weights_device;
    return launch_prefill(a, in_dtype, as_stream(hip_stream));
}

// ---------------------------------------------------------------- backward
namespace {

struct BackwardLayout {
    size_t stat, counters, part, amax, exps, q16, k16, v16, do16, total;   // byte offsets, and the size
};

// Keys whose dK/dV the dK/dV kernel writes per query head (summed over the group afterwards): with
// grouped-query attention in block-sparse mode, the 128-key pairs holding sink blocks.
int64_t backward_part_keys(int64_t seq, int32_t hq, int32_t hkv, bool sparse, int64_t sink_blocks) {
    if (!sparse || hq == hkv || sink_blocks <= 0) return 0;
    const int64_t pairs = std::min(ceil_div(sink_blocks, 2), ceil_div(ceil_div(seq, 64), 2));
    return std::min(128 * pairs, seq);
}

BackwardLayout backward_layout(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                               int64_t part_keys) {
    BackwardLayout w;
    const int64_t nqb = ceil_div(seq, 64);
    w.stat = 0;
    w.counters = align256((size_t)batch * hq * nqb * 128 * sizeof(float));
    w.part = w.counters + 256;
    const size_t part_bytes = (size_t)batch * part_keys * hq * head_dim * sizeof(float);
    w.amax = w.part + 2 * align256(part_bytes);
    w.exps = w.amax + align256((size_t)4 * batch * hkv * flux::kAbsmaxChunks * sizeof(uint32_t));
    w.q16 = w.exps + align256((size_t)4 * batch * hkv * sizeof(int));
    const size_t qb = align256((size_t)batch * seq * hq * head_dim * 2), kb = align256((size_t)batch * seq * hkv * head_dim * 2);
    w.k16 = w.q16 + qb;
    w.v16 = w.k16 + kb;
    w.do16 = w.v16 + kb;
    w.total = w.do16 + qb;
    return w;
}

}  // namespace

size_t flux_attn_backward_workspace_size(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                                         int32_t mode, int32_t block, int32_t sink_tokens) {
    if (batch < 1 || seq < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || head_dim < 1) return 0;
    if (mode != FLUX_MODE_DENSE && mode != FLUX_MODE_SPARSE) return 0;
    if (block < 1 || sink_tokens < 0 || sink_tokens % block != 0) return 0;
    const int64_t pk = backward_part_keys(seq, hq, hkv, mode == FLUX_MODE_SPARSE, sink_tokens / block);
    return backward_layout(batch, seq, hq, hkv, head_dim, pk).total;
}

int flux_attn_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                       float* dq, float* dk, float* dv, int32_t in_dtype, int32_t o_dtype, int64_t batch,
                       int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim, float scale, int32_t causal,
                       int32_t mode, int32_t block, int32_t sink_tokens, int32_t window_tokens, void* workspace,
                       size_t workspace_bytes, void* hip_stream) {
    if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv)
        return fail(FLUX_ERR_INVALID_ARG, "q, k, v, o, d_o, lse, dq, dk and dv must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return fail(FLUX_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FLUX_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (batch < 1 || seq < 1) return fail(FLUX_ERR_INVALID_ARG, "batch and seq must be >= 1");
    if (hq < 1 || hkv < 1 || hq % hkv != 0)
        return fail(FLUX_ERR_INVALID_ARG, "hq (%d) must be a positive multiple of hkv (%d)", hq, hkv);
    if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(FLUX_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (in_dtype != FLUX_DTYPE_BF16 && in_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "in_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    if (o_dtype != FLUX_DTYPE_BF16 && o_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "o_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    MaskSpec ms;
    int st = check_mask_spec(seq, seq, block, sink_tokens, window_tokens, causal, mode, &ms);
    if (st != FLUX_OK) return st;
    if (head_dim != 64 && head_dim != 128)
        return fail(FLUX_ERR_UNSUPPORTED, "head_dim %d not supported by the backward pass (64 or 128)", head_dim);
    if (block != flux::kBlock) return fail(FLUX_ERR_UNSUPPORTED, "block %d not supported (64)", block);
    if (batch * (int64_t)hq * ceil_div(seq, 64) * 64 > INT32_MAX)
        return fail(FLUX_ERR_UNSUPPORTED, "batch * hq * seq exceeds the work-unit range");
    if (seq * (int64_t)std::max(hq, hkv) * head_dim > INT32_MAX)
        return fail(FLUX_ERR_UNSUPPORTED, "seq * max(hq, hkv) * head_dim must stay below 2^31 elements");
    if (in_dtype == FLUX_DTYPE_BF16 && batch * hkv > 65535)
        return fail(FLUX_ERR_UNSUPPORTED, "batch * hkv must stay below 65536 (one scale group per KV head)");
    const int64_t part_keys = backward_part_keys(seq, hq, hkv, ms.sparse && causal, ms.sink_blocks);
    const BackwardLayout w = backward_layout(batch, seq, hq, hkv, head_dim, part_keys);
    if (!workspace || workspace_bytes < w.total)
        return fail(FLUX_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(FLUX_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (dk == dv || dq == dk || dq == dv) return fail(FLUX_ERR_INVALID_ARG, "dq, dk and dv must be distinct");
    flux::BackwardArgs a;
    char* ws = reinterpret_cast<char*>(workspace);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.d_o = d_o;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.stat = reinterpret_cast<float*>(ws + w.stat);
    a.counters = reinterpret_cast<int*>(ws + w.counters);
    if (part_keys > 0) {
        const size_t pb = align256((size_t)batch * part_keys * hq * head_dim * sizeof(float));
        a.dk_part = reinterpret_cast<float*>(ws + w.part);
        a.dv_part = reinterpret_cast<float*>(ws + w.part + pb);
    } else {
        a.dk_part = nullptr;
        a.dv_part = nullptr;
    }
    a.part_keys = part_keys;
    a.amax = reinterpret_cast<uint32_t*>(ws + w.amax);
    a.exps = reinterpret_cast<int*>(ws + w.exps);
    a.q16 = ws + w.q16;
    a.k16 = ws + w.k16;
    a.v16 = ws + w.v16;
    a.do16 = ws + w.do16;
    a.batch = batch;
    a.seq = seq;
    a.hq = hq;
    a.hkv = hkv;
    a.head_dim = head_dim;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.causal = causal;
    a.sparse = ms.sparse ? 1 : 0;
    a.sink_blocks = (int)ms.sink_blocks;
    a.window_blocks = (int)ms.window_blocks;
    a.n_qblk = (int)ceil_div(seq, 64);
    a.num_cu = device_cu_count();
    a.o_f32 = o_dtype == FLUX_DTYPE_F32;
    a.in_f32 = in_dtype == FLUX_DTYPE_F32;
    hipError_t e = flux::launch_backward(a, as_stream(hip_stream));
    if (e == hipSuccess) e = hipGetLastError();
    return hip_status(e, "backward launch");
}

int flux_route_soft_weights(const float* logits, const float* uniforms, float tau, int32_t n_layers,
                            float* weights_out, void* hip_stream) {
    if (!logits || !uniforms || !weights_out) return fail(FLUX_ERR_INVALID_ARG, "pointers must be non-NULL");
    if (n_layers < 1) return fail(FLUX_ERR_INVALID_ARG, "n_layers must be >= 1");
    if (!(tau > 0.0f) || !std::isfinite(tau)) return fail(FLUX_ERR_INVALID_ARG, "tau must be finite and > 0");
    hipError_t e = flux::launch_route_soft(logits, uniforms, tau, n_layers, weights_out, as_stream(hip_stream));
    if (e == hipSuccess) e = hipGetLastError();
    return hip_status(e, "soft routing launch");
}

size_t flux_decode_workspace_size(int64_t batch, int32_t hq, int32_t hkv, int64_t kv_len, int32_t head_dim,
                                  int32_t mode, int32_t block, int32_t sink_tokens, int32_t window_tokens,
                                  int32_t num_splits) {
    DecodePlan p;
    if (plan_decode(batch, hq, hkv, kv_len, head_dim, mode, block, sink_tokens, window_tokens, num_splits, &p) !=
        FLUX_OK)
        return 0;
    return p.ws_bytes;
}

int flux_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int32_t in_dtype,
                     int32_t out_dtype, int64_t batch, int64_t kv_len, int64_t kv_capacity, int32_t hq, int32_t hkv,
                     int32_t head_dim, float scale, int32_t mode, int32_t block, int32_t sink_tokens,
                     int32_t window_tokens, int32_t num_splits, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
    if (kv_capacity == 0) kv_capacity = kv_len;
    if (kv_capacity < kv_len) return fail(FLUX_ERR_INVALID_ARG, "kv_capacity must be 0 or >= kv_len");
    return run_decode(q, k_cache, v_cache, nullptr, nullptr, o, lse, in_dtype, out_dtype, batch, kv_len, kv_capacity,
                      FLUX_KV_FULL, hq, hkv, head_dim, scale, mode, block, sink_tokens, window_tokens, num_splits,
                      workspace, workspace_bytes, hip_stream);
}

int flux_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                             int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t kv_len, int64_t kv_capacity,
                             int32_t hq, int32_t hkv, int32_t head_dim, float scale, int32_t mode, int32_t block,
                             int32_t sink_tokens, int32_t window_tokens, int32_t num_splits, void* hip_stream) {
    static_assert(flux::kDecodeScratchBytes == (size_t)FLUX_DECODE_SCRATCH_BYTES, "scratch size");
    if (kv_capacity == 0) kv_capacity = kv_len;
    if (kv_capacity < kv_len) return fail(FLUX_ERR_INVALID_ARG, "kv_capacity must be 0 or >= kv_len");
    DecodePlan p;
    int st = plan_decode(batch, hq, hkv, kv_len, head_dim, mode, block, sink_tokens, window_tokens, num_splits, &p);
    if (st != FLUX_OK) return st;
    if (p.ws_bytes > flux::kDecodeScratchBytes)
        return fail(FLUX_ERR_CAPACITY,
                    "the split partials need %zu bytes, more than the %zu-byte scratch of the no-allocation "
                    "decode (fewer sequences, query heads or splits per call, or flux_attn_decode with a workspace)",
                    p.ws_bytes, flux::kDecodeScratchBytes);
    // every other argument is validated before the scratch lookup (the first HIP call); the placeholder
    // stands for the scratch in that check only and is never dereferenced
    void* const validate_only_ws = reinterpret_cast<void*>(uintptr_t(256));
    st = run_decode(q, k_cache, v_cache, nullptr, nullptr, o, lse, in_dtype, out_dtype, batch, kv_len, kv_capacity,
                    FLUX_KV_FULL, hq, hkv, head_dim, scale, mode, block, sink_tokens, window_tokens, num_splits,
                    validate_only_ws, flux::kDecodeScratchBytes, hip_stream, false);
    if (st != FLUX_OK) return st;
    void* scratch = nullptr;
    hipError_t e = flux::decode_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "decode scratch lookup");
    return run_decode(q, k_cache, v_cache, nullptr, nullptr, o, lse, in_dtype, out_dtype, batch, kv_len, kv_capacity,
                      FLUX_KV_FULL, hq, hkv, head_dim, scale, mode, block, sink_tokens, window_tokens, num_splits,
                      scratch, flux::kDecodeScratchBytes, hip_stream);
}

int64_t flux_window_cache_rows(int32_t block, int32_t sink_tokens, int32_t window_tokens) {
    if (block != flux::kBlock || sink_tokens < 0 || window_tokens < block || sink_tokens % block ||
        window_tokens % block)
        return 0;
    return (int64_t)sink_tokens + window_tokens;
}

int flux_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* o,
                     float* lse, int32_t out_dtype, int64_t batch, int64_t pos, int64_t cache_rows, int32_t layout,
                     int32_t hq, int32_t hkv, int32_t head_dim, float scale, int32_t mode, int32_t block,
                     int32_t sink_tokens, int32_t window_tokens, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
    if (!k_new || !v_new) return fail(FLUX_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(FLUX_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    if (pos < 0) return fail(FLUX_ERR_INVALID_ARG, "pos must be >= 0");
    if (layout == FLUX_KV_FULL) {
        if (cache_rows <= pos) return fail(FLUX_ERR_CAPACITY, "cache_rows %lld must exceed pos %lld",
                                           (long long)cache_rows, (long long)pos);
    } else if (layout == FLUX_KV_WINDOW) {
        if (mode != FLUX_MODE_SPARSE) return fail(FLUX_ERR_INVALID_ARG, "the window cache holds sparse layers only");
        const int64_t rows = flux_window_cache_rows(block, sink_tokens, window_tokens);
        if (rows == 0 || cache_rows != rows)
            return fail(FLUX_ERR_INVALID_ARG, "window cache must have sink_tokens + window_tokens = %lld rows",
                        (long long)rows);
    } else {
        return fail(FLUX_ERR_INVALID_ARG, "layout must be FLUX_KV_FULL or FLUX_KV_WINDOW");
    }
    return run_decode(q, k_cache, v_cache, k_new, v_new, o, lse, FLUX_DTYPE_BF16, out_dtype, batch, pos + 1,
                      cache_rows, layout, hq, hkv, head_dim, scale, mode, block, sink_tokens, window_tokens,
                      num_splits, workspace, workspace_bytes, hip_stream);
}

int flux_decode_step_layers(int32_t n_layers, const int32_t* modes_host, const void* const* q,
                            const void* const* k_new, const void* const* v_new, void* const* k_cache,
                            void* const* v_cache, void* const* o, float* const* lse, int32_t out_dtype, int64_t batch,
                            int64_t pos, int64_t dense_cache_rows, int32_t hq, int32_t hkv, int32_t head_dim,
                            float scale, int32_t block, int32_t sink_tokens, int32_t window_tokens, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
    if (n_layers < 1) return fail(FLUX_ERR_INVALID_ARG, "n_layers must be >= 1");
    if (!modes_host || !q || !k_new || !v_new || !k_cache || !v_cache || !o)
        return fail(FLUX_ERR_INVALID_ARG, "layer arrays must be non-NULL");
    const int64_t wrows = flux_window_cache_rows(block, sink_tokens, window_tokens);
    for (int pass = 0; pass < 2; ++pass) {   // pass 0 validates every layer, pass 1 launches
        for (int32_t l = 0; l < n_layers; ++l) {
            const int32_t m = modes_host[l];
            if (m != FLUX_MODE_DENSE && m != FLUX_MODE_SPARSE)
                return fail(FLUX_ERR_INVALID_ARG, "layer %d: mode %d is neither dense nor sparse", l, m);
            const int32_t layout = m == FLUX_MODE_SPARSE ? FLUX_KV_WINDOW : FLUX_KV_FULL;
            const int64_t rows = m == FLUX_MODE_SPARSE ? wrows : dense_cache_rows;
            int st;
            if (pass == 0) {
                st = check_decode_step(q[l], k_new[l], v_new[l], k_cache[l], v_cache[l], o[l], lse ? lse[l] : nullptr,
                                       out_dtype, batch, pos, rows, layout, hq, hkv, head_dim, scale, m, block,
                                       sink_tokens, window_tokens, workspace, workspace_bytes);
            } else {
                st = flux_decode_step(q[l], k_new[l], v_new[l], k_cache[l], v_cache[l], o[l], lse ? lse[l] : nullptr,
                                      out_dtype, batch, pos, rows, layout, hq, hkv, head_dim, scale, m, block,
                                      sink_tokens, window_tokens, 0, workspace, workspace_bytes, hip_stream);
            }
            if (st != FLUX_OK) {
                char tmp[512];
                snprintf(tmp, sizeof tmp, "layer %d: %s", l, g_detail);
                return fail(st, "%s", tmp);
            }
        }
    }
    return ok();
}

size_t flux_route_workspace_size(int32_t n_layers, int32_t hq, int32_t head_dim, int32_t hidden) {
    if (n_layers < 1 || hq < 1 || head_dim < 1 || hidden < 1) return 0;
    const size_t nf = (size_t)hq * head_dim;
    return align256((size_t)n_layers * nf * sizeof(float)) + align256((size_t)n_layers * hidden * sizeof(float)) +
           align256((size_t)n_layers * sizeof(int32_t));
}

int flux_route_layers(const void* const* q_layers, int32_t n_layers, int64_t seq, int32_t hq, int32_t head_dim,
                      int32_t in_dtype, int32_t pool_tokens, const float* w_enc, const float* b_enc, int32_t hidden,
                      const float* w_head, const float* b_head, float* logits_out, int32_t* modes_out,
                      void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!q_layers || n_layers < 1) return fail(FLUX_ERR_INVALID_ARG, "q_layers must hold n_layers >= 1 pointers");
    if (!w_enc || !b_enc || !w_head || !b_head || !modes_out)
        return fail(FLUX_ERR_INVALID_ARG, "weights and modes_out must be non-NULL");
    for (int32_t l = 0; l < n_layers; ++l) {
        if (!q_layers[l]) return fail(FLUX_ERR_INVALID_ARG, "q_layers[%d] is NULL", l);
        if (!aligned16(q_layers[l])) return fail(FLUX_ERR_INVALID_ARG, "q_layers[%d] must be 16-byte aligned", l);
    }
    if (seq < 1 || hq < 1 || head_dim < 1 || hidden < 1 || pool_tokens < 1)
        return fail(FLUX_ERR_INVALID_ARG, "seq, hq, head_dim, hidden and pool_tokens must be >= 1");
    if (in_dtype != FLUX_DTYPE_BF16 && in_dtype != FLUX_DTYPE_F32)
        return fail(FLUX_ERR_INVALID_ARG, "in_dtype must be FLUX_DTYPE_BF16 or FLUX_DTYPE_F32");
    const int64_t nf = (int64_t)hq * head_dim;
    if (nf % 8 != 0 || nf > (1 << 24)) return fail(FLUX_ERR_UNSUPPORTED, "hq*head_dim must be a multiple of 8");
    if (!aligned16(w_enc)) return fail(FLUX_ERR_INVALID_ARG, "w_enc must be 16-byte aligned");
    const size_t need = flux_route_workspace_size(n_layers, hq, head_dim, hidden);
    if (!workspace || workspace_bytes < need)
        return fail(FLUX_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(FLUX_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    float* pooled = reinterpret_cast<float*>(workspace);
    float* z = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                        align256((size_t)n_layers * nf * sizeof(float)));
    int32_t* counters = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(z) +
                                                   align256((size_t)n_layers * hidden * sizeof(float)));
    for (int32_t l0 = 0; l0 < n_layers; l0 += flux::kMaxRouteLayers) {
        flux::RouteArgs a;
        a.n_layers = std::min(n_layers - l0, flux::kMaxRouteLayers);
        for (int i = 0; i < a.n_layers; ++i) a.xq[i] = q_layers[l0 + i];
        a.layer0 = l0;
        a.seq = seq;
        a.n_feat = (int)nf;
        a.in_f32 = in_dtype == FLUX_DTYPE_F32;
        a.pool_tokens = pool_tokens;
        a.w_enc = w_enc;
        a.b_enc = b_enc;
        a.hidden = hidden;
        a.w_head = w_head;
        a.b_head = b_head;
        a.logits = logits_out;
        a.modes = modes_out;
        a.pooled = pooled;
        a.z = z;
        a.counters = counters;
        hipError_t e = flux::launch_route(a, as_stream(hip_stream));
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e, "router launch");
    }
    return ok();
}

}  // extern "C"
