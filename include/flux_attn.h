/*
 * flux_attn.h -- C ABI of the MI355X (gfx950) tiled attention library.
 *
 * Exact softmax attention computed tile by tile with an online softmax
 * (running row maximum and running row sum; earlier partial results are
 * rescaled by exp(m_old - m_new) when the maximum grows), in the two per-layer
 * modes of Flux Attention:
 *   - FLUX_MODE_DENSE  ("full attention", router index 0): every causal key;
 *   - FLUX_MODE_SPARSE ("sparse attention", router index 1): 64x64 blocks, an
 *     always-kept sink of leading blocks and a causal local window of blocks;
 *     blocks outside that set are skipped and their K/V are never read.
 *
 * Sources (pages on the method):
 *   [FA]  "Flux Attention: context-aware hybrid attention for efficient LLM
 *         inference" (aitrends.kr): router paragraphs (prefix/suffix pooling of
 *         xQ [s x h x d'], MLP context encoder, router head with logits
 *         (pi_FA, pi_SA), argmax at inference), layer-granularity paragraph,
 *         architecture paragraph (KV loading bypassed in sparse mode) and
 *         implementation paragraph (64-granular blocks, 128-token sink).
 *   [NL]  openads.co.kr FlashAttention newsletter: sections "Softmax is not a
 *         simple function" (attention definition), "The hidden cost of
 *         numerical stability" (max subtraction), "FlashAttention: reduce memory
 *         movement" (tiling, one HBM round trip) and "Online Softmax".
 *   [SA]  "After self-attention: what comes after transformers"
 *         (datadaily.news): "why self-attention is expensive" (plain attention
 *         with scale 1/sqrt(d_k); tensors (batch, seq_len, d_model)) and the
 *         hybrid-architectures section (sliding window, cost O(N*W)).
 *
 * Conventions for every entry point:
 *   - Returns an int status (FLUX_OK = 0); never throws; never allocates
 *     device memory; never synchronizes the stream unless stated.
 *   - All arguments are validated on the host before any launch; on failure
 *     nothing is written to any output and flux_last_error_detail() names the
 *     offending argument.
 *   - Device buffers are owned by the caller.  Results are valid once the
 *     caller has synchronized `hip_stream` (a hipStream_t; NULL = the default
 *     stream of the current device).
 *   - Tensors are dense row-major.  Sizes are 64-bit where they scale with
 *     sequence length.
 *   - Device pointers to bf16/f32 tensors must be 16-byte aligned.
 */
#ifndef FLUX_ATTN_H
#define FLUX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define FLUX_OK 0
#define FLUX_ERR_INVALID_ARG 1 /* a pointer, size or flag is outside its documented range  */
#define FLUX_ERR_UNSUPPORTED 2 /* valid request, but not a shape/dtype this build handles  */
#define FLUX_ERR_CAPACITY 3    /* an output array is too small (required size reported)   */
#define FLUX_ERR_WORKSPACE 4   /* workspace missing or smaller than the required size      */
#define FLUX_ERR_HIP 5         /* a HIP runtime call or kernel launch failed                */

/* ---- element types ----------------------------------------------------- */
#define FLUX_DTYPE_BF16 0
#define FLUX_DTYPE_F32 1

/* ---- per-layer attention modes (router argmax index, [FA]) -------------- */
#define FLUX_MODE_DENSE 0  /* pi_FA: full (dense) attention   */
#define FLUX_MODE_SPARSE 1 /* pi_SA: block-sparse attention   */

/* ---- KV-cache layouts (decode) ----------------------------------------- */
#define FLUX_KV_FULL 0   /* [batch, rows, hkv, head_dim]: token t at row t                       */
#define FLUX_KV_WINDOW 1 /* [batch, sink+window, hkv, head_dim]: token t < sink at row t; a later  \
                            token t at row sink + ((t/64) mod (window/64))*64 + t mod 64 (a ring  \
                            of window blocks; a block's slot is reused once it has left the window) */

/* Static text for a status code (never NULL). */
const char* flux_status_string(int status);

/* Thread-local text describing the most recent failure on this thread: which
 * argument was rejected, or the HIP error string.  Empty after success. */
const char* flux_last_error_detail(void);

/* Library ABI version (major * 100 + minor). */
int flux_version(void);

/*
 * flux_build_block_mask -- list the active key blocks of every query block.
 *
 * Defines the block-sparse pattern of [FA] implementation paragraph: key and
 * query positions are cut into blocks of `block` tokens (64 in the method);
 * with mode == FLUX_MODE_SPARSE, key block J is active for query block I iff
 *     J <= I  and  ( J < sink_tokens/block  or  I - J < window_tokens/block ),
 * i.e. the always-kept sink blocks plus a causal local window of blocks that
 * ends at (and includes) the query's own block ([SA] sliding window).  With
 * mode == FLUX_MODE_DENSE every causal block (J <= I), or every block when
 * causal == 0, is active and sink/window are ignored.
 *
 * Host-only and bit-exact; touches no device.  Output is CSR:
 *   row_ptr [nbq + 1] int32 (nbq = ceil(seq_q / block)), row_ptr[0] = 0;
 *   col_idx [nnz] int32, ascending within each row.
 * col_idx may be NULL (with col_capacity 0) to ask only for *nnz_out; row_ptr
 * may then be NULL too.  If col_capacity < nnz the call returns
 * FLUX_ERR_CAPACITY, writes *nnz_out and leaves row_ptr/col_idx unspecified.
 * Requires: seq_q, seq_k >= 1; block >= 1; sparse mode: causal == 1,
 * sink_tokens >= 0 and window_tokens >= block, both multiples of block.
 */
int flux_build_block_mask(int64_t seq_q, int64_t seq_k, int32_t block, int32_t sink_tokens,
                          int32_t window_tokens, int32_t causal, int32_t mode, int32_t* row_ptr,
                          int32_t* col_idx, int64_t col_capacity, int64_t* nnz_out);

/*
 * flux_attn_prefill -- one layer of tiled attention for all heads.
 *
 * O = softmax(scale * Q K^T + mask) V per (batch, query head) ([NL] attention
 * definition; [SA] scale 1/sqrt(d_k)), computed tile by tile with an online
 * softmax ([NL] "Online Softmax"); the score matrix is never written.
 *   q   [batch, seq, hq,  head_dim]   device, in_dtype
 *   k,v [batch, seq, hkv, head_dim]   device, in_dtype
 *   o   [batch, seq, hq,  head_dim]   device, out_dtype
 *   lse [batch, hq, seq] float32 natural-log sum-exp of the scaled scores, or NULL
 * Query head h reads KV head h / (hq / hkv) (grouped-query attention).
 * mode == FLUX_MODE_DENSE: causal (key <= query) if causal != 0, else all keys.
 * mode == FLUX_MODE_SPARSE: requires causal == 1.  The active key blocks are
 *   those flux_build_block_mask(seq, seq, block, sink_tokens, window_tokens,
 *   1, FLUX_MODE_SPARSE, ...) lists.  Either pass that device CSR
 *   (blk_row_ptr [nbq+1], blk_col_idx [blk_nnz], int32; blk_nnz is checked
 *   against the pattern) and the kernels walk it, or pass both NULL and the
 *   kernels derive the same blocks from (sink_tokens, window_tokens) with
 *   integer arithmetic (no per-tile index loads; bit-identical results).
 *   Inside an active block every key is visible except keys after the query
 *   in the diagonal block.  Dense mode ignores the CSR arguments.
 * Supported: (in, out) = (BF16, BF16), (BF16, F32), (F32, F32);
 * head_dim in {64, 128}; block == 64; hq % hkv == 0; scale finite and > 0.
 */
int flux_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                      int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t seq, int32_t hq,
                      int32_t hkv, int32_t head_dim, float scale, int32_t causal, int32_t mode,
                      int32_t block, int32_t sink_tokens, int32_t window_tokens,
                      const int32_t* blk_row_ptr, const int32_t* blk_col_idx, int64_t blk_nnz,
                      void* hip_stream);

/*
 * flux_attn_prefill_layers -- per-layer dispatch of a routed layer stack.
 *
 * One mode per layer, never mixed across heads ([FA] layer-granularity
 * paragraph).  For layer l, runs flux_attn_prefill(q[l], k[l], v[l], o[l],
 * lse ? lse[l] : NULL, ..., causal = 1, mode = modes_host[l], ...) on
 * `hip_stream`.  modes_host is a HOST array of n_layers entries (the router
 * output copied to the host).  All layers share shape, dtypes, block, sink,
 * window and the optional sparse CSR (as for flux_attn_prefill: the CSR, or
 * both pointers NULL).  Layers are validated before the first launch.
 */
int flux_attn_prefill_layers(int32_t n_layers, const int32_t* modes_host, const void* const* q,
                             const void* const* k, const void* const* v, void* const* o,
                             float* const* lse, int32_t in_dtype, int32_t out_dtype, int64_t batch,
                             int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                             int32_t block, int32_t sink_tokens, int32_t window_tokens,
                             const int32_t* blk_row_ptr, const int32_t* blk_col_idx, int64_t blk_nnz,
                             void* hip_stream);

/*
 * flux_attn_prefill_layers_routed -- per-layer dispatch driven by the router's
 * DEVICE output, with no host round trip.
 *
 * Same as flux_attn_prefill_layers, except that the mode of layer l is read by
 * the prefill kernels themselves from modes_device[l] (device int32, as written
 * by flux_route_layers into modes_out: 0 = dense causal, any other value =
 * block-sparse) when they start.  The router ([FA] router paragraphs: argmax of
 * the router head at inference) and the attention of the layer therefore run
 * back to back on `hip_stream`; the host never waits for the mode.  Because
 * any layer may turn out sparse, every layer is validated as for
 * FLUX_MODE_SPARSE (the CSR arguments: that CSR, or both NULL to derive the
 * blocks from sink and window).  modes_device must stay valid until the
 * launches have run.
 */
int flux_attn_prefill_layers_routed(int32_t n_layers, const int32_t* modes_device,
                                    const void* const* q, const void* const* k,
                                    const void* const* v, void* const* o, float* const* lse,
                                    int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t seq,
                                    int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                                    int32_t block, int32_t sink_tokens, int32_t window_tokens,
                                    const int32_t* blk_row_ptr, const int32_t* blk_col_idx,
                                    int64_t blk_nnz, void* hip_stream);

/*
 * flux_route_soft_weights -- Gumbel-softmax routing weights of the training-time
 * relaxation ([FA] router paragraph): for each layer l,
 *   g_i = -ln(-ln u[l][i]),  w[l][i] = exp((pi[l][i] + g_i) / tau) / sum_j exp((pi[l][j] + g_j) / tau)
 * over i in {0 = FA, 1 = SA}.  logits [n_layers, 2] (e.g. flux_route_layers' logits_out), uniforms
 * [n_layers, 2] in (0, 1) (the random draw, supplied by the caller) and weights_out [n_layers, 2]:
 * device float32.  tau > 0 and finite.
 */
int flux_route_soft_weights(const float* logits, const float* uniforms, float tau, int32_t n_layers,
                            float* weights_out, void* hip_stream);

/* flux_prefill_soft_workspace_size -- bytes flux_attn_prefill_soft needs (an fp32 [B, S, Hq, d] buffer,
 * 16-byte aligned). */
size_t flux_prefill_soft_workspace_size(int64_t batch, int64_t seq, int32_t hq, int32_t head_dim);

/*
 * flux_attn_prefill_soft -- soft-routed layer output for training ([FA] router paragraph: the full
 * and sparse attention outputs weighted by the Gumbel-softmax probabilities):
 *   o = w[0] * attention(dense causal) + w[1] * attention(block-sparse)
 * with weights_device [2] device float32 (one row of flux_route_soft_weights' output).  One launch:
 * the dense-causal pass visits each row's sink and window blocks first, takes the row's block-sparse
 * output there (into `workspace`, fp32) and mixes both at the end, so the blocks the two modes share
 * are computed once.  Inputs BF16; out_dtype BF16 or F32.  The block pattern is the one of
 * flux_build_block_mask(seq, seq, block, sink_tokens, window_tokens, 1, FLUX_MODE_SPARSE); the CSR
 * arguments may be NULL (with blk_nnz ignored) or that CSR, which is then checked as for
 * flux_attn_prefill in sparse mode.  No LSE (the output is a mixture of two softmaxes).
 */
int flux_attn_prefill_soft(const void* q, const void* k, const void* v, void* o, int32_t in_dtype,
                           int32_t out_dtype, int64_t batch, int64_t seq, int32_t hq, int32_t hkv,
                           int32_t head_dim, float scale, int32_t block, int32_t sink_tokens,
                           int32_t window_tokens, const int32_t* blk_row_ptr,
                           const int32_t* blk_col_idx, int64_t blk_nnz,
                           const float* weights_device, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/* flux_attn_backward_workspace_size -- bytes flux_attn_backward needs for these sizes and this mask
 * (0 if invalid): per-row statistics (fp32 [batch, hq, ceil(seq/64)*64, 2]), two counters, with
 * grouped-query attention in block-sparse mode two fp32 [batch, K, hq, head_dim] per-query-head dK/dV
 * buffers for the K = min(seq, 128 * ceil(sink_blocks / 2)) keys of the key pairs holding sink blocks
 * (every query sees them, so they are not grouped by KV head), and for bf16 inputs fp16 copies of
 * q, k, v and d_o (2 * batch * seq * (hq + hkv) * head_dim * 2 bytes) with their per-KV-head scales
 * (the size covers them for either input type).  mode, block and sink_tokens as passed to
 * flux_attn_backward. */
size_t flux_attn_backward_workspace_size(int64_t batch, int64_t seq, int32_t hq, int32_t hkv,
                                         int32_t head_dim, int32_t mode, int32_t block, int32_t sink_tokens);

/*
 * flux_attn_backward -- gradients of one layer of attention with respect to Q, K and V.
 *
 * For O = softmax(scale Q K^T + mask) V (the forward of flux_attn_prefill, same mask arguments)
 * and an output gradient dO, per (batch, query head), with P the row probabilities:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
 *   dQ = scale dS K,  dK = scale dS^T Q
 * (chain rule through the softmax of the [NL] attention definition; the gradients the [FA]
 * router training over a frozen backbone needs).  P is rebuilt tile by tile from Q, K and the
 * forward pass's lse; inactive blocks of the sparse pattern are skipped and never read.  With
 * grouped-query attention the query heads sharing a KV head add into its dK/dV (head order).
 *   q, d_o    [batch, seq, hq,  head_dim]  device, in_dtype (d_o: dL/dO)
 *   o         [batch, seq, hq,  head_dim]  device, o_dtype BF16 or F32: the forward output (only
 *                                          D = rowsum(dO * O) reads it; an fp32 O keeps D exact
 *                                          to fp32, a bf16 O perturbs D by its rounding)
 *   k, v      [batch, seq, hkv, head_dim]  device, in_dtype
 *   lse       [batch, hq, seq]             device fp32, as written by flux_attn_prefill
 *   dq        [batch, seq, hq,  head_dim]  device fp32 (written)
 *   dk, dv    [batch, seq, hkv, head_dim]  device fp32 (written, not accumulated into)
 * mode, causal, block, sink_tokens, window_tokens: as for flux_attn_prefill; the sparse key set
 * is derived from (block, sink_tokens, window_tokens), the pattern flux_build_block_mask builds.
 * workspace: device, >= flux_attn_backward_workspace_size(...) bytes, 16-byte aligned; its
 * contents on entry do not matter.  Deterministic: no atomics on gradients, fixed summation order.
 * in_dtype BF16: q, k, v, d_o bf16, matrix-core kernels on fp16 operands with fp32 accumulation:
 * the inputs are copied to fp16 scaled by a power of two per (batch, KV head) and tensor (exact for
 * every value above 2^-29 of its group's largest; smaller ones may be flushed), S and dP are the
 * products of those copies, and P and dS enter the gradient products rounded once to fp16.  The
 * scales stay in fp32's range as long as max|Q| * max|K| and max|dO| * max|V| over each KV head's
 * group lie in [2^-90, 2^150] (inputs must be finite).  in_dtype F32: q, k, v, d_o float32, vector-ALU kernels for small layers (as the
 * float32 forward).
 * Supported: head_dim 64 or 128, block 64; bf16 inputs: batch * hkv < 65536.
 */
int flux_attn_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                       const float* lse, float* dq, float* dk, float* dv, int32_t in_dtype,
                       int32_t o_dtype, int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                       float scale, int32_t causal, int32_t mode, int32_t block,
                       int32_t sink_tokens, int32_t window_tokens, void* workspace,
                       size_t workspace_bytes, void* hip_stream);

/*
 * flux_decode_workspace_size -- bytes of workspace flux_attn_decode needs.
 * Same meaning of arguments as flux_attn_decode (num_splits = 0: automatic;
 * the automatic split count depends on batch * hkv, so hkv is needed here).
 * Returns 0 if the arguments are invalid or unsupported.
 */
size_t flux_decode_workspace_size(int64_t batch, int32_t hq, int32_t hkv, int64_t kv_len,
                                  int32_t head_dim, int32_t mode, int32_t block,
                                  int32_t sink_tokens, int32_t window_tokens, int32_t num_splits);

/*
 * flux_attn_decode -- single-token GQA decode with split-KV partials.
 *
 * One new query per sequence at position kv_len-1, whose own K/V are already
 * in the cache; its allowed keys are those of prefill row kv_len-1 (dense:
 * all kv_len keys; sparse: the sink blocks and the window blocks ending at the
 * query's block -- inactive cache blocks are never read, [FA] architecture
 * paragraph).  The active keys are cut into `num_splits` chunks (0 = chosen by
 * the library); each chunk's partial result (O_s, lse_s) goes to the
 * workspace and a second kernel merges them with the online-softmax rule
 * ([NL] "Online Softmax"): LSE = M + ln sum_s exp(lse_s - M), O = sum_s
 * exp(lse_s - LSE) O_s, with empty chunks weighted 0.
 *   q       [batch, hq, head_dim]                    device, bf16
 *   k_cache [batch, kv_capacity, hkv, head_dim]      device, bf16 (positions < kv_len used)
 *   v_cache [batch, kv_capacity, hkv, head_dim]      device, bf16
 *   o       [batch, hq, head_dim]                    device, out_dtype
 *   lse     [batch, hq] float32 or NULL
 *   kv_capacity: cache length per sequence (0 means kv_len); >= kv_len.
 *   workspace: device, >= flux_decode_workspace_size(...) bytes, 256-byte aligned.
 * Supported: in_dtype BF16, out_dtype BF16 or F32, head_dim in {64, 128},
 * hq/hkv in {1, 2, 4, 8}, block == 64.
 */
int flux_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                     int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t kv_len,
                     int64_t kv_capacity, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                     int32_t mode, int32_t block, int32_t sink_tokens, int32_t window_tokens,
                     int32_t num_splits, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of the fixed device scratch flux_attn_decode_noalloc keeps its split partials in. */
#define FLUX_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * flux_attn_decode_noalloc -- flux_attn_decode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Same arguments, meaning and results as flux_attn_decode (same kernels), minus the workspace:
 * the split partials go to a fixed scratch array of FLUX_DECODE_SCRATCH_BYTES in device memory
 * that the library holds on each GPU it runs on until the process ends.  Nothing is allocated
 * and nothing is cleared per call (the partials are written before they are read).  A call whose
 * partials, flux_decode_workspace_size(...) bytes for the same arguments, exceed the scratch is
 * rejected with FLUX_ERR_CAPACITY before any launch (batch 8 x 32 query heads at head_dim 128 with
 * the automatic split count needs 4.03 MiB).  Every call on one GPU shares that GPU's scratch:
 * calls that may overlap on one GPU (several streams, several threads) race and must be
 * serialised by the caller; calls in order on one stream are safe.
 */
int flux_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                             int32_t in_dtype, int32_t out_dtype, int64_t batch, int64_t kv_len,
                             int64_t kv_capacity, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                             int32_t mode, int32_t block, int32_t sink_tokens, int32_t window_tokens,
                             int32_t num_splits, void* hip_stream);

/*
 * flux_window_cache_rows -- rows of a FLUX_KV_WINDOW cache: sink_tokens + window_tokens.
 * Returns 0 if block != 64 or sink/window are not valid multiples of block (window >= block).
 */
int64_t flux_window_cache_rows(int32_t block, int32_t sink_tokens, int32_t window_tokens);

/*
 * flux_decode_step -- append one token to a layer's KV cache and attend from it.
 *
 * The decode loop of a routed model ([FA] architecture paragraph: a sparse layer loads only its sink
 * and window KV; layer-granularity paragraph: one mode per layer).  For each sequence b the new token
 * sits at position pos (all sequences of the batch advance together): its key/value k_new, v_new
 * [batch, hkv, head_dim] bf16 are stored into the cache and the query q [batch, hq, head_dim] bf16
 * attends to tokens 0..pos under `mode` exactly as flux_attn_decode with kv_len = pos + 1 (a small
 * launch stores the new token before the attention launches, in stream order).
 *   layout FLUX_KV_FULL:   k_cache/v_cache [batch, cache_rows, hkv, head_dim], cache_rows > pos, any mode;
 *   layout FLUX_KV_WINDOW: cache_rows == flux_window_cache_rows(block, sink, window), mode SPARSE; the
 *     tokens the sparse pattern can still reach (sink and last window blocks) are all the cache keeps.
 * Earlier tokens must already be in the cache (written by earlier steps or by the caller).
 * workspace: flux_decode_workspace_size(batch, hq, hkv, pos + 1, head_dim, mode, block, sink, window,
 * num_splits) bytes.  out_dtype BF16 or F32; lse [batch, hq] fp32 or NULL.
 */
int flux_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, void* o, float* lse, int32_t out_dtype, int64_t batch, int64_t pos,
                     int64_t cache_rows, int32_t layout, int32_t hq, int32_t hkv, int32_t head_dim,
                     float scale, int32_t mode, int32_t block, int32_t sink_tokens,
                     int32_t window_tokens, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* hip_stream);

/*
 * flux_decode_step_layers -- one decode step over a routed layer stack.
 *
 * Layer l runs flux_decode_step with mode modes_host[l] (the prefill-time router decision, host
 * array): dense layers on FLUX_KV_FULL caches of dense_cache_rows rows, sparse layers on
 * FLUX_KV_WINDOW caches.  One workspace, sized for the largest layer (the dense one), is reused by
 * the layers in stream order.  All layers are validated before the first launch.
 */
int flux_decode_step_layers(int32_t n_layers, const int32_t* modes_host, const void* const* q,
                            const void* const* k_new, const void* const* v_new,
                            void* const* k_cache, void* const* v_cache, void* const* o,
                            float* const* lse, int32_t out_dtype, int64_t batch, int64_t pos,
                            int64_t dense_cache_rows, int32_t hq, int32_t hkv, int32_t head_dim,
                            float scale, int32_t block, int32_t sink_tokens, int32_t window_tokens,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * flux_route_workspace_size -- bytes of workspace flux_route_layers needs:
 * the pooled features [n_layers, hq*head_dim] and the encoder activations
 * [n_layers, hidden], float32, then one int32 arrival counter per layer (set by
 * the call itself: the workspace needs no clearing), each part 256-byte aligned.
 * 0 if invalid.  Calls that share a workspace must be ordered (one stream).
 */
size_t flux_route_workspace_size(int32_t n_layers, int32_t hq, int32_t head_dim, int32_t hidden);

/*
 * flux_route_layers -- the layer router ([FA] router paragraphs).
 *
 * For each layer l (xQ = q_layers[l], one sequence, [seq, hq, head_dim]):
 *   pooled = mean of xQ over token indices [0, P) U [seq-P, seq), each index
 *            counted once (P = pool_tokens, 100 in the method), flattened to
 *            hq*head_dim features;
 *   z      = ReLU(w_enc[l] pooled + b_enc[l])          (context encoder MLP)
 *   pi     = w_head[l] z + b_head[l]                    (router head: pi_FA, pi_SA)
 *   mode   = argmax(pi), a tie selecting FLUX_MODE_DENSE.
 * q_layers: HOST array of n_layers device pointers (in_dtype BF16 or F32).
 * w_enc [n_layers, hidden, hq*head_dim], b_enc [n_layers, hidden],
 * w_head [n_layers, 2, hidden], b_head [n_layers, 2]: device float32.
 * logits_out [n_layers, 2] device float32 (may be NULL); modes_out
 * [n_layers] device int32.  workspace: device, 256-byte aligned, at least
 * flux_route_workspace_size(...) bytes.  modes_out can feed
 * flux_attn_prefill_layers_routed directly (no host round trip), or be copied to
 * the host for flux_attn_prefill_layers / flux_decode_step_layers.
 * Supported: hq*head_dim a multiple of 8, pool_tokens >= 1.
 */
int flux_route_layers(const void* const* q_layers, int32_t n_layers, int64_t seq, int32_t hq,
                      int32_t head_dim, int32_t in_dtype, int32_t pool_tokens, const float* w_enc,
                      const float* b_enc, int32_t hidden, const float* w_head, const float* b_head,
                      float* logits_out, int32_t* modes_out, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUX_ATTN_H */
