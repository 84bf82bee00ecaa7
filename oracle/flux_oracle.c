/*
 * flux_oracle.c -- plain fp64 CPU reference of the tiled-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the GPU
 * path.
 *
 * Every quantity is computed from its definition, in double precision, with
 * no tiling, no online rescaling and no fusion:
 *
 *   - attention:  O = softmax(scale * Q K^T + mask) V, evaluated row by row
 *     with an explicit two-pass, max-subtracted softmax.  Sources: the
 *     attention definition in the "Softmax is not a simple function" section of
 *     the openads.co.kr FlashAttention newsletter and the self_attention listing
 *     in the "why self-attention is expensive" section of "After self-attention:
 *     what comes after transformers" (datadaily.news); the max subtraction and
 *     its shift invariance from the newsletter's "hidden cost of numerical
 *     stability" section.
 *   - the block-sparse key set: 64-token blocks, an always-kept 128-token sink
 *     and a causal local window of blocks, from the implementation paragraph of
 *     "Flux Attention: context-aware hybrid attention for efficient LLM
 *     inference" (aitrends.kr) and the sliding-window bullet of the hybrid
 *     architectures section of the datadaily.news page.
 *   - the layer router: prefix/suffix mean pooling of xQ over the first and
 *     last P tokens, an MLP context encoder, a two-logit router head and an
 *     argmax (ties to index 0 = full attention), from the router paragraphs of
 *     the Flux Attention page.
 *   - the backward pass (gradients of the attention output with respect to Q,
 *     K and V for a given output gradient dO), from the chain rule through the
 *     same definition: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
 *     dQ = scale dS K, dK = scale dS^T Q -- the softmax Jacobian
 *     diag(p) - p p^T applied row by row.  Needed to train the router over a
 *     frozen backbone (Flux Attention page, router and architecture paragraphs).
 *   - soft routing (the training-time relaxation in the same router paragraph):
 *     r = softmax((pi + g) / tau) over (pi_FA, pi_SA) with Gumbel noise
 *     g = -ln(-ln u) drawn from uniforms u in (0, 1), and the layer output
 *     r_FA * O_FA + r_SA * O_SA (full and sparse attention outputs).
 *
 * Inputs are read either as float32 or as bfloat16 bit patterns; both widen
 * to double exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_KIND_F32 0
#define ORACLE_KIND_BF16 1

/* Exact widening of one stored element to double. */
static double load_elem(const void* base, int kind, int64_t idx) {
    if (kind == ORACLE_KIND_F32) return (double)((const float*)base)[idx];
    uint32_t u = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * May query position i attend to key position j?
 *   dense, causal:     j <= i
 *   dense, non-causal: every j
 *   sparse (always causal): j <= i and (key block is a sink block, or the key
 *   block lies within the last `window` blocks ending at the query's block).
 * window_tokens == 0 in dense mode means "no window".
 *
 * The block tests are restated as two key thresholds that depend on i only:
 * j/block < sink_blocks  <=>  j < sink_blocks * block, and
 * i/block - j/block < window_blocks  <=>  j >= (i/block - window_blocks + 1) * block
 * (floor division, j >= 0), so a scan over the keys of one row does no division.
 */
typedef struct {
    int64_t last;           /* last key position the row may see: i when causal or sparse, else seq_k - 1 */
    int64_t sink_end;       /* sparse: keys before this are sink keys */
    int64_t window_start;   /* sparse: keys from here on lie in the row's window */
    int sparse;
} key_rule;

static key_rule row_rule(int64_t i, int64_t seq_k, int causal, int sparse, int64_t block, int64_t sink_tokens,
                         int64_t window_tokens) {
    key_rule r;
    r.last = (causal || sparse) && i < seq_k - 1 ? i : seq_k - 1;
    r.sparse = sparse;
    r.sink_end = sparse ? (sink_tokens / block) * block : 0;
    r.window_start = sparse ? (i / block - window_tokens / block + 1) * block : 0;
    return r;
}

static int rule_allows(const key_rule* r, int64_t j) {
    if (j < 0 || j > r->last) return 0;
    if (r->sparse && !(j < r->sink_end || j >= r->window_start)) return 0;
    return 1;
}

static int key_allowed(int64_t i, int64_t j, int64_t seq_k, int causal, int sparse,
                       int64_t block, int64_t sink_tokens, int64_t window_tokens) {
    const key_rule r = row_rule(i, seq_k, causal, sparse, block, sink_tokens, window_tokens);
    return rule_allows(&r, j);
}

/*
 * One output row: query vector q (d values at q_base+q_off), keys/values of KV
 * head g, query position i.  Two passes over the allowed keys:
 *   pass 1: s_j = scale * <q, k_j>,  m = max_j s_j
 *   pass 2: p_j = exp(s_j - m),  l = sum p_j,  o = sum p_j v_j / l,  lse = m + ln l
 */
static void attend_row(const void* q, int64_t q_off, const void* k, const void* v, int kind,
                       int64_t kv_base, int64_t kv_row_stride, int64_t seq_k, int d, double scale,
                       int64_t i, int causal, int sparse, int64_t block, int64_t sink, int64_t window,
                       double* s_buf, double* acc, double* out, double* lse) {
    const key_rule rule = row_rule(i, seq_k, causal, sparse, block, sink, window);
    double m = -INFINITY;
    int64_t n_allowed = 0;
    for (int64_t j = 0; j < seq_k; ++j) {
        if (!rule_allows(&rule, j)) continue;
        double s = 0.0;
        for (int t = 0; t < d; ++t)
            s += load_elem(q, kind, q_off + t) * load_elem(k, kind, kv_base + j * kv_row_stride + t);
        s *= scale;
        s_buf[j] = s;
        if (s > m) m = s;
        ++n_allowed;
    }
    for (int t = 0; t < d; ++t) acc[t] = 0.0;
    if (n_allowed == 0) {
        for (int t = 0; t < d; ++t) out[t] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < seq_k; ++j) {
        if (!rule_allows(&rule, j)) continue;
        double p = exp(s_buf[j] - m);
        l += p;
        for (int t = 0; t < d; ++t) acc[t] += p * load_elem(v, kind, kv_base + j * kv_row_stride + t);
    }
    for (int t = 0; t < d; ++t) out[t] = acc[t] / l;
    *lse = m + log(l);
}

static int check_shapes(int64_t batch, int64_t seq_k, int hq, int hkv, int d) {
    if (batch <= 0 || seq_k <= 0 || hq <= 0 || hkv <= 0 || d <= 0) return 1;
    if (hq % hkv != 0) return 1;
    return 0;
}

/*
 * Prefill rows.  q [B, seq_q, Hq, d], k/v [B, seq_k, Hkv, d] (row-major).
 * Query head h reads KV head h / (Hq/Hkv).  Query index i is also its position.
 * rows: n_rows triples (b, h, i); rows == NULL means every row in (b, i, h)
 * order, so `out` then has the layout [B, seq_q, Hq, d].
 * out: [n_rows, d] doubles; lse: [n_rows] doubles (natural log).
 */
int oracle_attention_rows(const void* q, const void* k, const void* v, int kind,
                          int64_t batch, int64_t seq_q, int64_t seq_k, int hq, int hkv, int d,
                          double scale, int causal, int sparse, int block, int sink_tokens,
                          int window_tokens, const int64_t* rows, int64_t n_rows, int n_threads,
                          double* out, double* lse) {
    if (check_shapes(batch, seq_k, hq, hkv, d) || seq_q <= 0) return 1;
    if (sparse && block <= 0) return 1;
    int64_t total = rows ? n_rows : batch * seq_q * hq;
    int group = hq / hkv;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    int err = 0;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * (size_t)seq_k);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s_buf || !acc) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < total; ++r) {
                int64_t b, h, i;
                if (rows) {
                    b = rows[3 * r];
                    h = rows[3 * r + 1];
                    i = rows[3 * r + 2];
                } else {
                    b = r / (seq_q * hq);
                    i = (r / hq) % seq_q;
                    h = r % hq;
                }
                if (b < 0 || b >= batch || h < 0 || h >= hq || i < 0 || i >= seq_q) {
#pragma omp atomic write
                    err = 1;
                    continue;
                }
                int64_t g = h / group;
                int64_t q_off = ((b * seq_q + i) * hq + h) * (int64_t)d;
                int64_t kv_base = (b * seq_k * hkv + g) * (int64_t)d;
                attend_row(q, q_off, k, v, kind, kv_base, (int64_t)hkv * d, seq_k, d, scale, i, causal,
                           sparse, block, sink_tokens, window_tokens, s_buf, acc, out + r * d, lse + r);
            }
        }
        free(s_buf);
        free(acc);
    }
    return err;
}

/*
 * Decode: one new query per sequence at position kv_len-1, whose own K/V is
 * already in the cache.  q [B, Hq, d], k_cache/v_cache [B, kv_len, Hkv, d].
 * The allowed keys are those of prefill row kv_len-1 (causal; sparse adds the
 * sink/window rule).  rows: n_rows pairs (b, h); NULL means all in (b, h)
 * order, out [B, Hq, d].
 */
int oracle_decode(const void* q, const void* k_cache, const void* v_cache, int kind,
                  int64_t batch, int64_t kv_len, int hq, int hkv, int d, double scale,
                  int sparse, int block, int sink_tokens, int window_tokens,
                  const int64_t* rows, int64_t n_rows, int n_threads, double* out, double* lse) {
    if (check_shapes(batch, kv_len, hq, hkv, d)) return 1;
    if (sparse && block <= 0) return 1;
    int64_t total = rows ? n_rows : batch * hq;
    int group = hq / hkv;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    int err = 0;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * (size_t)kv_len);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s_buf || !acc) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < total; ++r) {
                int64_t b = rows ? rows[2 * r] : r / hq;
                int64_t h = rows ? rows[2 * r + 1] : r % hq;
                if (b < 0 || b >= batch || h < 0 || h >= hq) {
#pragma omp atomic write
                    err = 1;
                    continue;
                }
                int64_t g = h / group;
                int64_t q_off = (b * hq + h) * (int64_t)d;
                int64_t kv_base = (b * kv_len * hkv + g) * (int64_t)d;
                attend_row(q, q_off, k_cache, v_cache, kind, kv_base, (int64_t)hkv * d, kv_len, d, scale,
                           kv_len - 1, 1, sparse, block, sink_tokens, window_tokens, s_buf, acc,
                           out + r * d, lse + r);
            }
        }
        free(s_buf);
        free(acc);
    }
    return err;
}

/*
 * Block mask as a dense bitmap [nbq, nbk] (row = query block I, column = key
 * block J).  A block pair is active when
 *   dense:  (J <= I when causal) -- every causal block, or every block;
 *   sparse: J <= I and (J < sink_blocks or I - J < window_blocks).
 * Returns the number of active pairs (or -1 on bad arguments).  bitmap may be
 * NULL to count only.
 */
int64_t oracle_block_mask(int64_t seq_q, int64_t seq_k, int block, int sink_tokens, int window_tokens,
                          int causal, int sparse, uint8_t* bitmap) {
    if (seq_q <= 0 || seq_k <= 0 || block <= 0) return -1;
    int64_t nbq = (seq_q + block - 1) / block, nbk = (seq_k + block - 1) / block;
    int64_t sink_blocks = sink_tokens / block, window_blocks = window_tokens / block;
    int64_t count = 0;
    for (int64_t I = 0; I < nbq; ++I) {
        for (int64_t J = 0; J < nbk; ++J) {
            int on;
            if (sparse)
                on = (J <= I) && (J < sink_blocks || I - J < window_blocks);
            else
                on = causal ? (J <= I) : 1;
            if (bitmap) bitmap[I * nbk + J] = (uint8_t)on;
            count += on;
        }
    }
    return count;
}

/*
 * Number of (query, key) pairs the token-level rule allows, by enumeration.
 * Useful FLOPs of one head = 4 * d * pairs (2 per multiply-add in QK^T and in PV).
 */
int64_t oracle_count_pairs(int64_t seq_q, int64_t seq_k, int causal, int sparse, int block,
                           int sink_tokens, int window_tokens, int n_threads) {
    if (seq_q <= 0 || seq_k <= 0 || (sparse && block <= 0)) return -1;
    int64_t count = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
#pragma omp parallel for reduction(+ : count) schedule(dynamic, 64)
    for (int64_t i = 0; i < seq_q; ++i)
        for (int64_t j = 0; j < seq_k; ++j)
            count += key_allowed(i, j, seq_k, causal, sparse, block, sink_tokens, window_tokens);
    return count;
}

/*
 * Layer router.  For layer l, xq_layers[l] points at xQ [seq, hq, d] (one
 * sequence).  Steps:
 *   pooled[f] = mean over token indices t in [0, P) U [seq-P, seq) (each index
 *               once; P = pool_tokens) of xQ[t, f], f over the flattened hq*d
 *   z[u]      = max(0, sum_f w_enc[l,u,f] * pooled[f] + b_enc[l,u])
 *   pi[c]     = sum_u w_head[l,c,u] * z[u] + b_head[l,c]      (c=0: full, c=1: sparse)
 *   mode      = 1 if pi[1] > pi[0] else 0                      (a tie selects full attention)
 * Weights: w_enc [L, hidden, hq*d], b_enc [L, hidden], w_head [L, 2, hidden], b_head [L, 2].
 * pooled_out [L, hq*d] may be NULL; logits_out [L, 2]; modes_out [L].
 */
int oracle_route(const void* const* xq_layers, int kind, int n_layers, int64_t seq, int hq, int d,
                 int pool_tokens, const float* w_enc, const float* b_enc, int hidden,
                 const float* w_head, const float* b_head, double* pooled_out, double* logits_out,
                 int* modes_out) {
    if (n_layers <= 0 || seq <= 0 || hq <= 0 || d <= 0 || pool_tokens <= 0 || hidden <= 0) return 1;
    int64_t nf = (int64_t)hq * d;
    double* pooled = (double*)malloc(sizeof(double) * (size_t)nf);
    double* z = (double*)malloc(sizeof(double) * (size_t)hidden);
    if (!pooled || !z) {
        free(pooled);
        free(z);
        return 2;
    }
    for (int l = 0; l < n_layers; ++l) {
        const void* xq = xq_layers[l];
        int64_t n_tok = 0;
        for (int64_t f = 0; f < nf; ++f) pooled[f] = 0.0;
        for (int64_t t = 0; t < seq; ++t) {
            if (!(t < pool_tokens || t >= seq - pool_tokens)) continue;
            ++n_tok;
            for (int64_t f = 0; f < nf; ++f) pooled[f] += load_elem(xq, kind, t * nf + f);
        }
        for (int64_t f = 0; f < nf; ++f) pooled[f] /= (double)n_tok;
        if (pooled_out)
            for (int64_t f = 0; f < nf; ++f) pooled_out[(int64_t)l * nf + f] = pooled[f];
        for (int u = 0; u < hidden; ++u) {
            const float* w = w_enc + ((int64_t)l * hidden + u) * nf;
            double a = (double)b_enc[(int64_t)l * hidden + u];
            for (int64_t f = 0; f < nf; ++f) a += (double)w[f] * pooled[f];
            z[u] = a > 0.0 ? a : 0.0;
        }
        double pi[2];
        for (int c = 0; c < 2; ++c) {
            const float* w = w_head + ((int64_t)l * 2 + c) * hidden;
            double a = (double)b_head[(int64_t)l * 2 + c];
            for (int u = 0; u < hidden; ++u) a += (double)w[u] * z[u];
            pi[c] = a;
        }
        logits_out[2 * l] = pi[0];
        logits_out[2 * l + 1] = pi[1];
        modes_out[l] = pi[1] > pi[0] ? 1 : 0;
    }
    free(pooled);
    free(z);
    return 0;
}

/*
 * Soft-routing weights per layer (Flux Attention page, router paragraph: the
 * Gumbel-Softmax relaxation used in training).  logits [L, 2] = (pi_FA, pi_SA),
 * uniforms [L, 2] in (0, 1) -> Gumbel noise g = -ln(-ln u); weights [L, 2] =
 * exp((pi_i + g_i) / tau) / sum_j exp((pi_j + g_j) / tau), computed with the
 * larger exponent subtracted.  Returns 1 on a bad argument.
 */
int oracle_soft_weights(const double* logits, const double* uniforms, double tau, int n_layers,
                        double* weights) {
    if (n_layers <= 0 || !(tau > 0.0)) return 1;
    for (int l = 0; l < n_layers; ++l) {
        double x[2];
        for (int c = 0; c < 2; ++c) {
            double u = uniforms[2 * l + c];
            if (!(u > 0.0 && u < 1.0)) return 1;
            x[c] = (logits[2 * l + c] - log(-log(u))) / tau;
        }
        double m = x[0] > x[1] ? x[0] : x[1];
        double e0 = exp(x[0] - m), e1 = exp(x[1] - m);
        weights[2 * l] = e0 / (e0 + e1);
        weights[2 * l + 1] = e1 / (e0 + e1);
    }
    return 0;
}

/* out[i] = w0 * o_full[i] + w1 * o_sparse[i]: the soft-routed layer output (same page). */
void oracle_mix(const double* o_full, const double* o_sparse, double w0, double w1, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = w0 * o_full[i] + w1 * o_sparse[i];
}

/*
 * Backward pass.  q, d_o [B, S, Hq, d]; k, v [B, S, Hkv, d] (same element kind);
 * outputs dq [B, S, Hq, d], dk, dv [B, S, Hkv, d] in double.  For each (b, h, i):
 * the row's probabilities p_j (two-pass softmax over the allowed keys, as in
 * attend_row), dp_j = <dO_i, v_j>, D = sum_j p_j dp_j, ds_j = p_j (dp_j - D);
 * dq_i = scale sum_j ds_j k_j, dk_j += scale ds_j q_i, dv_j += p_j dO_i.  The
 * query heads sharing a KV head accumulate into its dk/dv.  Parallel over
 * (batch, kv head), so no two threads write the same dk/dv row.
 */
int oracle_attention_backward(const void* q, const void* k, const void* v, const void* d_o, int kind,
                              int64_t batch, int64_t seq, int hq, int hkv, int d, double scale, int causal,
                              int sparse, int block, int sink_tokens, int window_tokens, int n_threads,
                              double* dq, double* dk, double* dv) {
    if (check_shapes(batch, seq, hq, hkv, d)) return 1;
    if (sparse && (!causal || block <= 0)) return 1;
    const int G = hq / hkv;
    const int64_t q_stride = (int64_t)hq * d, kv_stride = (int64_t)hkv * d;
    memset(dk, 0, sizeof(double) * (size_t)(batch * seq * kv_stride));
    memset(dv, 0, sizeof(double) * (size_t)(batch * seq * kv_stride));
    const int64_t units = batch * hkv;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)seq);
        double* dp = (double*)malloc(sizeof(double) * (size_t)seq);
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
        for (int64_t u = 0; u < units; ++u) {
            const int64_t b = u / hkv;
            const int g = (int)(u % hkv);
            const int64_t kv_base = b * seq * kv_stride + (int64_t)g * d;
            for (int hh = 0; hh < G; ++hh) {
                const int h = g * G + hh;
                for (int64_t i = 0; i < seq; ++i) {
                    const int64_t q_off = (b * seq + i) * q_stride + (int64_t)h * d;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < seq; ++j) {
                        if (!key_allowed(i, j, seq, causal, sparse, block, sink_tokens, window_tokens)) continue;
                        double s = 0.0;
                        for (int t = 0; t < d; ++t)
                            s += load_elem(q, kind, q_off + t) * load_elem(k, kind, kv_base + j * kv_stride + t);
                        p[j] = s * scale;
                        if (p[j] > m) m = p[j];
                    }
                    double l = 0.0;
                    for (int64_t j = 0; j < seq; ++j) {
                        if (!key_allowed(i, j, seq, causal, sparse, block, sink_tokens, window_tokens)) continue;
                        p[j] = exp(p[j] - m);
                        l += p[j];
                    }
                    double D = 0.0;
                    for (int64_t j = 0; j < seq; ++j) {
                        if (!key_allowed(i, j, seq, causal, sparse, block, sink_tokens, window_tokens)) continue;
                        p[j] /= l;
                        double a = 0.0;
                        for (int t = 0; t < d; ++t)
                            a += load_elem(d_o, kind, q_off + t) * load_elem(v, kind, kv_base + j * kv_stride + t);
                        dp[j] = a;
                        D += p[j] * a;
                    }
                    double* dq_row = dq + q_off;
                    for (int t = 0; t < d; ++t) dq_row[t] = 0.0;
                    for (int64_t j = 0; j < seq; ++j) {
                        if (!key_allowed(i, j, seq, causal, sparse, block, sink_tokens, window_tokens)) continue;
                        const double ds = p[j] * (dp[j] - D);
                        const int64_t kv_off = kv_base + j * kv_stride;
                        for (int t = 0; t < d; ++t) {
                            dq_row[t] += scale * ds * load_elem(k, kind, kv_off + t);
                            dk[kv_off + t] += scale * ds * load_elem(q, kind, q_off + t);
                            dv[kv_off + t] += p[j] * load_elem(d_o, kind, q_off + t);
                        }
                    }
                }
            }
        }
        free(p);
        free(dp);
    }
    return 0;
}

/*
 * dK and dV of selected keys only (same definition as oracle_attention_backward, restricted to
 * the requested key rows), for checking gradients at sizes where the full backward is too slow.
 * keys: n_keys triples (b, g, j) = (batch, KV head, key position); dk, dv: [n_keys, d] doubles.
 * For a requested key j of KV head g:
 *   dv_j = sum over query heads h of the group and rows i that may attend to j of p_ij dO_i
 *   dk_j = sum over the same (h, i) of scale * p_ij (dp_ij - D_i) q_i
 * with p_ij the row's softmax probability, dp_ij = <dO_i, v_j> and D_i = sum_j' p_ij' dp_ij' over
 * the row's allowed keys.  Step 1 marks the rows that see a requested key; step 2 computes those
 * rows' statistics (max m, sum l, D) with the two-pass softmax; step 3 sums each requested key's
 * gradient over its rows.  Returns 0, 1 on bad arguments, 2 if out of memory.
 */
int oracle_attention_backward_keys(const void* q, const void* k, const void* v, const void* d_o, int kind,
                                   int64_t batch, int64_t seq, int hq, int hkv, int d, double scale, int causal,
                                   int sparse, int block, int sink_tokens, int window_tokens,
                                   const int64_t* keys, int64_t n_keys, int n_threads, double* dk, double* dv) {
    if (check_shapes(batch, seq, hq, hkv, d)) return 1;
    if (sparse && (!causal || block <= 0)) return 1;
    for (int64_t r = 0; r < n_keys; ++r)
        if (keys[3 * r] < 0 || keys[3 * r] >= batch || keys[3 * r + 1] < 0 || keys[3 * r + 1] >= hkv ||
            keys[3 * r + 2] < 0 || keys[3 * r + 2] >= seq)
            return 1;
    const int G = hq / hkv;
    const int64_t q_stride = (int64_t)hq * d, kv_stride = (int64_t)hkv * d;
    const int64_t n_rows = batch * hq * seq;   /* row index (b * hq + h) * seq + i */
    unsigned char* need = (unsigned char*)calloc((size_t)n_rows, 1);
    double* m_row = (double*)malloc(sizeof(double) * (size_t)n_rows);
    double* l_row = (double*)malloc(sizeof(double) * (size_t)n_rows);
    double* D_row = (double*)malloc(sizeof(double) * (size_t)n_rows);
    if (!need || !m_row || !l_row || !D_row) {
        free(need);
        free(m_row);
        free(l_row);
        free(D_row);
        return 2;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    /* step 1: rows that may attend to at least one requested key of their KV head */
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t b = r / ((int64_t)hq * seq), h = (r / seq) % hq, i = r % seq;
        for (int64_t t = 0; t < n_keys; ++t)
            if (keys[3 * t] == b && keys[3 * t + 1] == h / G &&
                key_allowed(i, keys[3 * t + 2], seq, causal, sparse, block, sink_tokens, window_tokens)) {
                need[r] = 1;
                break;
            }
    }
    /* step 2: statistics of those rows: m = max_j s_j, l = sum_j exp(s_j - m), D = sum_j p_j dp_j, over
     * the row's allowed keys (listed once, in ascending order, by the first pass) */
    int err = 0;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * (size_t)seq);
        int64_t* allowed = (int64_t*)malloc(sizeof(int64_t) * (size_t)seq);
        if (!s_buf || !allowed) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < n_rows; ++r) {
                if (!need[r]) continue;
                const int64_t b = r / ((int64_t)hq * seq), h = (r / seq) % hq, i = r % seq;
                const int64_t q_off = (b * seq + i) * q_stride + h * d;
                const int64_t kv_base = b * seq * kv_stride + (h / G) * d;
                const key_rule rule = row_rule(i, seq, causal, sparse, block, sink_tokens, window_tokens);
                int64_t n_allowed = 0;
                double m = -INFINITY;
                for (int64_t j = 0; j < seq; ++j) {
                    if (!rule_allows(&rule, j)) continue;
                    double s = 0.0;
                    for (int t = 0; t < d; ++t)
                        s += load_elem(q, kind, q_off + t) * load_elem(k, kind, kv_base + j * kv_stride + t);
                    s_buf[n_allowed] = s * scale;
                    allowed[n_allowed++] = j;
                    if (s * scale > m) m = s * scale;
                }
                double l = 0.0;
                for (int64_t a = 0; a < n_allowed; ++a) l += exp(s_buf[a] - m);
                double D = 0.0;
                for (int64_t a = 0; a < n_allowed; ++a) {
                    const int64_t j = allowed[a];
                    double dp = 0.0;
                    for (int t = 0; t < d; ++t)
                        dp += load_elem(d_o, kind, q_off + t) * load_elem(v, kind, kv_base + j * kv_stride + t);
                    D += exp(s_buf[a] - m) / l * dp;
                }
                m_row[r] = m;
                l_row[r] = l;
                D_row[r] = D;
            }
        }
        free(s_buf);
        free(allowed);
    }
    /* step 3: each requested key's dk, dv over the rows that see it */
    if (!err) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_keys; ++t) {
            const int64_t b = keys[3 * t], g = keys[3 * t + 1], j = keys[3 * t + 2];
            const int64_t kv_off = b * seq * kv_stride + j * kv_stride + g * d;
            double* dk_t = dk + t * d;
            double* dv_t = dv + t * d;
            for (int c = 0; c < d; ++c) dk_t[c] = dv_t[c] = 0.0;
            for (int hh = 0; hh < G; ++hh) {
                const int64_t h = g * G + hh;
                for (int64_t i = 0; i < seq; ++i) {
                    if (!key_allowed(i, j, seq, causal, sparse, block, sink_tokens, window_tokens)) continue;
                    const int64_t r = (b * hq + h) * seq + i;
                    const int64_t q_off = (b * seq + i) * q_stride + h * d;
                    double s = 0.0, dp = 0.0;
                    for (int c = 0; c < d; ++c) {
                        s += load_elem(q, kind, q_off + c) * load_elem(k, kind, kv_off + c);
                        dp += load_elem(d_o, kind, q_off + c) * load_elem(v, kind, kv_off + c);
                    }
                    const double p = exp(s * scale - m_row[r]) / l_row[r];
                    const double ds = p * (dp - D_row[r]);
                    for (int c = 0; c < d; ++c) {
                        dv_t[c] += p * load_elem(d_o, kind, q_off + c);
                        dk_t[c] += scale * ds * load_elem(q, kind, q_off + c);
                    }
                }
            }
        }
    }
    free(need);
    free(m_row);
    free(l_row);
    free(D_row);
    return err;
}
