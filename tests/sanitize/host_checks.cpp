// host_checks.cpp -- drives the library's host layer (block-mask builder, argument validation,
// workspace sizing, status reporting) and the fp64 oracle through their pointer-writing paths,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side (see
// tests/test_sanitized_host.py).  No GPU: every library call below is host-only or is rejected
// by validation before its first HIP call (the fake device pointers are never dereferenced).
// Exit status 0 when every check holds; any sanitizer report aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "flux_attn.h"

// the oracle's entry points (oracle/flux_oracle.c, test infrastructure)
extern "C" {
int64_t oracle_block_mask(int64_t seq_q, int64_t seq_k, int block, int sink_tokens, int window_tokens, int causal,
                          int sparse, uint8_t* bitmap);
int64_t oracle_count_pairs(int64_t seq_q, int64_t seq_k, int causal, int sparse, int block, int sink_tokens,
                           int window_tokens, int n_threads);
int oracle_attention_rows(const void* q, const void* k, const void* v, int kind, int64_t batch, int64_t seq_q,
                          int64_t seq_k, int hq, int hkv, int d, double scale, int causal, int sparse, int block,
                          int sink_tokens, int window_tokens, const int64_t* rows, int64_t n_rows, int n_threads,
                          double* out, double* lse);
int oracle_decode(const void* q, const void* k_cache, const void* v_cache, int kind, int64_t batch, int64_t kv_len,
                  int hq, int hkv, int d, double scale, int sparse, int block, int sink_tokens, int window_tokens,
                  const int64_t* rows, int64_t n_rows, int n_threads, double* out, double* lse);
int oracle_route(const void* const* xq_layers, int kind, int n_layers, int64_t seq, int hq, int d, int pool_tokens,
                 const float* w_enc, const float* b_enc, int hidden, const float* w_head, const float* b_head,
                 double* pooled_out, double* logits_out, int* modes_out);
int oracle_soft_weights(const double* logits, const double* uniforms, double tau, int n_layers, double* weights);
int oracle_attention_backward(const void* q, const void* k, const void* v, const void* d_o, int kind,
                              int64_t batch, int64_t seq, int hq, int hkv, int d, double scale, int causal,
                              int sparse, int block, int sink_tokens, int window_tokens, int n_threads, double* dq,
                              double* dk, double* dv);
int oracle_attention_backward_keys(const void* q, const void* k, const void* v, const void* d_o, int kind,
                                   int64_t batch, int64_t seq, int hq, int hkv, int d, double scale, int causal,
                                   int sparse, int block, int sink_tokens, int window_tokens, const int64_t* keys,
                                   int64_t n_keys, int n_threads, double* dk, double* dv);
}

static int g_fail = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++g_fail;                                                            \
        }                                                                        \
    } while (0)

// 256-byte aligned addresses that are never dereferenced (validation rejects every call first)
static void* fake(uintptr_t k) { return reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull) + 256 * k); }

static void mask_checks() {
    struct Case { int64_t s; int block, sink, window, causal, mode; };
    const Case cases[] = {{512, 64, 128, 128, 1, 1}, {1000, 64, 128, 256, 1, 1}, {97, 16, 0, 16, 1, 1},
                          {64, 64, 128, 64, 1, 1},   {777, 32, 64, 96, 1, 1},   {65536, 64, 128, 2048, 1, 1},
                          {300, 64, 0, 0, 1, 0},     {300, 64, 0, 0, 0, 0},     {1, 64, 0, 64, 1, 1}};
    for (const Case& c : cases) {
        int64_t nbq = (c.s + c.block - 1) / c.block;
        std::vector<int32_t> rp(nbq + 1, -7);
        int64_t nnz = -1;
        CHECK(flux_build_block_mask(c.s, c.s, c.block, c.sink, c.window, c.causal, c.mode, rp.data(), nullptr, 0,
                                    &nnz) == FLUX_OK);
        std::vector<int32_t> ci(nnz > 0 ? nnz : 1, -7);
        CHECK(flux_build_block_mask(c.s, c.s, c.block, c.sink, c.window, c.causal, c.mode, rp.data(), ci.data(), nnz,
                                    &nnz) == FLUX_OK);
        std::vector<uint8_t> bm(nbq * nbq);
        int64_t cnt = oracle_block_mask(c.s, c.s, c.block, c.sink, c.window, c.causal, c.mode, bm.data());
        CHECK(cnt == nnz);
        for (int64_t i = 0; i < nbq; ++i)
            for (int32_t p = rp[i]; p < rp[i + 1]; ++p) CHECK(bm[i * nbq + ci[p]] == 1);
        if (nnz > 1) {   // one entry short: FLUX_ERR_CAPACITY, nothing written past the capacity
            std::vector<int32_t> small(nnz, -7);
            CHECK(flux_build_block_mask(c.s, c.s, c.block, c.sink, c.window, c.causal, c.mode, rp.data(), small.data(),
                                        nnz - 1, &nnz) == FLUX_ERR_CAPACITY);
            CHECK(small[nnz - 1] == -7);
        }
    }
    int32_t rp[16];
    int64_t nnz;
    CHECK(flux_build_block_mask(0, 64, 64, 0, 64, 1, 1, rp, nullptr, 0, &nnz) == FLUX_ERR_INVALID_ARG);
    CHECK(flux_build_block_mask(640, 640, 64, 100, 128, 1, 1, rp, nullptr, 0, &nnz) == FLUX_ERR_INVALID_ARG);
    CHECK(flux_build_block_mask(640, 640, 64, 128, 128, 0, 1, rp, nullptr, 0, &nnz) == FLUX_ERR_INVALID_ARG);
    int32_t ci[64];
    CHECK(flux_build_block_mask(640, 640, 64, 128, 128, 1, 1, nullptr, ci, 64, &nnz) == FLUX_ERR_INVALID_ARG);
    CHECK(flux_build_block_mask(640, 640, 64, 128, 128, 1, 1, rp, nullptr, 5, &nnz) == FLUX_ERR_INVALID_ARG);
    CHECK(flux_build_block_mask(640, 640, 64, 128, 128, 1, 1, rp, ci, 64, nullptr) == FLUX_ERR_INVALID_ARG);
    CHECK(flux_build_block_mask(640, 640, 64, 128, 128, 1, 1, nullptr, nullptr, 0, &nnz) == FLUX_OK && nnz == 34);
}

static void validation_checks() {
    void *q = fake(1), *k = fake(2), *v = fake(3), *o = fake(4), *ws = fake(5);
    const int E = FLUX_ERR_INVALID_ARG, U = FLUX_ERR_UNSUPPORTED;
    // prefill
    CHECK(flux_attn_prefill(nullptr, k, v, o, nullptr, 0, 1, 1, 512, 8, 2, 128, 0.08f, 1, 0, 64, 128, 2048, nullptr,
                            nullptr, 0, nullptr) == E);
    CHECK(flux_attn_prefill(q, k, v, o, nullptr, 0, 1, 1, 512, 8, 3, 128, 0.08f, 1, 0, 64, 128, 2048, nullptr,
                            nullptr, 0, nullptr) == E);
    CHECK(flux_attn_prefill(q, k, v, o, nullptr, 0, 1, 1, 512, 8, 2, 96, 0.08f, 1, 0, 64, 128, 2048, nullptr, nullptr,
                            0, nullptr) == U);
    CHECK(flux_attn_prefill(q, k, v, o, nullptr, 0, 1, 1, 512, 8, 2, 128, -1.0f, 1, 0, 64, 128, 2048, nullptr,
                            nullptr, 0, nullptr) == E);
    CHECK(flux_attn_prefill(q, k, v, o, nullptr, 0, 1, 1, 512, 8, 2, 128, 0.08f, 1, 1, 64, 128, 2048,
                            (const int32_t*)ws, nullptr, 0, nullptr) == E);   // half a CSR
    CHECK(flux_attn_prefill(q, k, v, o, nullptr, 0, 1, 1, 512, 8, 2, 128, 0.08f, 1, 1, 64, 128, 2048,
                            (const int32_t*)ws, (const int32_t*)ws, 7, nullptr) == E);   // nnz not the pattern's
    // per-layer dispatch: a NULL pointer in layer 1 is found before anything launches
    const void* qs[2] = {q, nullptr};
    const void* ks[2] = {k, k};
    const void* vs[2] = {v, v};
    void* os[2] = {o, o};
    int32_t modes[2] = {0, 0};
    CHECK(flux_attn_prefill_layers(2, modes, qs, ks, vs, os, nullptr, 0, 1, 1, 512, 8, 2, 128, 0.08f, 64, 128, 2048,
                                   nullptr, nullptr, 0, nullptr) == E);
    CHECK(std::strstr(flux_last_error_detail(), "1") != nullptr);
    // decode, no-allocation decode, decode step layers
    CHECK(flux_attn_decode(q, k, v, o, nullptr, 0, 1, 2, 4096, 0, 8, 2, 128, 0.08f, 0, 64, 128, 2048, 0, nullptr, 0,
                           nullptr) == FLUX_ERR_WORKSPACE);
    CHECK(flux_attn_decode(q, k, v, o, nullptr, 0, 1, 2, 4096, 100, 8, 2, 128, 0.08f, 0, 64, 128, 2048, 0, ws,
                           1 << 30, nullptr) == E);
    CHECK(flux_attn_decode_noalloc(q, k, v, o, nullptr, 0, 1, 64, 4096, 0, 32, 8, 128, 0.08f, 0, 64, 128, 2048, 64,
                                   nullptr) == FLUX_ERR_CAPACITY);
    CHECK(flux_attn_decode_noalloc(q, k, v, o, nullptr, 0, 1, 2, 4096, 0, 32, 2, 128, 0.08f, 0, 64, 128, 2048, 0,
                                   nullptr) == U);
    const void* qd[3] = {q, q, q};
    const void* kn[3] = {k, k, nullptr};
    void* kc[3] = {k, k, k};
    void* od[3] = {o, o, o};
    int32_t dmodes[3] = {0, 1, 0};
    CHECK(flux_decode_step_layers(3, dmodes, qd, kn, kn, kc, kc, od, nullptr, 1, 2, 100, 4096, 8, 2, 128, 0.08f, 64,
                                  128, 2048, ws, 1 << 30, nullptr) == E);
    // backward
    CHECK(flux_attn_backward(q, k, v, o, q, (const float*)ws, (float*)o, (float*)k, nullptr, 0, 1, 1, 512, 8, 2, 128,
                             0.08f, 1, 0, 64, 0, 0, ws, 1 << 30, nullptr) == E);
    // soft routing
    CHECK(flux_route_soft_weights((const float*)q, (const float*)k, 0.0f, 4, (float*)o, nullptr) == E);
    CHECK(flux_attn_prefill_soft(q, k, v, o, 0, 1, 1, 512, 8, 2, 128, 0.08f, 64, 128, 2048, nullptr, nullptr, 0,
                                 (const float*)ws, nullptr, 0, nullptr) != FLUX_OK);
    // router: NULL layer pointer, tiny workspace
    const void* xs[2] = {q, nullptr};
    CHECK(flux_route_layers(xs, 2, 1000, 32, 128, 0, 100, (const float*)ws, (const float*)ws, 256, (const float*)ws,
                            (const float*)ws, nullptr, (int32_t*)o, ws, 1 << 30, nullptr) == E);
    CHECK(flux_route_layers(xs, 1, 1000, 32, 128, 0, 100, (const float*)ws, (const float*)ws, 256, (const float*)ws,
                            (const float*)ws, nullptr, (int32_t*)o, ws, 100, nullptr) == FLUX_ERR_WORKSPACE);
    // sizing
    CHECK(flux_decode_workspace_size(8, 32, 8, 262144, 128, 0, 64, 128, 2048, 0) > 0);
    CHECK(flux_decode_workspace_size(8, 32, 5, 262144, 128, 0, 64, 128, 2048, 0) == 0);
    CHECK(flux_attn_backward_workspace_size(1, 65536, 32, 8, 128, 1, 64, 128) > 0);
    CHECK(flux_route_workspace_size(36, 32, 128, 256) > 0);
    CHECK(flux_prefill_soft_workspace_size(1, 8192, 32, 128) == size_t(8192) * 32 * 128 * 4);
    CHECK(flux_window_cache_rows(64, 128, 2048) == 2176);
    CHECK(flux_window_cache_rows(64, 100, 2048) == 0);
    for (int s = 0; s < 8; ++s) CHECK(flux_status_string(s) != nullptr && std::strlen(flux_status_string(s)) > 0);
}

static uint16_t bf16_bits(float x) {   // round to nearest even
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static void oracle_checks() {
    const int B = 2, S = 70, Hq = 4, Hkv = 2, d = 8;
    std::vector<uint16_t> q(B * S * Hq * d), k(B * S * Hkv * d), v(B * S * Hkv * d), g(B * S * Hq * d);
    uint32_t st = 12345;
    auto rnd = [&]() { st = st * 1664525u + 1013904223u; return ((st >> 8) & 0xffff) / 32768.0f - 1.0f; };
    for (auto& x : q) x = bf16_bits(rnd());
    for (auto& x : k) x = bf16_bits(rnd());
    for (auto& x : v) x = bf16_bits(rnd());
    for (auto& x : g) x = bf16_bits(rnd());
    const int kind = 1;
    std::vector<double> out(B * S * Hq * d), lse(B * S * Hq);
    for (int sparse = 0; sparse < 2; ++sparse) {
        CHECK(oracle_attention_rows(q.data(), k.data(), v.data(), kind, B, S, S, Hq, Hkv, d, 0.3, 1, sparse, 8, 16, 16,
                                    nullptr, 0, 2, out.data(), lse.data()) == 0);
        for (double x : out) CHECK(std::isfinite(x));
    }
    int64_t rows[6] = {0, 1, 5, 1, 3, 69};
    CHECK(oracle_attention_rows(q.data(), k.data(), v.data(), kind, B, S, S, Hq, Hkv, d, 0.3, 1, 1, 8, 16, 16, rows, 2,
                                1, out.data(), lse.data()) == 0);
    int64_t bad_rows[3] = {0, 9, 5};
    CHECK(oracle_attention_rows(q.data(), k.data(), v.data(), kind, B, S, S, Hq, Hkv, d, 0.3, 1, 1, 8, 16, 16, bad_rows,
                                1, 1, out.data(), lse.data()) != 0);
    std::vector<double> dout(B * Hq * d), dlse(B * Hq);
    CHECK(oracle_decode(q.data(), k.data(), v.data(), kind, B, S, Hq, Hkv, d, 0.3, 1, 8, 16, 16, nullptr, 0, 2,
                        dout.data(), dlse.data()) == 0);
    std::vector<double> dq(B * S * Hq * d), dk(B * S * Hkv * d), dv(B * S * Hkv * d);
    CHECK(oracle_attention_backward(q.data(), k.data(), v.data(), g.data(), kind, B, S, Hq, Hkv, d, 0.3, 1, 1, 8, 16,
                                    16, 2, dq.data(), dk.data(), dv.data()) == 0);
    int64_t keys[9] = {0, 0, 0, 1, 1, 69, 1, 0, 33};
    std::vector<double> kk(3 * d), kv(3 * d);
    CHECK(oracle_attention_backward_keys(q.data(), k.data(), v.data(), g.data(), kind, B, S, Hq, Hkv, d, 0.3, 1, 1, 8,
                                         16, 16, keys, 3, 2, kk.data(), kv.data()) == 0);
    for (int t = 0; t < 3; ++t)
        for (int c = 0; c < d; ++c) {
            const int64_t idx = ((keys[3 * t] * S + keys[3 * t + 2]) * Hkv + keys[3 * t + 1]) * d + c;
            CHECK(std::fabs(kk[t * d + c] - dk[idx]) <= 1e-12 + 1e-10 * std::fabs(dk[idx]));
            CHECK(std::fabs(kv[t * d + c] - dv[idx]) <= 1e-12 + 1e-10 * std::fabs(dv[idx]));
        }
    CHECK(oracle_count_pairs(S, S, 1, 1, 8, 16, 16, 1) > 0);
    // router on two layers of xq [S, Hq, d]
    const int hidden = 5, nf = Hq * d;
    std::vector<float> we(2 * hidden * nf), be(2 * hidden), wh(2 * 2 * hidden), bh(4);
    for (auto& x : we) x = rnd();
    for (auto& x : be) x = rnd();
    for (auto& x : wh) x = rnd();
    for (auto& x : bh) x = rnd();
    const void* xs[2] = {q.data(), q.data() + S * Hq * d};
    std::vector<double> pooled(2 * nf), logits(4);
    int m[2] = {-1, -1};
    CHECK(oracle_route(xs, kind, 2, S, Hq, d, 100, we.data(), be.data(), hidden, wh.data(), bh.data(), pooled.data(),
                       logits.data(), m) == 0);
    CHECK((m[0] == 0 || m[0] == 1) && (m[1] == 0 || m[1] == 1));
    double u[4] = {0.2, 0.7, 0.5, 0.5}, w[4];
    CHECK(oracle_soft_weights(logits.data(), u, 0.5, 2, w) == 0);
    CHECK(std::fabs(w[0] + w[1] - 1.0) < 1e-12);
}

int main() {
    mask_checks();
    validation_checks();
    oracle_checks();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
