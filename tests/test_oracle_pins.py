"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a closed form,
a worked example printed on the pages (tests/golden/), an invariant, a special
case that reduces to a library routine, or brute force on tiny inputs.  Chosen so
that a dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
import synth


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _scores_as_attention(scores, shift=0.0):
    """One query, n keys, d = n: q = e_0, k_j = (s_j + shift) e_0, v_j = e_j, scale 1.

    Then O[j] is exactly softmax(s)_j."""
    s = np.asarray(scores, np.float64) + shift
    n = len(s)
    q = np.zeros((1, 1, 1, n), np.float32); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n, 1, n), np.float32); k[0, :, 0, 0] = s.astype(np.float32)
    v = np.zeros((1, n, 1, n), np.float32)
    for j in range(n):
        v[0, j, 0, j] = 1.0
    out, lse = oracle.attention(q, k, v, 1.0, causal=False)
    return out[0, 0, 0], lse[0, 0, 0]


def test_softmax_closed_form_page_example(golden_dir):
    g = _load(golden_dir, "softmax_example.json")
    s = g["scores"]
    p, lse = _scores_as_attention(s)
    e = [math.exp(x) for x in s]
    closed = [x / sum(e) for x in e]
    np.testing.assert_allclose(p, closed, rtol=1e-15, atol=0)
    assert abs(p.sum() - 1.0) < 1e-15
    assert abs(lse - math.log(sum(e))) < 1e-15
    # the page's simple normalisation x / sum(x) is right to its two printed digits
    simple = np.asarray(s) / np.sum(s)
    np.testing.assert_allclose(simple, g["page_simple_normalisation"], atol=0.005)
    # the page's printed softmax is off; it still lies within 0.025 of the closed form
    np.testing.assert_allclose(p, g["page_softmax_as_printed"], atol=0.025)
    assert np.max(np.abs(p - np.asarray(g["page_softmax_as_printed"]))) > 0.01  # and really differs


@pytest.mark.parametrize("shift", [1000.0, -1000.0, 1.0e4, -1.0e4])
def test_shift_invariance(shift):
    s = [2.0, 1.0, 0.5, -3.0]
    p0, lse0 = _scores_as_attention(s)
    p1, lse1 = _scores_as_attention(s, shift)
    # without the max subtraction exp(1e4) overflows double and the result is NaN
    assert np.all(np.isfinite(p1))
    np.testing.assert_allclose(p1, p0, rtol=1e-12, atol=1e-15)
    assert abs((lse1 - shift) - lse0) < 1e-9


def test_fp16_overflow_threshold(golden_dir):
    g = _load(golden_dir, "fp16_overflow.json")
    thr = math.log(float(np.finfo(np.float16).max))
    assert abs(thr - g["page_threshold"]) < 0.1
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float16(thr + 0.01)))
        assert np.isfinite(np.exp(np.float16(thr - 0.01)))
    # the oracle's max subtraction keeps every exponent <= 0: scores far above the
    # fp16 limit still give the closed-form softmax
    p, _ = _scores_as_attention([40.0, 39.0, 12.0])
    e = np.exp(np.array([0.0, -1.0, -28.0]))
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-14)


def _online_softmax_weights(scores, block):
    """Blockwise online softmax (running max m, running sum l, rescale by exp(m_old - m_new))."""
    m, l = -np.inf, 0.0
    weights = []           # (block start, unnormalised weights relative to current m)
    for b0 in range(0, len(scores), block):
        x = np.asarray(scores[b0:b0 + block], np.float64)
        m_new = max(m, x.max())
        alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
        weights = [(s0, w * alpha) for (s0, w) in weights]
        p = np.exp(x - m_new)
        l = l * alpha + p.sum()
        weights.append((b0, p))
        m = m_new
    return np.concatenate([w for _, w in weights]) / l, m, l


def test_online_softmax_page_example_equals_oracle(golden_dir):
    g = _load(golden_dir, "online_softmax_example.json")
    s = g["scores"]
    blk = g["block"]
    assert max(s[:blk]) == g["block1_max"] and max(s[blk:]) == g["block2_max"]
    # the oracle reads the scores through float32 keys; feed the online version the same values
    s32 = np.asarray(s, np.float32).astype(np.float64)
    p_online, m, l = _online_softmax_weights(s32, blk)
    assert m == np.float32(g["block2_max"])
    p_oracle, lse = _scores_as_attention(s)
    np.testing.assert_allclose(p_online, p_oracle, rtol=1e-14, atol=0)
    assert abs((m + math.log(l)) - lse) < 1e-14


def _online_attention(q, k, v, scale, allowed, block):
    """Independent blockwise online-softmax attention (fp64, numpy) for one row set."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                for j0 in range(0, S, block):
                    js = np.arange(j0, min(S, j0 + block))
                    js = js[allowed[i, js]]
                    if len(js) == 0:
                        continue
                    sc = scale * (k[b, js, g] @ q[b, i, h])
                    m_new = max(m, sc.max())
                    alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
                    p = np.exp(sc - m_new)
                    l = l * alpha + p.sum()
                    acc = acc * alpha + p @ v[b, js, g]
                    m = m_new
                out[b, i, h] = acc / l
    return out


def _allowed_matrix(S, causal=True, sparse=False, block=64, sink=0, window=0):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    a = np.ones((S, S), bool)
    if causal or sparse:
        a &= j <= i
    if sparse:
        ib, jb = i // block, j // block
        a &= (jb < sink // block) | (ib - jb < window // block)
    return a


def _brute_force(q, k, v, scale, allowed):
    """Materialise the masked score matrix and use scipy's softmax (P5-style plain attention)."""
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kk = k[b, :, h // G].astype(np.float64)
            vv = v[b, :, h // G].astype(np.float64)
            sc = scale * (q[b, :, h].astype(np.float64) @ kk.T)
            sc = np.where(allowed, sc, -np.inf)
            out[b, :, h] = scipy_softmax(sc, axis=-1) @ vv
    return out


CASES = [
    # B, S, Hq, Hkv, d, causal, sparse, block, sink, window
    (1, 96, 2, 2, 16, True, False, 16, 0, 0),
    (2, 77, 4, 2, 8, False, False, 16, 0, 0),
    (1, 200, 4, 1, 16, True, True, 16, 32, 32),
    (1, 130, 2, 2, 8, True, True, 16, 16, 16),
    (1, 512, 2, 2, 64, True, True, 64, 128, 128),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,d,causal,sparse,block,sink,window", CASES)
def test_oracle_equals_brute_force(B, S, Hq, Hkv, d, causal, sparse, block, sink, window):
    q, k, v = synth.qkv_f32(B, S, Hq, Hkv, d, seed=7)
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.attention(q, k, v, scale, causal=causal, sparse=sparse, block=block, sink_tokens=sink,
                                window_tokens=window)
    ref = _brute_force(q, k, v, scale, _allowed_matrix(S, causal, sparse, block, sink, window))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,S,Hq,Hkv,d,causal,sparse,block,sink,window", CASES[:4])
def test_online_blockwise_equals_two_pass(B, S, Hq, Hkv, d, causal, sparse, block, sink, window):
    q, k, v = synth.qkv_f32(B, S, Hq, Hkv, d, seed=11)
    scale = 1.0 / math.sqrt(d)
    out, _ = oracle.attention(q, k, v, scale, causal=causal, sparse=sparse, block=block, sink_tokens=sink,
                              window_tokens=window)
    allowed = _allowed_matrix(S, causal, sparse, block, sink, window)
    for tile in (4, 16, 37):
        on = _online_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale,
                               allowed, tile)
        np.testing.assert_allclose(out, on, rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = synth.qkv_f32(1, 90, 8, 2, 16, seed=3)
    kr = np.repeat(k, 4, axis=2)
    vr = np.repeat(v, 4, axis=2)
    for sparse in (False, True):
        a, la = oracle.attention(q, k, v, 0.25, sparse=sparse, block=16, sink_tokens=16, window_tokens=32)
        b, lb = oracle.attention(q, kr, vr, 0.25, sparse=sparse, block=16, sink_tokens=16, window_tokens=32)
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(la, lb)


def test_sparse_with_full_window_equals_dense_causal():
    S = 300
    q, k, v = synth.qkv_f32(1, S, 2, 1, 16, seed=5)
    dense, _ = oracle.attention(q, k, v, 0.25, causal=True)
    sp, _ = oracle.attention(q, k, v, 0.25, sparse=True, block=64, sink_tokens=128, window_tokens=64 * 5)
    np.testing.assert_array_equal(dense, sp)
    bm_sp = oracle.block_mask(S, S, 64, 128, 64 * 5, causal=True, sparse=True)
    bm_d = oracle.block_mask(S, S, 64, 0, 0, causal=True, sparse=False)
    np.testing.assert_array_equal(bm_sp, bm_d)


def test_bf16_bits_input_matches_float32_input():
    qb, kb, vb = synth.qkv_bf16(1, 70, 2, 1, 16, seed=9)
    qf, kf, vf = (synth.bf16_bits_to_f32(x) for x in (qb, kb, vb))
    a, _ = oracle.attention(qb, kb, vb, 0.25)
    b, _ = oracle.attention(qf, kf, vf, 0.25)
    np.testing.assert_array_equal(a, b)


def test_constant_values_give_constant_output():
    q, k, v = synth.qkv_f32(1, 150, 2, 2, 8, seed=1)
    v[:] = np.float32(1.75)
    for sparse in (False, True):
        out, _ = oracle.attention(q, k, v, 0.3, sparse=sparse, block=16, sink_tokens=16, window_tokens=32)
        np.testing.assert_allclose(out, 1.75, rtol=1e-14, atol=0)  # a few ulps of summation


def test_zero_keys_give_mean_of_allowed_values():
    S, block, sink, window = 160, 16, 32, 48
    q, k, v = synth.qkv_f32(1, S, 2, 2, 8, seed=2)
    k[:] = 0
    vv = v[0].astype(np.float64)
    dense, _ = oracle.attention(q, k, v, 0.5, causal=True)
    prefix_mean = np.cumsum(vv, axis=0) / np.arange(1, S + 1)[:, None, None]
    np.testing.assert_allclose(dense[0], prefix_mean, rtol=0, atol=1e-13)
    sp, _ = oracle.attention(q, k, v, 0.5, sparse=True, block=block, sink_tokens=sink, window_tokens=window)
    for i in range(S):
        ib = i // block
        keys = [j for j in range(i + 1) if j // block < sink // block or ib - j // block < window // block]
        np.testing.assert_allclose(sp[0, i], vv[keys].mean(axis=0), rtol=0, atol=1e-13)


@pytest.mark.parametrize("L", [333, 320])
@pytest.mark.parametrize("sparse", [False, True])
def test_decode_equals_last_prefill_row(sparse, L):
    """L = 320 is a block multiple: there a decode from position L instead of L-1 would see another
    window (blocks 8..10 instead of 7..9) and fail."""
    Hq, Hkv, d = 4, 2, 16
    q, k, v = synth.qkv_f32(2, L, Hq, Hkv, d, seed=4)
    kw = dict(sparse=sparse, block=32, sink_tokens=64, window_tokens=96)
    pre, plse = oracle.attention(q, k, v, 0.25, causal=True, **kw)
    dec, dlse = oracle.decode(np.ascontiguousarray(q[:, -1]), k, v, 0.25, **kw)
    np.testing.assert_array_equal(dec, pre[:, -1])
    np.testing.assert_array_equal(dlse, plse[:, -1])


@pytest.mark.parametrize("L", [256, 2304])
def test_decode_sparse_is_sink_plus_last_window_tokens(L):
    """With the cache length a multiple of the block, the sparse decode row attends to exactly the sink
    tokens and the last `window` tokens (the decode workload's own wording: sink 128 plus the last 2048
    tokens); checked against scipy's softmax over that explicit token set."""
    from scipy.special import softmax as scipy_softmax
    block, sink, window = (32, 64, 96) if L == 256 else (64, 128, 2048)
    Hq, Hkv, d = 2, 1, 16
    q, k, v = synth.qkv_f32(1, L, Hq, Hkv, d, seed=L)
    qd = np.ascontiguousarray(q[:, -1])
    dec, dlse = oracle.decode(qd, k, v, 0.25, sparse=True, block=block, sink_tokens=sink, window_tokens=window)
    keys = np.r_[0:sink, L - window:L]
    k64, v64 = k[0, keys, 0].astype(np.float64), v[0, keys, 0].astype(np.float64)
    for h in range(Hq):
        s = 0.25 * (k64 @ qd[0, h].astype(np.float64))
        np.testing.assert_allclose(dec[0, h], scipy_softmax(s) @ v64, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dlse[0, h], np.log(np.sum(np.exp(s))), rtol=1e-14)


def test_rows_subset_matches_full():
    q, k, v = synth.qkv_f32(2, 65, 4, 2, 8, seed=6)
    full, flse = oracle.attention(q, k, v, 0.3, sparse=True, block=16, sink_tokens=16, window_tokens=16)
    rows = np.array([[0, 0, 0], [1, 3, 64], [1, 2, 17], [0, 1, 33]])
    sub, slse = oracle.attention(q, k, v, 0.3, sparse=True, block=16, sink_tokens=16, window_tokens=16,
                                 rows=rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(sub[r], full[b, i, h])
        assert slse[r] == flse[b, i, h]
