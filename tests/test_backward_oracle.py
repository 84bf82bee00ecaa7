"""Pins of the oracle's backward pass (gradients of the attention output).  Checked against
central finite differences of an independent brute-force forward (scipy softmax over a materialised
score matrix), against the GQA/MHA equivalence, and against closed-form special cases."""
import math

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
import synth


def _allowed(S, causal, sparse, block, sink, window):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    a = np.ones((S, S), bool)
    if causal or sparse:
        a &= j <= i
    if sparse:
        a &= (j // block < sink // block) | (i // block - j // block < window // block)
    return a


def _forward(q, k, v, scale, allowed):
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for h in range(Hq):
            sc = scale * (q[b, :, h] @ k[b, :, h // G].T)
            out[b, :, h] = scipy_softmax(np.where(allowed, sc, -np.inf), axis=-1) @ v[b, :, h // G]
    return out


CASES = [
    # S, Hq, Hkv, d, causal, sparse, block, sink, window
    (24, 2, 1, 8, True, False, 4, 0, 0),
    (20, 2, 2, 8, False, False, 4, 0, 0),
    (32, 4, 2, 4, True, True, 4, 4, 8),
]


@pytest.mark.parametrize("S,Hq,Hkv,d,causal,sparse,block,sink,window", CASES)
def test_backward_matches_finite_differences(S, Hq, Hkv, d, causal, sparse, block, sink, window):
    rng = np.random.default_rng(S + Hq)
    q = rng.normal(size=(1, S, Hq, d))
    k = rng.normal(size=(1, S, Hkv, d))
    v = rng.normal(size=(1, S, Hkv, d))
    d_o = rng.normal(size=(1, S, Hq, d))
    scale = 1.0 / math.sqrt(d)
    allowed = _allowed(S, causal, sparse, block, sink, window)
    f32 = lambda x: np.ascontiguousarray(x, np.float32).astype(np.float64)
    q, k, v, d_o = (f32(x) for x in (q, k, v, d_o))   # values exactly representable in float32
    dq, dk, dv = oracle.attention_backward(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                                           d_o.astype(np.float32), scale, causal=causal, sparse=sparse, block=block,
                                           sink_tokens=sink, window_tokens=window)
    loss = lambda qq, kk, vv: float(np.sum(d_o * _forward(qq, kk, vv, scale, allowed)))
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert grad[idx] == pytest.approx(fd, rel=1e-5, abs=1e-7), (name, idx)


def test_gqa_gradients_equal_summed_mha():
    B, S, Hq, Hkv, d = 1, 40, 4, 2, 8
    q, k, v = synth.qkv_f32(B, S, Hq, Hkv, d, seed=81)
    d_o = synth.normal_f32((B, S, Hq, d), 81, 0, 5)
    scale = 0.3
    dq, dk, dv = oracle.attention_backward(q, k, v, d_o, scale)
    kr = np.ascontiguousarray(np.repeat(k, Hq // Hkv, axis=2))
    vr = np.ascontiguousarray(np.repeat(v, Hq // Hkv, axis=2))
    dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, d_o, scale)
    assert np.allclose(dq, dq2, atol=1e-12)
    assert np.allclose(dk, dk2.reshape(B, S, Hkv, Hq // Hkv, d).sum(axis=3), atol=1e-12)
    assert np.allclose(dv, dv2.reshape(B, S, Hkv, Hq // Hkv, d).sum(axis=3), atol=1e-12)


def test_constant_values_give_zero_query_and_key_gradients():
    B, S, Hq, Hkv, d = 1, 30, 2, 1, 8
    q, k, _ = synth.qkv_f32(B, S, Hq, Hkv, d, seed=82)
    v = np.ascontiguousarray(np.broadcast_to(np.linspace(-1, 1, d, dtype=np.float32), (B, S, Hkv, d)))
    d_o = synth.normal_f32((B, S, Hq, d), 82, 0, 5)
    dq, dk, dv = oracle.attention_backward(q, k, v, d_o, 0.35)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.abs(dv).max() > 0.1


def test_zero_output_gradient_gives_zero_gradients():
    q, k, v = synth.qkv_f32(1, 20, 2, 2, 8, seed=83)
    z = np.zeros_like(q)
    dq, dk, dv = oracle.attention_backward(q, k, v, z, 0.35)
    assert not dq.any() and not dk.any() and not dv.any()


def test_sparse_full_window_equals_dense_causal():
    q, k, v = synth.qkv_f32(1, 48, 2, 1, 8, seed=84)
    d_o = synth.normal_f32((1, 48, 2, 8), 84, 0, 5)
    a = oracle.attention_backward(q, k, v, d_o, 0.35, causal=True)
    b = oracle.attention_backward(q, k, v, d_o, 0.35, causal=True, sparse=True, block=8, sink_tokens=8,
                                  window_tokens=48)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


KEY_CASES = [
    # B, S, Hq, Hkv, d, causal, sparse, block, sink, window
    (1, 40, 2, 1, 8, True, False, 8, 0, 0),
    (2, 37, 4, 2, 8, False, False, 8, 0, 0),
    (2, 70, 6, 2, 4, True, True, 8, 16, 16),   # ragged, sink 2 blocks, window 2 blocks, odd group
    (1, 64, 8, 1, 8, True, True, 8, 0, 8),      # no sink, diagonal blocks only
]


@pytest.mark.parametrize("B,S,Hq,Hkv,d,causal,sparse,block,sink,window", KEY_CASES)
def test_backward_keys_equals_full_backward(B, S, Hq, Hkv, d, causal, sparse, block, sink, window):
    """dK/dV of a key subset equal the full backward's rows for those keys (every key, then a random
    subset in shuffled order, so a key written to another's slot fails)."""
    q, k, v = synth.qkv_bf16(B, S, Hq, Hkv, d, seed=S + Hq)
    g = synth.normal_bf16_bits((B, S, Hq, d), seed=S + Hq, tensor_id=7)
    scale = 1.0 / math.sqrt(d)
    kw = dict(causal=causal, sparse=sparse, block=block, sink_tokens=sink, window_tokens=window)
    _, dk, dv = oracle.attention_backward(q, k, v, g, scale, **kw)
    all_keys = np.array([(b, h, j) for b in range(B) for h in range(Hkv) for j in range(S)], np.int64)
    rng = np.random.default_rng(S)
    for keys in (all_keys, rng.permutation(all_keys)[: max(3, len(all_keys) // 5)]):
        gk, gv = oracle.attention_backward_keys(q, k, v, g, scale, keys, **kw)
        want_k = np.stack([dk[b, j, h] for b, h, j in keys])
        want_v = np.stack([dv[b, j, h] for b, h, j in keys])
        np.testing.assert_allclose(gk, want_k, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gv, want_v, rtol=1e-11, atol=1e-12)


def test_backward_keys_rejects_bad_keys():
    q, k, v = synth.qkv_bf16(1, 16, 2, 1, 4, seed=3)
    g = synth.normal_bf16_bits((1, 16, 2, 4), seed=3, tensor_id=7)
    for bad in ((0, 1, 0), (1, 0, 0), (0, 0, 16), (0, 0, -1)):
        with pytest.raises(ValueError):
            oracle.attention_backward_keys(q, k, v, g, 0.5, np.array([bad]))
