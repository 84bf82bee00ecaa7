"""Pins of the oracle's soft routing (Gumbel-softmax relaxation of the router, Flux Attention page,
router paragraph): weights r = softmax((pi + g)/tau) with g = -ln(-ln u), and the soft-routed layer
output r_FA * O_full + r_SA * O_sparse.  Each check is computed independently of the oracle: closed
forms of the two-way softmax (a logistic), limits, and a brute-force attention with scipy."""
import math

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
import synth


def _logistic(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_zero_noise_gives_plain_softmax_of_logits():
    # u = 1/e  ->  g = -ln(-ln(1/e)) = -ln 1 = 0
    u = math.exp(-1.0)
    for pi0, pi1, tau in [(1.0, 0.0, 1.0), (0.3, 0.9, 0.5), (-2.0, 5.0, 3.0)]:
        w = oracle.soft_weights([[pi0, pi1]], [[u, u]], tau)
        assert w[0, 0] == pytest.approx(_logistic((pi0 - pi1) / tau), rel=1e-14)
        assert w[0, 1] == pytest.approx(_logistic((pi1 - pi0) / tau), rel=1e-14)


def test_gumbel_transform_of_the_uniforms():
    # u = exp(-exp(-g)) has Gumbel value exactly g
    g0, g1, pi0, pi1, tau = 2.0, -1.0, 0.5, 0.3, 0.7
    u = [[math.exp(-math.exp(-g0)), math.exp(-math.exp(-g1))]]
    w = oracle.soft_weights([[pi0, pi1]], u, tau)
    assert w[0, 0] == pytest.approx(_logistic(((pi0 + g0) - (pi1 + g1)) / tau), rel=1e-12)


def test_weights_are_a_distribution_and_shift_invariant():
    rng = np.random.default_rng(3)
    logits = rng.normal(size=(16, 2)) * 3
    u = rng.uniform(0.01, 0.99, size=(16, 2))
    w = oracle.soft_weights(logits, u, 0.8)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    assert (w > 0).all()
    w2 = oracle.soft_weights(logits + 123.0, u, 0.8)
    assert np.allclose(w, w2, atol=1e-12)


def test_small_temperature_approaches_hard_routing():
    rng = np.random.default_rng(4)
    logits = rng.normal(size=(32, 2))
    u = rng.uniform(0.05, 0.95, size=(32, 2))
    w = oracle.soft_weights(logits, u, 1e-6)
    perturbed = logits - np.log(-np.log(u))
    hard = np.argmax(perturbed, axis=1)
    assert np.array_equal(np.argmax(w, axis=1), hard)
    assert np.allclose(w.max(axis=1), 1.0, atol=1e-9)


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.soft_weights([[0.0, 1.0]], [[0.0, 0.5]], 1.0)
    with pytest.raises(ValueError):
        oracle.soft_weights([[0.0, 1.0]], [[0.5, 0.5]], 0.0)


def _brute(q, k, v, scale, allowed):
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kk = k[b, :, h // G].astype(np.float64)
            vv = v[b, :, h // G].astype(np.float64)
            sc = scale * (q[b, :, h].astype(np.float64) @ kk.T)
            out[b, :, h] = scipy_softmax(np.where(allowed, sc, -np.inf), axis=-1) @ vv
    return out


@pytest.mark.parametrize("w0", [1.0, 0.0, 0.3])
def test_soft_output_is_the_weighted_sum_of_full_and_sparse(w0):
    B, S, Hq, Hkv, d, block, sink, window = 1, 160, 2, 1, 16, 16, 32, 32
    q, k, v = synth.qkv_f32(B, S, Hq, Hkv, d, seed=9)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    causal = j <= i
    sparse = causal & ((j // block < sink // block) | (i // block - j // block < window // block))
    scale = 1.0 / math.sqrt(d)
    want = w0 * _brute(q, k, v, scale, causal) + (1 - w0) * _brute(q, k, v, scale, sparse)
    got = oracle.attention_soft(q, k, v, scale, (w0, 1.0 - w0), block=block, sink_tokens=sink, window_tokens=window)
    assert np.abs(got - want).max() < 1e-12
