"""Pins of the oracle's block mask, pair counts and layer router."""
import json
import os

import numpy as np
import pytest

import oracle
import synth


def _token_level_block_bitmap(S, block, sink, window):
    """A block pair is active iff some (query, key) pair inside it is allowed (token-level brute force)."""
    nb = -(-S // block)
    bm = np.zeros((nb, nb), np.uint8)
    for i in range(S):
        for j in range(i + 1):
            ib, jb = i // block, j // block
            if jb < sink // block or ib - jb < window // block:
                bm[ib, jb] = 1
    return bm


@pytest.mark.parametrize("S,block,sink,window", [(512, 64, 128, 128), (300, 32, 64, 96), (97, 16, 0, 16),
                                                  (640, 64, 128, 2048)])
def test_block_mask_equals_token_level_enumeration(S, block, sink, window):
    bm = oracle.block_mask(S, S, block, sink, window, causal=True, sparse=True)
    np.testing.assert_array_equal(bm, _token_level_block_bitmap(S, block, sink, window))


def test_block_mask_c1_rows():
    # 512 tokens, 64-token blocks, sink 128 (2 blocks), window 2 blocks
    bm = oracle.block_mask(512, 512, 64, 128, 128)
    assert list(bm.sum(1)) == [1, 2, 3, 4, 4, 4, 4, 4]
    assert bm.sum() == 26


@pytest.mark.parametrize("nb", [33, 64, 1024, 2048])
def test_block_mask_closed_form_count(nb):
    # sink 2 blocks, window 32 blocks: rows 0..31 keep every causal block (528 in total),
    # row 32 keeps 33 (block 0 + window 1..32), every later row keeps 34 (sink 2 + window 32).
    bm = oracle.block_mask(64 * nb, 64 * nb, 64, 128, 2048)
    assert bm.sum() == 528 + 33 + 34 * (nb - 33)


def test_dense_causal_mask_is_lower_triangle():
    bm = oracle.block_mask(1000, 1000, 64, 0, 0, causal=True, sparse=False)
    nb = bm.shape[0]
    np.testing.assert_array_equal(bm, np.tril(np.ones((nb, nb), np.uint8)))
    assert oracle.block_mask(1000, 1000, 64, 0, 0, causal=False, sparse=False).all()


def test_reachability_across_block_edges():
    """With a window of >= 2 blocks every token sees its left neighbour; with a 1-block window
    (no sink), a token at the start of a block cannot see the token just before it -- the
    block-edge disconnection described in 'The reachability gap: why locality fails in sparse
    attention' (tech.ajinhub.com)."""
    S, block = 512, 64
    for window_blocks in (2, 3, 8):
        bm = oracle.block_mask(S, S, block, 0, window_blocks * block)
        for i in range(1, S):
            assert bm[i // block, (i - 1) // block] == 1
    bm1 = oracle.block_mask(S, S, block, 0, block)
    cut = [i for i in range(1, S) if bm1[i // block, (i - 1) // block] == 0]
    assert cut == list(range(block, S, block))


def test_pair_counts_page_figures(golden_dir):
    with open(os.path.join(golden_dir, "pair_counts.json")) as f:
        g = json.load(f)
    for e in g["approximate_entries"]:
        n = e["seq_len"]
        if n <= 32768:
            c = oracle.count_pairs(n, n, causal=False)
            assert c == n * n
        else:
            c = n * n  # enumerating 1.7e10 pairs is too slow for the CPU suite; N*N checked above
        assert abs(c - e["page_value"]) <= 0.1 * e["page_value"], e
    for e in g["lower_bounds"]:
        assert e["seq_len"] ** 2 >= e["page_value"]


@pytest.mark.parametrize("S", [1, 63, 64, 1000])
def test_causal_pair_count(S):
    assert oracle.count_pairs(S, S, causal=True) == S * (S + 1) // 2


@pytest.mark.parametrize("S,block,sink,window", [(512, 64, 128, 128), (4096, 64, 128, 2048), (1000, 64, 128, 256)])
def test_sparse_pair_count_from_bitmap(S, block, sink, window):
    """Count by enumeration == count from active blocks (full off-diagonal blocks, triangular diagonal)."""
    bm = oracle.block_mask(S, S, block, sink, window)
    total = 0
    for I, J in zip(*np.nonzero(bm)):
        qn = min(S, (I + 1) * block) - I * block
        kn = min(S, (J + 1) * block) - J * block
        total += qn * (qn + 1) // 2 if I == J else qn * kn
    assert oracle.count_pairs(S, S, sparse=True, block=block, sink_tokens=sink, window_tokens=window) == total


# ------------------------------------------------------------------ router
def _one_hot_router(nf, hidden=4):
    w_enc = np.zeros((1, hidden, nf), np.float32)
    b_enc = np.zeros((1, hidden), np.float32)
    w_head = np.zeros((1, 2, hidden), np.float32)
    b_head = np.zeros((1, 2), np.float32)
    return w_enc, b_enc, w_head, b_head


def test_router_constant_input_pools_to_constant(golden_dir):
    with open(os.path.join(golden_dir, "flux_constants.json")) as f:
        P = json.load(f)["pool_tokens_each_end"]
    x = np.full((1000, 2, 8), 0.625, np.float32)
    w = synth.router_weights(1, 16, 8, seed=1)
    pooled, _, _ = oracle.route([x], *w, pool_tokens=P)
    np.testing.assert_allclose(pooled, 0.625, rtol=1e-15)


def test_router_pools_first_and_last_tokens():
    S, P = 1000, 100
    x = synth.normal_f32((S, 2, 8), seed=3)
    w = synth.router_weights(1, 16, 8, seed=1)
    pooled, _, _ = oracle.route([x], *w, pool_tokens=P)
    ref = np.concatenate([x[:P], x[S - P:]]).astype(np.float64).reshape(2 * P, -1).mean(0)
    np.testing.assert_allclose(pooled[0], ref, rtol=1e-13, atol=1e-15)
    # the middle of the prompt does not influence the pooled feature
    x2 = x.copy(); x2[P:S - P] = 123.0
    p2, _, _ = oracle.route([x2], *w, pool_tokens=P)
    np.testing.assert_array_equal(p2, pooled)


@pytest.mark.parametrize("S", [1, 50, 100, 150, 199, 200])
def test_router_short_prompt_counts_each_token_once(S):
    x = synth.normal_f32((S, 1, 4), seed=S)
    w = synth.router_weights(1, 4, 8, seed=2)
    pooled, _, _ = oracle.route([x], *w, pool_tokens=100)
    np.testing.assert_allclose(pooled[0], x.astype(np.float64).reshape(S, -1).mean(0), rtol=1e-13, atol=1e-15)


def test_router_hand_set_weights_known_logits():
    # pooled feature = mean of the constant rows = (1, 2, 3, 4)
    x = np.tile(np.array([1, 2, 3, 4], np.float32).reshape(1, 1, 4), (10, 1, 1))
    w_enc, b_enc, w_head, b_head = _one_hot_router(4, hidden=3)
    w_enc[0, 0] = [1, 0, 0, 0]      # z0 = relu(1 - 0.5) = 0.5
    b_enc[0, 0] = -0.5
    w_enc[0, 1] = [0, 1, 1, 0]      # z1 = relu(5 - 6) = 0 (ReLU clips)
    b_enc[0, 1] = -6.0
    w_enc[0, 2] = [0, 0, 0, 2]      # z2 = relu(8) = 8
    w_head[0, 0] = [2, 100, 0]      # pi_FA = 1 + 0 + 0.25 = 1.25
    b_head[0, 0] = 0.25
    w_head[0, 1] = [0, 0, 0.5]      # pi_SA = 4 - 1 = 3
    b_head[0, 1] = -1.0
    _, logits, modes = oracle.route([x], w_enc, b_enc, w_head, b_head)
    np.testing.assert_allclose(logits[0], [1.25, 3.0], rtol=1e-15)
    assert modes[0] == 1
    b_head[0, 1] = -2.75            # pi_SA = 1.25: a tie selects full attention
    _, logits, modes = oracle.route([x], w_enc, b_enc, w_head, b_head)
    assert logits[0, 0] == logits[0, 1] and modes[0] == 0
    b_head[0, 1] = -2.5             # pi_SA = 1.5 > 1.25
    _, _, modes = oracle.route([x], w_enc, b_enc, w_head, b_head)
    assert modes[0] == 1


def test_router_layers_are_independent():
    xs = [synth.normal_f32((300, 2, 8), seed=s) for s in range(3)]
    w = synth.router_weights(3, 16, 8, seed=5)
    _, logits, modes = oracle.route(xs, *w)
    for l in range(3):
        _, lg, md = oracle.route([xs[l]], *(a[l:l + 1] for a in w))
        np.testing.assert_array_equal(lg[0], logits[l])
        assert md[0] == modes[l]
