"""GPU parity of split-KV decode (+ LSE combine) and of the layer router, vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import bf16_tensors, check_close, check_lse, default_scale, dev_bits_to_host, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def fa():
    import long_context_attention_tiled_amd as fa
    assert torch.cuda.is_available()
    return fa


def _decode(fa, qd, kd, vd, out_dtype, mode, kv_len=None, sink=128, window=2048, num_splits=0):
    B, Hq, d = qd.shape
    cap, Hkv = kd.shape[1], kd.shape[2]
    kv_len = cap if kv_len is None else kv_len
    ws_bytes = fa.flux_decode_workspace_size(B, Hq, Hkv, kv_len, d, mode, 64, sink, window, num_splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    o = torch.full((B, Hq, d), float("nan"), dtype=out_dtype, device=DEV)      # unwritten elements fail
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    fa.flux_attn_decode(qd, kd, vd, o, lse, kv_len=kv_len, mode=mode, block=64, sink_tokens=sink,
                        window_tokens=window, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # B, L, Hq, Hkv, d, mode, sink, window, num_splits
    (1, 1, 4, 1, 128, 0, 128, 2048, 0),
    (2, 100, 8, 2, 128, 0, 128, 2048, 0),
    (3, 4097, 32, 8, 128, 0, 128, 2048, 0),
    (2, 5000, 8, 1, 128, 0, 128, 2048, 7),
    (2, 3000, 4, 4, 64, 0, 128, 2048, 2),
    (2, 3000, 16, 2, 64, 0, 128, 2048, 0),
    (2, 8192, 32, 8, 128, 1, 128, 2048, 0),
    (1, 10000, 8, 2, 128, 1, 128, 1024, 3),     # ragged L, sparse
    (2, 200, 8, 2, 128, 1, 128, 128, 0),         # window overlaps the sink
    (1, 90, 4, 1, 128, 1, 128, 2048, 0),         # L shorter than the sink
    (2, 6000, 8, 1, 64, 1, 0, 64, 0),            # no sink, one-block window, 8 query heads per KV head
    (1, 7777, 2, 2, 128, 1, 192, 320, 5),        # MHA, sink of 3 blocks, ragged L, forced splits
    (4, 65, 16, 8, 64, 1, 64, 64, 0),            # one key past the first block
]


@pytest.mark.parametrize("B,L,Hq,Hkv,d,mode,sink,window,ns", SMALL)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_small_full_oracle(fa, B, L, Hq, Hkv, d, mode, sink, window, ns, out_dtype):
    say("decode small", B, L, Hq, Hkv, d, "mode", mode, sink, window, ns, out_dtype)
    q = synth.normal_bf16_bits((B, Hq, d), 3000 + L, 0, synth.TENSOR_Q)
    k = synth.normal_bf16_bits((B, L, Hkv, d), 3000 + L, 0, synth.TENSOR_K)
    v = synth.normal_bf16_bits((B, L, Hkv, d), 3000 + L, 0, synth.TENSOR_V)
    qd, kd, vd = (synth.torch_bf16_from_bits(x) for x in (q, k, v))
    o, lse = _decode(fa, qd, kd, vd, out_dtype, mode, sink=sink, window=window, num_splits=ns)
    ref, ref_lse = oracle.decode(q, k, v, default_scale(d), sparse=bool(mode), block=64, sink_tokens=sink,
                                 window_tokens=window)
    check_close(o.float().cpu().numpy(), ref, "decode small", out_bf16=out_dtype == torch.bfloat16)
    check_lse(lse.cpu().numpy(), ref_lse, "decode lse")


def test_decode_uses_kv_len_inside_capacity(fa):
    """Cache capacity larger than kv_len: positions >= kv_len are never read."""
    B, cap, L, Hq, Hkv, d = 2, 3000, 2500, 8, 2, 128
    say("decode capacity")
    k = synth.normal_bf16_bits((B, cap, Hkv, d), 41, 0, 1)
    v = synth.normal_bf16_bits((B, cap, Hkv, d), 41, 0, 2)
    q = synth.normal_bf16_bits((B, Hq, d), 41, 0, 0)
    kd, vd, qd = (synth.torch_bf16_from_bits(x) for x in (k, v, q))
    kd[:, L:] = float("nan")
    vd[:, L:] = float("nan")
    for mode in (0, 1):
        o, lse = _decode(fa, qd, kd, vd, torch.float32, mode, kv_len=L)
        ref, ref_lse = oracle.decode(q, np.ascontiguousarray(k[:, :L]), np.ascontiguousarray(v[:, :L]),
                                     default_scale(d), sparse=bool(mode), block=64, sink_tokens=128,
                                     window_tokens=2048)
        check_close(o.cpu().numpy(), ref, f"decode cap mode {mode}")


def test_decode_split_count_invariance(fa):
    B, L, Hq, Hkv, d = 2, 9000, 8, 2, 128
    say("decode split invariance")
    _, (qd4, kd, vd) = bf16_tensors(B, L, Hq, Hkv, d, seed=42)
    qd = qd4[:, -1].contiguous()
    for mode in (0, 1):
        base, base_lse = _decode(fa, qd, kd, vd, torch.float32, mode, num_splits=1)
        for ns in (2, 7, 0):
            o, lse = _decode(fa, qd, kd, vd, torch.float32, mode, num_splits=ns)
            assert (o - base).abs().max().item() <= 1e-5
            assert (lse - base_lse).abs().max().item() <= 1e-5


def test_decode_equals_prefill_last_row(fa):
    B, L, Hq, Hkv, d = 1, 3000, 8, 2, 128
    say("decode == prefill last row")
    _, (qd, kd, vd) = bf16_tensors(B, L, Hq, Hkv, d, seed=43)
    for mode in (0, 1):
        o = torch.empty((B, L, Hq, d), dtype=torch.float32, device=DEV)
        rp = ci = None
        if mode:
            r, c = fa.flux_build_block_mask(L, L, 64, 128, 512, 1, 1)
            rp, ci = torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV)
        fa.flux_attn_prefill(qd, kd, vd, o, None, causal=1, mode=mode, sink_tokens=128, window_tokens=512,
                             blk_row_ptr=rp, blk_col_idx=ci)
        dec, _ = _decode(fa, qd[:, -1].contiguous(), kd, vd, torch.float32, mode, sink=128, window=512)
        assert (dec - o[:, -1]).abs().max().item() <= 2e-3


def test_decode_full_size_dense_and_sparse(fa):
    """GQA decode: batch 8, KV length 262144, 32 query heads, 8 KV heads, head_dim 128, bf16 cache, dense
    and block-sparse (sink 128 + last 2048 tokens): every (sequence, head) output and LSE against the oracle,
    outputs NaN-filled before the call."""
    B, L, Hq, Hkv, d = 8, 262144, 32, 8, 128
    say("decode full size")
    qd = synth.torch_normal((B, Hq, d), 1005, torch.bfloat16)
    kd = synth.torch_normal((B, L, Hkv, d), 1006, torch.bfloat16)
    vd = synth.torch_normal((B, L, Hkv, d), 1007, torch.bfloat16)
    q = dev_bits_to_host(qd)
    outs = {mode: _decode(fa, qd, kd, vd, torch.float32, mode) for mode in (0, 1)}
    for mode, (o, lse) in outs.items():
        assert torch.isfinite(o).all() and torch.isfinite(lse).all(), f"mode {mode}: unwritten output"
    for b in range(B):
        kb = dev_bits_to_host(kd[b:b + 1])
        vb = dev_bits_to_host(vd[b:b + 1])
        for mode, (o, lse) in outs.items():
            ref, ref_lse = oracle.decode(np.ascontiguousarray(q[b:b + 1]), kb, vb, default_scale(d),
                                         sparse=bool(mode), block=64, sink_tokens=128, window_tokens=2048)
            check_close(o[b:b + 1].cpu().numpy(), ref, f"decode full mode {mode} b {b}")
            check_lse(lse[b:b + 1].cpu().numpy(), ref_lse, f"decode full lse mode {mode} b {b}")
    del qd, kd, vd
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ router
def _route_gpu(fa, xs_dev, w):
    L = len(xs_dev)
    wd = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w]
    modes = torch.full((L,), -7, dtype=torch.int32, device=DEV)
    logits = torch.full((L, 2), float("nan"), dtype=torch.float32, device=DEV)
    fa.flux_route_layers(xs_dev, *wd, modes, logits, pool_tokens=100)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), modes.cpu().numpy()


def _check_route(logits, modes, ref_logits, ref_modes, what):
    err = np.abs(logits - ref_logits)
    scale = np.maximum(1.0, np.abs(ref_logits))
    assert np.all(err <= 1e-4 * scale), f"{what}: logits max err {err.max():.3e}"
    margin = np.abs(ref_logits[:, 1] - ref_logits[:, 0])
    decided = margin > 1e-3          # decisions fp32 rounding cannot flip
    assert decided.mean() > 0.9, f"{what}: too many near-ties"
    np.testing.assert_array_equal(modes[decided], ref_modes[decided])
    # near-ties (if any) must still be the argmax of the GPU's own logits, tie -> dense
    own = (logits[:, 1] > logits[:, 0]).astype(np.int32)
    np.testing.assert_array_equal(modes, own)


@pytest.mark.parametrize("S,Hq,d,L", [(1, 2, 64, 3), (150, 4, 64, 5), (200, 8, 128, 4), (5000, 32, 128, 6)])
def test_router_small(fa, S, Hq, d, L):
    say("router", S, Hq, d, L)
    xs = [synth.normal_bf16_bits((S, Hq, d), 4000 + S, l, 0) for l in range(L)]
    w = synth.router_weights(L, Hq * d, 256, seed=4001)
    logits, modes = _route_gpu(fa, [synth.torch_bf16_from_bits(x) for x in xs], w)
    _, ref_logits, ref_modes = oracle.route(xs, *w)
    _check_route(logits, modes, ref_logits, ref_modes, "router small")


@pytest.mark.parametrize("hidden", [5, 37])
def test_router_odd_hidden_ragged_features_reused_workspace(fa, hidden):
    """A hidden width that is not a multiple of the encoder's 4 units per workgroup, 192 features (one
    and a half pooling blocks), and three calls on one workspace: each call resets the layers' arrival
    counters itself, so the last-arriving encoder workgroup runs the head every time."""
    S, Hq, d, L = 300, 3, 64, 2
    say("router odd hidden", hidden)
    xs = [synth.normal_bf16_bits((S, Hq, d), 4100 + hidden, l, 0) for l in range(L)]
    xs_dev = [synth.torch_bf16_from_bits(x) for x in xs]
    w = synth.router_weights(L, Hq * d, hidden, seed=4003)
    wd = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w]
    ws = torch.full((fa.flux_route_workspace_size(L, Hq, d, hidden),), 0x5A, dtype=torch.uint8, device=DEV)
    _, ref_logits, ref_modes = oracle.route(xs, *w)
    for rep in range(3):
        modes = torch.full((L,), -7, dtype=torch.int32, device=DEV)
        logits = torch.full((L, 2), float("nan"), dtype=torch.float32, device=DEV)
        fa.flux_route_layers(xs_dev, *wd, modes, logits, workspace=ws, pool_tokens=100)
        torch.cuda.synchronize()
        _check_route(logits.cpu().numpy(), modes.cpu().numpy(), ref_logits, ref_modes, f"router call {rep}")


def test_router_qwen_stack_shape(fa):
    """36 layers, seq 131072, 32 heads x 128: the pooled rows are the first and last 100 tokens."""
    S, Hq, d, L = 131072, 32, 128, 36
    say("router 36 layers")
    xs_dev = [synth.torch_normal((S, Hq, d), 5000 + l, torch.bfloat16) for l in range(L)]
    w = synth.router_weights(L, Hq * d, 256, seed=4002)
    logits, modes = _route_gpu(fa, xs_dev, w)
    # the oracle reads the 200 pooled rows only: [0,100) U [S-100, S) as a 200-token prompt
    xs_host = [np.concatenate([dev_bits_to_host(x[:100]), dev_bits_to_host(x[S - 100:])]) for x in xs_dev]
    _, ref_logits, ref_modes = oracle.route(xs_host, *w)
    _check_route(logits, modes, ref_logits, ref_modes, "router 36 layers")
    del xs_dev
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ decode loop: append + attend
def _window_row(t, sink, window):
    """Row of token t in a FLUX_KV_WINDOW cache (the layout documented in flux_attn.h)."""
    return t if t < sink else sink + ((t // 64) % (window // 64)) * 64 + t % 64


def test_decode_step_full_cache_appends_and_matches_oracle(fa):
    """Full-cache layout: the new token is written at row pos and attended to in the same launch."""
    B, Hq, Hkv, d, cap, pos = 2, 8, 2, 128, 1200, 777
    say("decode step full cache")
    k = synth.normal_bf16_bits((B, pos + 1, Hkv, d), 51, 0, synth.TENSOR_K)
    v = synth.normal_bf16_bits((B, pos + 1, Hkv, d), 51, 0, synth.TENSOR_V)
    q = synth.normal_bf16_bits((B, Hq, d), 51, 0, synth.TENSOR_Q)
    for mode in (0, 1):
        kc = torch.zeros((B, cap, Hkv, d), dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        kc[:, :pos] = synth.torch_bf16_from_bits(np.ascontiguousarray(k[:, :pos]))
        vc[:, :pos] = synth.torch_bf16_from_bits(np.ascontiguousarray(v[:, :pos]))
        kn = synth.torch_bf16_from_bits(np.ascontiguousarray(k[:, pos]))
        vn = synth.torch_bf16_from_bits(np.ascontiguousarray(v[:, pos]))
        qd = synth.torch_bf16_from_bits(q)
        o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        ws = torch.empty(fa.flux_decode_workspace_size(B, Hq, Hkv, pos + 1, d, mode, 64, 128, 256), dtype=torch.uint8,
                         device=DEV)
        fa.flux_decode_step(qd, kn, vn, kc, vc, o, lse, pos=pos, layout=fa.FLUX_KV_FULL, mode=mode, sink_tokens=128,
                            window_tokens=256, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(dev_bits_to_host(kc[:, pos]), k[:, pos])
        assert np.array_equal(dev_bits_to_host(vc[:, pos]), v[:, pos])
        assert not dev_bits_to_host(kc[:, pos + 1:]).any()
        ref, ref_lse = oracle.decode(q, k, v, default_scale(d), sparse=bool(mode), block=64, sink_tokens=128,
                                     window_tokens=256)
        check_close(o.cpu().numpy(), ref, f"decode step full mode {mode}")
        check_lse(lse.cpu().numpy(), ref_lse, "decode step lse")


def test_decode_loop_window_cache_ring(fa):
    """Sparse layer on a window cache, token by token from position 0: the cache keeps only the sink
    and a ring of window blocks, the ring wraps several times, and every step matches the oracle run
    on the full history (sink 128 tokens, window 256 = 4 blocks; 700 steps)."""
    B, Hq, Hkv, d, sink, window, n = 2, 4, 1, 128, 128, 256, 700
    say("decode loop window cache")
    rows = fa.flux_window_cache_rows(64, sink, window)
    assert rows == sink + window
    k = synth.normal_bf16_bits((B, n, Hkv, d), 52, 0, synth.TENSOR_K)
    v = synth.normal_bf16_bits((B, n, Hkv, d), 52, 0, synth.TENSOR_V)
    q = synth.normal_bf16_bits((n, B, Hq, d), 52, 0, synth.TENSOR_Q)
    kd, vd, qd = (synth.torch_bf16_from_bits(x) for x in (k, v, q))
    kc = torch.zeros((B, rows, Hkv, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    out = torch.full((n, B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.flux_decode_workspace_size(B, Hq, Hkv, n, d, 1, 64, sink, window), dtype=torch.uint8,
                     device=DEV)
    kn_all = kd.transpose(0, 1).contiguous()   # [n, B, Hkv, d]
    vn_all = vd.transpose(0, 1).contiguous()
    for pos in range(n):
        fa.flux_decode_step(qd[pos], kn_all[pos], vn_all[pos], kc, vc, out[pos], None, pos=pos,
                            layout=fa.FLUX_KV_WINDOW, mode=fa.FLUX_MODE_SPARSE, sink_tokens=sink,
                            window_tokens=window, workspace=ws)
    torch.cuda.synchronize()
    # the ring holds exactly the tokens the pattern can still reach at the last position
    kc_h = dev_bits_to_host(kc)
    last_blk = (n - 1) // 64
    for t in list(range(sink)) + list(range(max(sink, (last_blk - window // 64 + 1) * 64), n)):
        assert np.array_equal(kc_h[:, _window_row(t, sink, window)], k[:, t]), t
    out_h = out.cpu().numpy()
    for pos in sorted({0, 1, 63, 64, 127, 128, 129, 191, 192, 255, 256, 383, 384, 385, 447, 448, 511, 512, 575, 576,
                       640, 641, n - 1} | set(range(5, n, 37))):
        ref, _ = oracle.decode(q[pos], np.ascontiguousarray(k[:, :pos + 1]), np.ascontiguousarray(v[:, :pos + 1]),
                               default_scale(d), sparse=True, block=64, sink_tokens=sink, window_tokens=window)
        check_close(out_h[pos], ref, f"window decode pos {pos}")


def test_decode_step_layers_routed_stack(fa):
    """Three layers, modes [sparse, dense, sparse]: dense on a full cache, sparse on window caches."""
    B, Hq, Hkv, d, sink, window, pos, cap = 2, 8, 2, 128, 128, 256, 900, 1024
    say("decode step layers")
    modes = [1, 0, 1]
    L = len(modes)
    wrows = fa.flux_window_cache_rows(64, sink, window)
    ks = [synth.normal_bf16_bits((B, pos + 1, Hkv, d), 53, l, synth.TENSOR_K) for l in range(L)]
    vs = [synth.normal_bf16_bits((B, pos + 1, Hkv, d), 53, l, synth.TENSOR_V) for l in range(L)]
    qs = [synth.normal_bf16_bits((B, Hq, d), 53, l, synth.TENSOR_Q) for l in range(L)]
    kcs, vcs = [], []
    for l in range(L):
        if modes[l] == 0:
            kc = torch.zeros((B, cap, Hkv, d), dtype=torch.bfloat16, device=DEV)
            vc = torch.zeros_like(kc)
            kc[:, :pos] = synth.torch_bf16_from_bits(np.ascontiguousarray(ks[l][:, :pos]))
            vc[:, :pos] = synth.torch_bf16_from_bits(np.ascontiguousarray(vs[l][:, :pos]))
        else:   # fill the window cache with the tokens it holds before position pos
            kh = np.zeros((B, wrows, Hkv, d), np.uint16)
            vh = np.zeros_like(kh)
            blk = pos // 64
            for t in list(range(sink)) + list(range(max(sink, (blk - window // 64 + 1) * 64), pos)):
                kh[:, _window_row(t, sink, window)] = ks[l][:, t]
                vh[:, _window_row(t, sink, window)] = vs[l][:, t]
            kc, vc = synth.torch_bf16_from_bits(kh), synth.torch_bf16_from_bits(vh)
        kcs.append(kc)
        vcs.append(vc)
    kns = [synth.torch_bf16_from_bits(np.ascontiguousarray(x[:, pos])) for x in ks]
    vns = [synth.torch_bf16_from_bits(np.ascontiguousarray(x[:, pos])) for x in vs]
    qds = [synth.torch_bf16_from_bits(x) for x in qs]
    os_ = [torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(L)]
    ws = torch.empty(fa.flux_decode_workspace_size(B, Hq, Hkv, pos + 1, d, 0, 64, sink, window), dtype=torch.uint8,
                     device=DEV)
    fa.flux_decode_step_layers(modes, qds, kns, vns, kcs, vcs, os_, None, pos=pos, dense_cache_rows=cap,
                               sink_tokens=sink, window_tokens=window, workspace=ws)
    torch.cuda.synchronize()
    for l in range(L):
        ref, _ = oracle.decode(qs[l], ks[l], vs[l], default_scale(d), sparse=bool(modes[l]), block=64,
                               sink_tokens=sink, window_tokens=window)
        check_close(os_[l].cpu().numpy(), ref, f"decode layers l={l}")


# ------------------------------------------------------------------ scores far from N(0,1)
@pytest.mark.parametrize("mode,ns", [(0, 0), (0, 5), (1, 0)])
def test_decode_rising_scores(fa, mode, ns):
    """Scores that grow along the cache (q and k share a direction along which k grows with the
    position, ~6 per 64 keys): every step raises the running max, and the splits' LSEs differ by
    hundreds, so the combine weights of the early splits underflow to zero."""
    B, L, Hq, Hkv, d = 2, 3000, 8, 2, 128
    say("decode rising scores", mode, ns)
    q = synth.bf16_bits_to_f32(synth.normal_bf16_bits((B, Hq, d), 3500, 0, synth.TENSOR_Q))
    k = synth.bf16_bits_to_f32(synth.normal_bf16_bits((B, L, Hkv, d), 3500, 0, synth.TENSOR_K))
    v = synth.normal_bf16_bits((B, L, Hkv, d), 3500, 0, synth.TENSOR_V)
    u = np.full(d, 1.0 / np.sqrt(d), np.float32)
    q = 0.5 * q + 6.0 * u
    k = 0.5 * k + (np.arange(L, dtype=np.float32) / 64.0 * np.sqrt(d))[None, :, None, None] * u
    q, k = (synth.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)) for x in (q, k))
    qd, kd, vd = (synth.torch_bf16_from_bits(x) for x in (q, k, v))
    o, lse = _decode(fa, qd, kd, vd, torch.float32, mode, sink=128, window=1024, num_splits=ns)
    ref, ref_lse = oracle.decode(q, k, v, default_scale(d), sparse=bool(mode), block=64, sink_tokens=128,
                                 window_tokens=1024)
    check_close(o.cpu().numpy(), ref, "decode rising")
    check_lse(lse.cpu().numpy(), ref_lse, "decode rising lse")


# ------------------------------------------------------------------ graph capture of a decode step
def test_decode_step_layers_graph_replay(fa):
    """The routed decode step of a small stack captured in a HIP graph (the launch-bound loop a serving
    engine replays): every replay, with eager work between replays, reproduces the eager outputs bit
    for bit (the step allocates nothing and issues no memset)."""
    B, Hq, Hkv, d, sink, window, pos, cap = 2, 8, 2, 128, 128, 256, 900, 1024
    say("decode step layers, graph replay")
    modes = [1, 0, 1, 0]
    L = len(modes)
    wrows = fa.flux_window_cache_rows(64, sink, window)
    qds = [synth.torch_normal((B, Hq, d), 61 + l, torch.bfloat16) for l in range(L)]
    kns = [synth.torch_normal((B, Hkv, d), 71 + l, torch.bfloat16) for l in range(L)]
    vns = [synth.torch_normal((B, Hkv, d), 81 + l, torch.bfloat16) for l in range(L)]
    kcs = [synth.torch_normal((B, cap if m == 0 else wrows, Hkv, d), 91 + l, torch.bfloat16) for l, m in enumerate(modes)]
    vcs = [synth.torch_normal((B, cap if m == 0 else wrows, Hkv, d), 101 + l, torch.bfloat16) for l, m in enumerate(modes)]
    os_ = [torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(L)]
    ws = torch.empty(fa.flux_decode_workspace_size(B, Hq, Hkv, pos + 1, d, 0, 64, sink, window), dtype=torch.uint8,
                     device=DEV)

    def step():
        fa.flux_decode_step_layers(modes, qds, kns, vns, kcs, vcs, os_, None, pos=pos, dense_cache_rows=cap,
                                   sink_tokens=sink, window_tokens=window, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in os_]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in os_:
            o.fill_(float("nan"))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(os_[l], eager[l]), f"replay {rep} layer {l}"
    del g
