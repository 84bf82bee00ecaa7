"""GPU parity of the attention backward (dQ, dK, dV) vs the fp64 oracle.

Every call goes through the C ABI (flux_attn_backward) via the thin binding.  Inputs: seeded iid
N(0,1) Q, K, V and output gradient dO, rounded to bf16; the oracle reads the same bits.  The
forward output O and row LSE handed to the backward come from the oracle's forward (fp64, rounded
to fp32) unless a test says otherwise.  Bar: max-abs <= 1e-2 and mean-abs <= 1e-3 on the fp32
gradients.  A bf16 O (one test) perturbs D = rowsum(dO * O) by its own rounding, which the kernel
cannot undo; that case is held to max-abs 2e-2.  At the full layer shape (seq 8192, 32/8 heads) the
oracle cannot run whole: there dQ rows of a causal prefix are compared (rows < T depend only on
keys < T), dK, dV are checked against identities that hold at any size and element-wise on four
sampled key blocks against the oracle's gradients of those keys only.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import check_close, default_scale, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128


@pytest.fixture(scope="module")
def fa():
    import long_context_attention_tiled_amd as fa
    assert torch.cuda.is_available()
    return fa


def _inputs(B, S, Hq, Hkv, seed, d=D):
    q, k, v = synth.qkv_bf16(B, S, Hq, Hkv, d, seed)
    g = synth.normal_bf16_bits((B, S, Hq, d), seed, tensor_id=7)
    return q, k, v, g


def _oracle_forward(q, k, v, scale, causal, sparse, sink, window):
    out, lse = oracle.attention(q, k, v, scale, causal=causal, sparse=sparse, block=64, sink_tokens=sink,
                                window_tokens=window)
    return out.astype(np.float32), np.ascontiguousarray(np.transpose(lse, (0, 2, 1))).astype(np.float32)


def _gpu_forward(fa, qd, kd, vd, causal, mode, sink, window, o_dtype=torch.float32):
    B, S, Hq, d = qd.shape
    o = torch.empty((B, S, Hq, d), dtype=o_dtype, device=DEV)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    rp = ci = None
    if mode == fa.FLUX_MODE_SPARSE:
        rp, ci = fa.flux_build_block_mask(S, S, 64, sink, window, 1, fa.FLUX_MODE_SPARSE)
        rp, ci = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    fa.flux_attn_prefill(qd, kd, vd, o, lse, causal=int(causal), mode=mode, block=64, sink_tokens=sink,
                         window_tokens=window, blk_row_ptr=rp, blk_col_idx=ci)
    return o, lse


def _backward(fa, qd, kd, vd, od, gd, lsed, causal, mode, sink, window):
    B, S, Hq, d = qd.shape
    Hkv = kd.shape[2]
    dq = torch.full((B, S, Hq, d), float("nan"), dtype=torch.float32, device=DEV)   # unwritten elements fail
    dk = torch.full((B, S, Hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full((B, S, Hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    fa.flux_attn_backward(qd, kd, vd, od, gd, lsed, dq, dk, dv, causal=causal, mode=mode, block=64,
                          sink_tokens=sink, window_tokens=window)
    torch.cuda.synchronize()
    return dq, dk, dv


def _run_case(fa, B, S, Hq, Hkv, seed, causal=True, mode=0, sink=0, window=0, gpu_forward=False, o_bf16=False,
              max_abs=None, d=D):
    say("backward", f"B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} seed={seed} causal={causal} mode={mode} sink={sink} "
        f"window={window} gpu_forward={gpu_forward} o_bf16={o_bf16}")
    scale = default_scale(d)
    sparse = mode == 1
    q, k, v, g = _inputs(B, S, Hq, Hkv, seed, d)
    qd, kd, vd, gd = (synth.torch_bf16_from_bits(x) for x in (q, k, v, g))
    if gpu_forward:
        od, lsed = _gpu_forward(fa, qd, kd, vd, causal, mode, sink, window,
                                torch.bfloat16 if o_bf16 else torch.float32)
    else:
        o32, lse = _oracle_forward(q, k, v, scale, causal, sparse, sink, window)
        od = synth.torch_bf16_from_bits(synth.f32_to_bf16_bits(o32)) if o_bf16 else torch.from_numpy(o32).to(DEV)
        lsed = torch.from_numpy(lse).to(DEV)
    dq, dk, dv = _backward(fa, qd, kd, vd, od, gd, lsed, causal, mode, sink, window)
    rq, rk, rv = oracle.attention_backward(q, k, v, g, scale, causal=causal, sparse=sparse, block=64,
                                           sink_tokens=sink, window_tokens=window)
    tag = f"S={S} Hq={Hq} Hkv={Hkv} d={d} mode={mode}"
    errs = [_close(t.cpu().numpy(), r, f"{name} {tag}", max_abs)
            for name, t, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))]
    say("max/mean abs err", " ".join(f"{e[0]:.2e}/{e[1]:.1e}" for e in errs))


def _close(gpu, ref, what, max_abs):
    if max_abs is None:
        return check_close(gpu, ref, what)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    assert np.all(np.isfinite(gpu)), what
    assert err.max() <= max_abs, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= 1e-3, f"{what}: mean-abs {err.mean():.3e}"
    return float(err.max()), float(err.mean())


# ------------------------------------------------------------- dense
@pytest.mark.parametrize("S", [1, 64, 65, 328])
def test_dense_causal_mha(fa, S):
    """Several key pairs and query pairs, a ragged last tile, and the one-row / one-tile edges."""
    _run_case(fa, 1, S, 2, 2, seed=4101 + S)


def test_dense_causal_gqa(fa):
    """Grouped-query attention (4 query heads on 2 KV heads): per-head dK/dV summed in head order."""
    _run_case(fa, 2, 256, 4, 2, seed=4201)


def test_dense_causal_odd_group(fa):
    """Three query heads per KV head (6 on 2)."""
    _run_case(fa, 1, 300, 6, 2, seed=4251)


def test_dense_noncausal(fa):
    """All keys visible; the ragged last key tile is masked by position."""
    _run_case(fa, 1, 200, 2, 1, causal=False, seed=4301)


def test_dense_causal_longer(fa):
    _run_case(fa, 1, 1100, 2, 1, seed=4401)


@pytest.mark.parametrize("causal", [True, False])
def test_head_dim_64(fa, causal):
    """head_dim 64 (the tiny layer's width), GQA 4 on 2, ragged end."""
    _run_case(fa, 1, 330, 4, 2, causal=causal, seed=4351, d=64)


def test_head_dim_64_sparse(fa):
    """head_dim 64, block-sparse with the tiny layer's pattern (sink 2 blocks, window 2 blocks)."""
    _run_case(fa, 1, 512, 2, 2, mode=1, sink=128, window=128, seed=4361, d=64)


# ------------------------------------------------------------- block-sparse
def test_sparse_sink_window(fa):
    """Sink 2 blocks, window 4 blocks over 16 query blocks: most blocks skipped, ragged end."""
    _run_case(fa, 1, 1000, 2, 1, mode=1, sink=128, window=256, seed=4501)


def test_sparse_odd_sink(fa):
    """One sink block: the first key pair straddles the sink boundary."""
    _run_case(fa, 1, 700, 2, 2, mode=1, sink=64, window=128, seed=4601)


def test_sparse_no_sink_min_window(fa):
    """No sink and a one-block window: only the diagonal blocks are visible."""
    _run_case(fa, 1, 450, 2, 1, mode=1, sink=0, window=64, seed=4701)


def test_sparse_batch2_gqa(fa):
    """Two sequences, 4 query heads on one KV head, sink 2 blocks, window 2 blocks, ragged end."""
    _run_case(fa, 2, 500, 4, 1, mode=1, sink=128, window=128, seed=4751)


def test_sparse_odd_group_two_sink_pairs(fa):
    """Three query heads per KV head, a 3-block sink (two key pairs hold sink blocks, so they run per query
    head and are summed over the group afterwards; the other pairs take the group's heads in one unit),
    two sequences, ragged end."""
    _run_case(fa, 2, 700, 6, 2, mode=1, sink=192, window=128, seed=4771)


def test_sparse_group_of_eight_no_sink(fa):
    """Eight query heads per KV head on the block-sparse path with no sink (every key pair is a grouped
    unit) and a 3-block window, ragged end."""
    _run_case(fa, 1, 600, 8, 1, mode=1, sink=0, window=192, seed=4791)


def test_dense_causal_group_of_eight_batch2(fa):
    """Two sequences, eight query heads per KV head, dense causal, ragged end."""
    _run_case(fa, 2, 390, 16, 2, seed=4793)


def test_bf16_output_input(fa):
    """O handed over in bf16: D carries O's rounding (up to 2^-9 relative per element)."""
    _run_case(fa, 1, 328, 2, 2, seed=4429, o_bf16=True, max_abs=2e-2)


# ------------------------------------------------------------- float32 inputs (vector-ALU kernels)
def _run_case_f32(fa, B, S, Hq, Hkv, d, seed, causal=True, mode=0, sink=0, window=0):
    say("backward f32", f"B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} seed={seed} causal={causal} mode={mode} sink={sink} "
        f"window={window}")
    scale = default_scale(d)
    sparse = mode == 1
    q, k, v = synth.qkv_f32(B, S, Hq, Hkv, d, seed)
    g = synth.normal_f32((B, S, Hq, d), seed, tensor_id=7)
    o32, lse = _oracle_forward(q, k, v, scale, causal, sparse, sink, window)
    qd, kd, vd, gd, od = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (q, k, v, g, o32))
    lsed = torch.from_numpy(lse).to(DEV)
    dq, dk, dv = _backward(fa, qd, kd, vd, od, gd, lsed, causal, mode, sink, window)
    rq, rk, rv = oracle.attention_backward(q, k, v, g, scale, causal=causal, sparse=sparse, block=64,
                                           sink_tokens=sink, window_tokens=window)
    tag = f"f32 S={S} Hq={Hq} Hkv={Hkv} d={d} mode={mode}"
    for name, t, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check_close(t.cpu().numpy(), r, f"{name} {tag}")


@pytest.mark.parametrize("mode", [0, 1])
def test_f32_tiny_layer(fa, mode):
    """The tiny float32 layer: batch 1, 2 heads, head_dim 64, seq 512; dense causal, then block-sparse
    with sink 2 blocks and window 2 blocks."""
    _run_case_f32(fa, 1, 512, 2, 2, 64, seed=5001, mode=mode, sink=128, window=128)


def test_f32_gqa_noncausal_ragged(fa):
    _run_case_f32(fa, 1, 330, 4, 2, 128, seed=5011, causal=False)


def test_f32_gqa_causal_ragged(fa):
    _run_case_f32(fa, 2, 200, 6, 2, 128, seed=5021)


# ------------------------------------------------------------- end to end with the GPU forward
@pytest.mark.parametrize("mode", [0, 1])
def test_after_gpu_forward(fa, mode):
    """O (fp32) and LSE from flux_attn_prefill, then the backward."""
    _run_case(fa, 1, 512, 4, 1, mode=mode, sink=128, window=128, seed=4801 + mode, gpu_forward=True)


# ------------------------------------------------------------- full layer shape
@pytest.mark.parametrize("S,mode", [(8192, 0), (8192, 1), (65536, 1)])
def test_full_shape_prefix_and_identities(fa, S, mode):
    """seq 8192 (dense and sparse) and seq 65536 sparse, 32 query heads on 8 KV heads: the shapes the
    benchmark times.
    dQ of the first T rows equals the backward of the length-T prefix (causal); dK, dV are checked
    against sum_j dV_j = sum over the group's heads of sum_i dO_i (rows of P sum to one) and
    sum_j dK_j = 0 (rows of dS sum to zero), and element-wise on four 64-key blocks (sink, window
    width, middle, last) against the oracle's gradients for those keys; every element written (NaN
    fill); a second run must be bit-identical."""
    B, Hq, Hkv, T = 1, 32, 8, 384
    sink, window = (128, 2048) if mode == 1 else (0, 0)
    say("backward full shape", f"S={S} mode={mode}")
    scale = default_scale(D)
    q, k, v, g = _inputs(B, S, Hq, Hkv, seed=4901 + mode + S)
    qd, kd, vd, gd = (synth.torch_bf16_from_bits(x) for x in (q, k, v, g))
    od, lsed = _gpu_forward(fa, qd, kd, vd, True, mode, sink, window)
    dq, dk, dv = _backward(fa, qd, kd, vd, od, gd, lsed, True, mode, sink, window)
    dq2, dk2, dv2 = _backward(fa, qd, kd, vd, od, gd, lsed, True, mode, sink, window)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), "not deterministic"
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()

    # prefix rows of dQ
    pq, pk, pv, pg = (np.ascontiguousarray(x[:, :T]) for x in (q, k, v, g))
    rq, _, _ = oracle.attention_backward(pq, pk, pv, pg, scale, causal=True, sparse=bool(mode), block=64,
                                         sink_tokens=sink, window_tokens=window)
    check_close(dq[:, :T].cpu().numpy(), rq, f"dq prefix mode {mode}")

    # identities over keys, per (batch, kv head, d)
    G = Hq // Hkv
    g64 = synth.bf16_bits_to_f32(g).astype(np.float64)                    # [B, S, Hq, d]
    want_dv = g64.sum(axis=1).reshape(B, Hkv, G, D).sum(axis=2)         # [B, Hkv, d]
    got_dv = dv.double().sum(dim=1).cpu().numpy()
    got_dk = dk.double().sum(dim=1).cpu().numpy()
    mag_v = float(np.abs(dv.cpu().numpy()).sum(axis=1).max())
    mag_k = float(np.abs(dk.cpu().numpy()).sum(axis=1).max())
    err_v = float(np.abs(got_dv - want_dv).max())
    err_k = float(np.abs(got_dk).max())
    say("identities", f"sum dV err {err_v:.3e} (scale {mag_v:.1f}), sum dK {err_k:.3e} (scale {mag_k:.1f})")
    # dV's identity is exact up to the rounding of the sums (measured ~1e-6 of the scale); dK's also carries
    # the forward's rounding of O through D = rowsum(dO * O) (measured ~1e-4 of the scale)
    assert err_v <= 2e-5 * mag_v, err_v
    assert err_k <= 1e-3 * mag_k, err_k

    # element-wise dK/dV of four key blocks, each on its own KV head: the first sink block, the block at the
    # window's width, a middle block and the last block (a key written to another block's rows fails here,
    # unlike the sums above)
    nb = S // 64
    picks = [(0, 0), (32, 3), (nb // 2 + 5, 5), (nb - 1, Hkv - 1)]
    keys = np.array([(0, kvh, 64 * blk + j) for blk, kvh in picks for j in range(64)], np.int64)
    say("dK/dV key blocks", picks)
    rk, rv = oracle.attention_backward_keys(q, k, v, g, scale, keys, causal=True, sparse=bool(mode), block=64,
                                            sink_tokens=sink, window_tokens=window)
    dk_h, dv_h = dk.cpu().numpy(), dv.cpu().numpy()
    for (blk, gh), sl in zip(picks, range(0, len(keys), 64)):
        rows = keys[sl:sl + 64]
        check_close(dk_h[rows[:, 0], rows[:, 2], rows[:, 1]], rk[sl:sl + 64], f"dK block {blk} kv head {gh}")
        check_close(dv_h[rows[:, 0], rows[:, 2], rows[:, 1]], rv[sl:sl + 64], f"dV block {blk} kv head {gh}")


# ------------------------------------------------------------- scores far from N(0,1)
@pytest.mark.parametrize("mode", [0, 1])
def test_sharp_scores(fa, mode):
    """Q, K scaled by 4 (scores of std ~16): P is nearly one-hot per row, exp2(S * scale * log2e - LSE *
    log2e) spans the whole fp32 range and underflows for most keys."""
    B, S, Hq, Hkv, d = 1, 400, 4, 2, 128
    say("backward sharp", mode)
    scale = default_scale(d)
    q, k, v = (synth.bf16_bits_to_f32(x) for x in synth.qkv_bf16(B, S, Hq, Hkv, d, 4951))
    q, k = (synth.f32_to_bf16_bits(np.ascontiguousarray(4.0 * x)) for x in (q, k))
    v = synth.f32_to_bf16_bits(v)
    g = synth.normal_bf16_bits((B, S, Hq, d), 4951, tensor_id=7)
    sink, window = (64, 128) if mode else (0, 0)
    qd, kd, vd, gd = (synth.torch_bf16_from_bits(x) for x in (q, k, v, g))
    o32, lse = _oracle_forward(q, k, v, scale, True, bool(mode), sink, window)
    dq, dk, dv = _backward(fa, qd, kd, vd, torch.from_numpy(o32).to(DEV), gd, torch.from_numpy(lse).to(DEV), True,
                           mode, sink, window)
    rq, rk, rv = oracle.attention_backward(q, k, v, g, scale, causal=True, sparse=bool(mode), block=64,
                                           sink_tokens=sink, window_tokens=window)
    for name, t, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _close(t.cpu().numpy(), r, f"sharp {name} mode {mode}", None)


# ------------------------------------------------------------- input magnitudes
@pytest.mark.parametrize("mode,d", [(0, 128), (1, 128), (1, 64)])
def test_group_magnitudes(fa, mode, d):
    """Each (batch, KV group)'s Q, K, V and dO scaled by its own powers of two, 2^-40 .. 2^20 (exact in bf16),
    with the softmax scale divided by the common Q K factor so the probabilities stay those of the unscaled
    layer.  The gradients scale exactly: dV by e, dK by c e / b, dQ by c e / a (a, b, c, e the group's Q, K,
    V, dO factors); divided by them they must meet the bar against the oracle's unscaled gradients, which
    only holds if the kernels' fp16 scaling follows each (batch, KV group)'s own range."""
    B, S, Hq, Hkv = 2, 328, 4, 2
    G = Hq // Hkv
    say("backward group magnitudes", mode, d)
    scale = default_scale(d)
    q, k, v, g = _inputs(B, S, Hq, Hkv, seed=5011, d=d)
    sink, window = (64, 128) if mode else (0, 0)
    o32, lse = _oracle_forward(q, k, v, scale, True, bool(mode), sink, window)
    rq, rk, rv = oracle.attention_backward(q, k, v, g, scale, causal=True, sparse=bool(mode), block=64,
                                           sink_tokens=sink, window_tokens=window)
    # per (batch, group): Q factor a, K factor b (a * b = 2^8 everywhere), V factor c, dO factor e
    fq = [[2.0 ** 20, 2.0 ** -4], [2.0 ** 3, 2.0 ** 9]]
    fk = [[2.0 ** -12, 2.0 ** 12], [2.0 ** 5, 2.0 ** -1]]
    fv = [[2.0 ** -30, 2.0 ** 6], [2.0 ** 11, 2.0 ** -17]]
    fo = [[2.0 ** -40, 2.0 ** 12], [2.0 ** -3, 2.0 ** -25]]
    qs, ks, vs, gs = (synth.bf16_bits_to_f32(x).copy() for x in (q, k, v, g))
    os_ = o32.copy()
    for bb in range(B):
        for grp in range(Hkv):
            assert fq[bb][grp] * fk[bb][grp] == 2.0 ** 8
            hs = slice(grp * G, (grp + 1) * G)
            qs[bb, :, hs] *= fq[bb][grp]
            gs[bb, :, hs] *= fo[bb][grp]
            os_[bb, :, hs] *= fv[bb][grp]
            ks[bb, :, grp] *= fk[bb][grp]
            vs[bb, :, grp] *= fv[bb][grp]
    qd, kd, vd, gd = (synth.torch_bf16_from_bits(synth.f32_to_bf16_bits(x)) for x in (qs, ks, vs, gs))
    dq = torch.full((B, S, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full((B, S, Hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full((B, S, Hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    fa.flux_attn_backward(qd, kd, vd, torch.from_numpy(os_).to(DEV), gd, torch.from_numpy(lse).to(DEV), dq, dk, dv,
                          causal=True, mode=mode, block=64, sink_tokens=sink, window_tokens=window,
                          scale=scale / 2.0 ** 8)
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    for bb in range(B):
        for grp in range(Hkv):
            hs = slice(grp * G, (grp + 1) * G)
            dq[bb, :, hs] /= fv[bb][grp] * fo[bb][grp] / fq[bb][grp]
            dk[bb, :, grp] /= fv[bb][grp] * fo[bb][grp] / fk[bb][grp]
            dv[bb, :, grp] /= fo[bb][grp]
    for name, t, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _close(t, r, f"magnitudes {name} mode {mode} d {d}", None)


def test_zero_output_gradient(fa):
    """dO = 0 (its scale exponent falls back to 0): every gradient is exactly zero."""
    B, S, Hq, Hkv, d = 1, 200, 4, 2, 128
    say("backward zero dO")
    scale = default_scale(d)
    q, k, v, _ = _inputs(B, S, Hq, Hkv, seed=5021)
    o32, lse = _oracle_forward(q, k, v, scale, True, False, 0, 0)
    qd, kd, vd = (synth.torch_bf16_from_bits(x) for x in (q, k, v))
    gd = torch.zeros((B, S, Hq, d), dtype=torch.bfloat16, device=DEV)
    dq, dk, dv = _backward(fa, qd, kd, vd, torch.from_numpy(o32).to(DEV), gd, torch.from_numpy(lse).to(DEV), True, 0,
                           0, 0)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool((t == 0).all()), name


# ------------------------------------------------------------- graph capture
def test_backward_graph_replay(fa):
    """The backward (row statistics, dK/dV, dQ, sink-key GQA sum) captured in a HIP graph: its work queues
    are reset by its own first kernel, so every replay, with eager work between replays, reproduces the
    eager gradients bit for bit."""
    B, S, Hq, Hkv, d, mode, sink, window = 1, 600, 4, 2, 128, 1, 128, 128
    say("backward graph replay")
    scale = default_scale(d)
    q, k, v, g = _inputs(B, S, Hq, Hkv, seed=4991)
    qd, kd, vd, gd = (synth.torch_bf16_from_bits(x) for x in (q, k, v, g))
    o32, lse = _oracle_forward(q, k, v, scale, True, True, sink, window)
    od, lsed = torch.from_numpy(o32).to(DEV), torch.from_numpy(lse).to(DEV)
    dq = torch.empty((B, S, Hq, d), dtype=torch.float32, device=DEV)
    dk = torch.empty((B, S, Hkv, d), dtype=torch.float32, device=DEV)
    dv = torch.empty_like(dk)
    ws = torch.empty(fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, mode, 64, sink), dtype=torch.uint8,
                     device=DEV)

    def step():
        fa.flux_attn_backward(qd, kd, vd, od, gd, lsed, dq, dk, dv, causal=True, mode=mode, block=64,
                              sink_tokens=sink, window_tokens=window, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("dq", "dk", "dv"), (dq, dk, dv), eager):
            assert torch.equal(t, e), f"replay {rep} {name}"
    del graph
