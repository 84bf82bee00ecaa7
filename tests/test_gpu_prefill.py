"""GPU parity of the prefill path (dense causal, dense non-causal, block-sparse) vs the fp64 oracle.

Every call goes through the C ABI (libflux_attn.so) via the thin binding.
Inputs: seeded iid N(0,1), rounded to bf16 (the fp32 case keeps float32); the
oracle reads exactly the same bits.  Bar: max-abs <= 1e-2 and mean-abs <= 1e-3
with fp32 outputs; bf16 outputs may differ by a further half bf16 ulp.  Output
buffers are NaN-filled before each call, so an element the kernels never write
fails.  At seq 8192 every row is compared; at seq 65536 and 131072 one seeded
row of every 32-row wave segment of every head (1024-row segments for the dense
seq-131072 layer), plus every element checked written.
"""
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


def _csr_dev(fa, S, sink, window):
    rp, ci = fa.flux_build_block_mask(S, S, 64, sink, window, 1, fa.FLUX_MODE_SPARSE)
    return torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)


def _run_prefill(fa, qd, kd, vd, out_dtype, mode, causal=1, sink=128, window=2048, with_lse=True):
    B, S, Hq, d = qd.shape
    # NaN-filled, so an output element the kernels never write fails the comparison
    o = torch.full((B, S, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV) if with_lse else None
    rp = ci = None
    if mode == fa.FLUX_MODE_SPARSE:
        rp, ci = _csr_dev(fa, S, sink, window)
    fa.flux_attn_prefill(qd, kd, vd, o, lse, causal=causal, mode=mode, block=64, sink_tokens=sink,
                         window_tokens=window, blk_row_ptr=rp, blk_col_idx=ci)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------- tiny fp32 layer (both modes)
@pytest.mark.parametrize("mode", [0, 1])
def test_tiny_fp32_layer(fa, mode):
    """batch 1, 2 query heads = 2 KV heads, head_dim 64, seq 512, scale 1/8; dense causal, then
    block-sparse with block 64, sink 128 (2 blocks), window 2 blocks."""
    B, S, H, d = 1, 512, 2, 64
    say("tiny fp32", "mode", mode)
    q, k, v = synth.qkv_f32(B, S, H, H, d, seed=1001)
    qd, kd, vd = (torch.from_numpy(x).to(DEV) for x in (q, k, v))
    o, lse = _run_prefill(fa, qd, kd, vd, torch.float32, mode, sink=128, window=128)
    ref, ref_lse = oracle.attention(q, k, v, 1.0 / 8, causal=True, sparse=bool(mode), block=64, sink_tokens=128,
                                    window_tokens=128)
    check_close(o.cpu().numpy(), ref, f"tiny fp32 mode {mode}")
    check_lse(lse.cpu().numpy(), np.transpose(ref_lse, (0, 2, 1)), "tiny fp32 lse")


# ------------------------------------------------------------- bf16, small shapes, full oracle
SMALL = [
    # B, S, Hq, Hkv, d, mode, causal, sink, window
    (1, 1, 4, 1, 128, 0, 1, 128, 2048),
    (1, 63, 4, 1, 128, 0, 1, 128, 2048),
    (1, 64, 2, 2, 128, 0, 1, 128, 2048),
    (2, 129, 8, 2, 128, 0, 1, 128, 2048),
    (1, 777, 4, 1, 128, 0, 1, 128, 2048),
    (1, 300, 4, 2, 64, 0, 1, 128, 2048),
    (1, 200, 2, 1, 128, 0, 0, 128, 2048),     # non-causal, ragged
    (2, 130, 4, 4, 64, 0, 0, 128, 2048),
    (1, 1000, 4, 1, 128, 1, 1, 128, 128),     # sparse, window 2 blocks, ragged tail
    (1, 1024, 4, 2, 128, 1, 1, 128, 256),
    (2, 517, 8, 2, 64, 1, 1, 64, 192),
    (1, 640, 2, 1, 128, 1, 1, 0, 64),          # no sink, window of one block
    (1, 100, 2, 1, 128, 1, 1, 128, 128),       # shorter than the sink
    (1, 700, 8, 1, 128, 1, 1, 128, 320),       # 8 query heads per KV head, window of 5 blocks, ragged
    (1, 450, 3, 1, 64, 1, 1, 192, 128),        # odd group (two query tiles per workgroup), sink of 3 blocks
    (1, 333, 6, 2, 128, 0, 1, 128, 2048),      # odd group, dense causal, ragged
    (3, 200, 2, 1, 128, 1, 1, 64, 64),         # batch 3, one-block sink and window
]


@pytest.mark.parametrize("B,S,Hq,Hkv,d,mode,causal,sink,window", SMALL)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_bf16_small_full_oracle(fa, B, S, Hq, Hkv, d, mode, causal, sink, window, out_dtype):
    say("bf16 small", B, S, Hq, Hkv, d, "mode", mode, "causal", causal, sink, window, out_dtype)
    (q, k, v), (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=2000 + S)
    o, lse = _run_prefill(fa, qd, kd, vd, out_dtype, mode, causal=causal, sink=sink, window=window)
    ref, ref_lse = oracle.attention(q, k, v, default_scale(d), causal=bool(causal), sparse=bool(mode), block=64,
                                    sink_tokens=sink, window_tokens=window)
    check_close(o.float().cpu().numpy(), ref, "bf16 small", out_bf16=out_dtype == torch.bfloat16)
    check_lse(lse.cpu().numpy(), np.transpose(ref_lse, (0, 2, 1)), "bf16 small lse")


def test_sparse_full_window_equals_dense(fa):
    """A window covering every block makes the sparse path identical to dense causal."""
    B, S, Hq, Hkv, d = 1, 700, 4, 2, 128
    say("sparse full window == dense")
    _, (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=31)
    o_d, l_d = _run_prefill(fa, qd, kd, vd, torch.float32, 0)
    o_s, l_s = _run_prefill(fa, qd, kd, vd, torch.float32, 1, sink=128, window=64 * 11)
    assert torch.equal(o_d, o_s) and torch.equal(l_d, l_s)


@pytest.mark.parametrize("B,S,Hq,Hkv,d,sink,window", [
    (1, 1000, 4, 1, 128, 128, 128),     # ragged tail, window 2 blocks
    (2, 517, 8, 2, 64, 64, 192),
    (1, 640, 2, 1, 128, 0, 64),          # no sink, one-block window
    (1, 100, 2, 1, 128, 128, 128),       # shorter than the sink
    (1, 450, 3, 1, 64, 192, 128),        # odd group (four query blocks per workgroup), 3-block sink
    (1, 700, 8, 1, 128, 128, 320),       # 8 query heads per KV head
])
def test_sparse_without_csr_equals_csr(fa, B, S, Hq, Hkv, d, sink, window):
    """Block-sparse prefill with no CSR derives the key blocks from (sink, window) arithmetically: the
    outputs equal the CSR walk's bit for bit, and the oracle's."""
    say("sparse without CSR", B, S, Hq, Hkv, d, sink, window)
    (q, k, v), (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=2400 + S)
    o_c, l_c = _run_prefill(fa, qd, kd, vd, torch.float32, 1, sink=sink, window=window)
    o_a = torch.full_like(o_c, float("nan"))
    l_a = torch.full_like(l_c, float("nan"))
    fa.flux_attn_prefill(qd, kd, vd, o_a, l_a, causal=1, mode=fa.FLUX_MODE_SPARSE, block=64, sink_tokens=sink,
                         window_tokens=window)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_c) and torch.equal(l_a, l_c)
    ref, _ = oracle.attention(q, k, v, default_scale(d), causal=True, sparse=True, block=64, sink_tokens=sink,
                              window_tokens=window)
    check_close(o_a.cpu().numpy(), ref, "sparse without CSR")


def test_sparse_without_csr_fp32_inputs(fa):
    """The float32-input kernel's arithmetic walk (tiny layer: 2 heads, head_dim 64, sink 2 blocks, window 2)."""
    B, S, H, d = 1, 512, 2, 64
    q, k, v = synth.qkv_f32(B, S, H, H, d, seed=1001)
    qd, kd, vd = (torch.from_numpy(x).to(DEV) for x in (q, k, v))
    o_c, _ = _run_prefill(fa, qd, kd, vd, torch.float32, 1, sink=128, window=128)
    o_a = torch.full_like(o_c, float("nan"))
    fa.flux_attn_prefill(qd, kd, vd, o_a, None, causal=1, mode=fa.FLUX_MODE_SPARSE, sink_tokens=128, window_tokens=128)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_c)


def test_prefill_deterministic(fa):
    B, S, Hq, Hkv, d = 1, 1500, 8, 2, 128
    say("determinism")
    _, (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=32)
    for mode in (0, 1):
        a, la = _run_prefill(fa, qd, kd, vd, torch.float32, mode, sink=128, window=256)
        b, lb = _run_prefill(fa, qd, kd, vd, torch.float32, mode, sink=128, window=256)
        assert torch.equal(a, b) and torch.equal(la, lb)


def test_gqa_matches_repeated_kv(fa):
    B, S, Hq, Hkv, d = 1, 333, 8, 2, 128
    say("gqa == mha repeated")
    _, (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=33)
    kr = kd.repeat_interleave(Hq // Hkv, dim=2).contiguous()
    vr = vd.repeat_interleave(Hq // Hkv, dim=2).contiguous()
    for mode in (0, 1):
        a, _ = _run_prefill(fa, qd, kd, vd, torch.float32, mode, sink=64, window=128)
        b, _ = _run_prefill(fa, qd, kr, vr, torch.float32, mode, sink=64, window=128)
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,S,Hq,Hkv,d,mode", [
    (1, 4000, 32, 8, 128, 0),   # persistent schedule (512 units), ragged last tile
    (1, 4000, 32, 8, 128, 1),
    (2, 1337, 6, 3, 64, 0),     # odd query-head group: two row tiles of one head per workgroup
    (1, 777, 4, 4, 64, 1),
])
def test_bf16_output_is_rounded_f32_output(fa, B, S, Hq, Hkv, d, mode):
    """bf16 outputs leave through a per-wave LDS stage as whole rows; fp32 outputs are written straight
    from the accumulator layout.  Both come from the same fp32 values, so the bf16 output must equal the
    fp32 output rounded to bf16 (round to nearest even) element for element, and the LSE must be equal:
    an element the stage put in the wrong row or column fails."""
    say("bf16 out == rounded fp32 out", B, S, Hq, Hkv, d, "mode", mode)
    _, (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=34 + S)
    o32, l32 = _run_prefill(fa, qd, kd, vd, torch.float32, mode, sink=128, window=512)
    o16, l16 = _run_prefill(fa, qd, kd, vd, torch.bfloat16, mode, sink=128, window=512)
    assert torch.isfinite(o32).all()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)


# ------------------------------------------------------------- full-size layers
def _wave_rows(B, Hq, S, stride, seed):
    """(b, h, i) rows: for every batch and head, one seeded row in each `stride`-row segment (so every
    32-row wave segment of every unit is sampled when stride <= 32), plus the block-edge positions."""
    rng = np.random.default_rng(seed)
    rows = set()
    edges = [0, 1, 63, 64, 127, 128, 2047, 2048, 2049, S // 2, S - 65, S - 64, S - 2, S - 1]
    for b in range(B):
        for h in range(Hq):
            for i in edges:
                if 0 <= i < S:
                    rows.add((b, h, i))
            starts = np.arange(0, S, stride)
            offs = rng.integers(0, stride, len(starts))
            for i in np.minimum(starts + offs, S - 1):
                rows.add((b, h, int(i)))
    return np.array(sorted(rows), np.int64)


def _check_rows(o, lse, rows, ref, ref_lse, what, out_bf16):
    o_h = o.float().cpu().numpy()
    got = o_h[rows[:, 0], rows[:, 2], rows[:, 1]]
    check_close(got, ref, what, out_bf16=out_bf16)
    if lse is not None:
        l_h = lse.cpu().numpy()
        check_lse(l_h[rows[:, 0], rows[:, 1], rows[:, 2]], ref_lse, what + " lse")


def _assert_all_written(*ts):
    for t in ts:
        if t is not None:
            assert torch.isfinite(t).all(), "an output element was not written (NaN fill survived)"


@pytest.fixture(scope="module")
def llama_layer(fa):
    """One Llama-3.1-8B-shaped layer: batch 1, seq 8192, 32 query heads, 8 KV heads, head_dim 128, with the
    fp64 oracle for EVERY row (about 10 s on 16 host threads)."""
    B, S, Hq, Hkv, d = 1, 8192, 32, 8, 128
    say("llama layer S=8192: inputs and full oracle")
    qd = synth.torch_normal((B, S, Hq, d), 1002, torch.bfloat16)
    kd = synth.torch_normal((B, S, Hkv, d), 1003, torch.bfloat16)
    vd = synth.torch_normal((B, S, Hkv, d), 1004, torch.bfloat16)
    q, k, v = (dev_bits_to_host(x) for x in (qd, kd, vd))
    ref, ref_lse = oracle.attention(q, k, v, default_scale(d), causal=True)
    return dict(qd=qd, kd=kd, vd=vd, q=q, ref=ref, ref_lse=np.transpose(ref_lse, (0, 2, 1)))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_llama_layer_dense_s8192_every_row(fa, llama_layer, out_dtype):
    """Dense causal prefill at seq 8192 (persistent schedule), every output row against the oracle."""
    L = llama_layer
    say("llama layer S=8192 every row", out_dtype)
    o, lse = _run_prefill(fa, L["qd"], L["kd"], L["vd"], out_dtype, 0)
    _assert_all_written(o, lse)
    check_close(o.float().cpu().numpy(), L["ref"], "S=8192 dense", out_bf16=out_dtype == torch.bfloat16)
    check_lse(lse.cpu().numpy(), L["ref_lse"], "S=8192 dense lse")


def test_headline_routed_layer_s8192_every_row(fa, llama_layer):
    """The benchmarked instance: router on the layer's queries (head bias +8 on the dense index) -> device
    mode -> flux_attn_prefill_layers_routed with bf16 output, i.e. prefill_bf16_kernel<128, kRouted> on the
    persistent schedule.  Bit-equal to host-mode dispatch and to the plain dense call; every row against the
    oracle (bf16 output bound)."""
    L = llama_layer
    qd, kd, vd = L["qd"], L["kd"], L["vd"]
    B, S, Hq, d = qd.shape
    say("headline routed layer S=8192")
    w = synth.router_weights(1, Hq * d, 256, seed=1005)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w)
    b_head[0, 0] += 8.0
    modes = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    rp, ci = _csr_dev(fa, S, 128, 2048)
    fa.flux_route_layers([qd[0]], w_enc, b_enc, w_head, b_head, modes, None, pool_tokens=100)
    outs = []
    for routed in (True, False):
        o = torch.full((B, S, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
        if routed:
            fa.flux_attn_prefill_layers_routed(modes, [qd], [kd], [vd], [o], [lse], block=64, sink_tokens=128,
                                               window_tokens=2048, blk_row_ptr=rp, blk_col_idx=ci)
        else:
            fa.flux_attn_prefill_layers([0], [qd], [kd], [vd], [o], [lse], block=64, sink_tokens=128,
                                        window_tokens=2048, blk_row_ptr=rp, blk_col_idx=ci)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert int(modes.cpu()[0]) == fa.FLUX_MODE_DENSE
    (o_r, l_r), (o_h, l_h) = outs
    _assert_all_written(o_r, l_r)
    assert torch.equal(o_r, o_h) and torch.equal(l_r, l_h), "routed != host-mode dispatch"
    check_close(o_r.float().cpu().numpy(), L["ref"], "headline routed S=8192", out_bf16=True)
    check_lse(l_r.cpu().numpy(), L["ref_lse"], "headline routed S=8192 lse")


@pytest.mark.parametrize("B,S,Hq,Hkv,d,mode", [
    (2, 8200, 16, 16, 64, 0),     # MHA (odd group: the two wave groups take two query tiles), ragged tail
    (2, 8200, 16, 16, 64, 1),
    (1, 16384, 8, 4, 128, 0),     # groups of 2 query heads
    (1, 16384, 8, 4, 128, 1),
])
def test_persistent_schedule_shapes(fa, B, S, Hq, Hkv, d, mode):
    """Shapes with at least two units per compute unit run on the persistent schedule; cover both unit
    pairings and a ragged sequence end.  NaN-filled outputs must all be written; one row of every 32-row
    wave segment of every head (block-sparse) or of every 256 rows (dense) against the oracle."""
    seed = 1020 + S + Hq
    say("persistent schedule", B, S, Hq, Hkv, d, "mode", mode)
    qd = synth.torch_normal((B, S, Hq, d), seed, torch.bfloat16)
    kd = synth.torch_normal((B, S, Hkv, d), seed + 1, torch.bfloat16)
    vd = synth.torch_normal((B, S, Hkv, d), seed + 2, torch.bfloat16)
    o, lse = _run_prefill(fa, qd, kd, vd, torch.float32, mode)
    _assert_all_written(o, lse)
    rows = _wave_rows(B, Hq, S, 32 if mode else 256, seed)
    ref, ref_lse = oracle.attention(dev_bits_to_host(qd), dev_bits_to_host(kd), dev_bits_to_host(vd),
                                    default_scale(d), causal=True, sparse=bool(mode), block=64, sink_tokens=128,
                                    window_tokens=2048, rows=rows)
    _check_rows(o, lse, rows, ref, ref_lse, f"persistent S={S} mode {mode}", False)


def test_layer_sparse_s65536(fa):
    """Same layer at seq 65536, block-sparse: block 64, sink 128, window 2048 (32 blocks).  Every output
    written (NaN fill); one seeded row of every 32-row wave segment of every head (65,536 rows) against
    the oracle."""
    B, S, Hq, Hkv, d = 1, 65536, 32, 8, 128
    say("sparse layer S=65536")
    qd = synth.torch_normal((B, S, Hq, d), 1003, torch.bfloat16)
    kd = synth.torch_normal((B, S, Hkv, d), 1004, torch.bfloat16)
    vd = synth.torch_normal((B, S, Hkv, d), 1005, torch.bfloat16)
    o, lse = _run_prefill(fa, qd, kd, vd, torch.float32, 1)
    _assert_all_written(o, lse)
    o_a = torch.full_like(o, float("nan"))
    fa.flux_attn_prefill(qd, kd, vd, o_a, None, causal=1, mode=fa.FLUX_MODE_SPARSE, sink_tokens=128,
                         window_tokens=2048)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o), "arithmetic walk differs from the CSR walk"
    del o_a
    rows = _wave_rows(B, Hq, S, 32, 1003)
    ref, ref_lse = oracle.attention(dev_bits_to_host(qd), dev_bits_to_host(kd), dev_bits_to_host(vd),
                                    default_scale(d), causal=True, sparse=True, block=64, sink_tokens=128,
                                    window_tokens=2048, rows=rows)
    _check_rows(o, lse, rows, ref, ref_lse, "S=65536 sparse", False)
    del qd, kd, vd, o, lse
    torch.cuda.empty_cache()


def test_routed_stack_layers_s131072(fa):
    """Qwen3-8B-shaped stack at seq 131072: one dense and one sparse layer whose modes come from the router
    (head bias) and stay on the device, run by flux_attn_prefill_layers_routed with bf16 outputs and no CSR
    as in the 36-layer benchmark, and again by host-mode dispatch with the CSR: bit-equal, every element
    written (NaN fill), and
    rows against the oracle -- one row of every 32-row wave segment of every head for the sparse layer, of
    every 1024 rows for the dense one."""
    S, Hq, Hkv, d = 131072, 32, 8, 128
    say("routed stack S=131072")
    plan = np.array([0, 1], np.int32)
    qs, ks, vs = [], [], []
    for l in range(2):
        qs.append(synth.torch_normal((1, S, Hq, d), 1004 + 10 * l, torch.bfloat16))
        ks.append(synth.torch_normal((1, S, Hkv, d), 1005 + 10 * l, torch.bfloat16))
        vs.append(synth.torch_normal((1, S, Hkv, d), 1006 + 10 * l, torch.bfloat16))
    w = synth.router_weights(2, Hq * d, 256, seed=1006)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w)
    for l in range(2):
        b_head[l, int(plan[l])] += 8.0
    modes = torch.full((2,), -1, dtype=torch.int32, device=DEV)
    fa.flux_route_layers([x[0] for x in qs], w_enc, b_enc, w_head, b_head, modes, None, pool_tokens=100)
    rp, ci = _csr_dev(fa, S, 128, 2048)
    res = {}
    for routed in (True, False):
        os_ = [torch.full((1, S, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
        ls = [torch.full((1, Hq, S), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
        if routed:   # as benchmarked: no CSR, the sparse layer derives its blocks from (sink, window)
            fa.flux_attn_prefill_layers_routed(modes, qs, ks, vs, os_, ls, block=64, sink_tokens=128,
                                               window_tokens=2048)
        else:
            fa.flux_attn_prefill_layers(plan, qs, ks, vs, os_, ls, block=64, sink_tokens=128, window_tokens=2048,
                                        blk_row_ptr=rp, blk_col_idx=ci)
        res[routed] = (os_, ls)
    torch.cuda.synchronize()
    assert np.array_equal(modes.cpu().numpy(), plan)
    for l in range(2):
        o_r, l_r = res[True][0][l], res[True][1][l]
        _assert_all_written(o_r, l_r)
        assert torch.equal(o_r, res[False][0][l]) and torch.equal(l_r, res[False][1][l]), f"layer {l}"
    del res[False]
    for l in range(2):
        say("stack layer", l, "oracle rows")
        rows = _wave_rows(1, Hq, S, 32 if plan[l] else 1024, 77 + l)
        ref, ref_lse = oracle.attention(dev_bits_to_host(qs[l]), dev_bits_to_host(ks[l]), dev_bits_to_host(vs[l]),
                                        default_scale(d), causal=True, sparse=bool(plan[l]), block=64,
                                        sink_tokens=128, window_tokens=2048, rows=rows)
        _check_rows(res[True][0][l], res[True][1][l], rows, ref, ref_lse, f"stack layer {l}", True)
    del qs, ks, vs, res
    torch.cuda.empty_cache()


def test_routed_dispatch_reads_device_modes(fa):
    """flux_attn_prefill_layers_routed: the router's device output selects each layer's mode with
    no host round trip.  Layers forced dense / sparse through the router head bias; outputs must
    equal the host-dispatched run bit for bit and match the oracle."""
    B, S, Hq, Hkv, d = 1, 700, 8, 2, 128
    L = 3
    plan = np.array([1, 0, 1], np.int32)
    say("routed dispatch", plan)
    host = [synth.qkv_bf16(B, S, Hq, Hkv, d, seed=60 + l) for l in range(L)]
    qs, ks, vs = ([synth.torch_bf16_from_bits(h[i]) for h in host] for i in range(3))
    w = synth.router_weights(L, Hq * d, 64, seed=61)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w)
    for l in range(L):
        b_head[l, int(plan[l])] += 50.0
    modes = torch.empty(L, dtype=torch.int32, device=DEV)
    fa.flux_route_layers([x[0] for x in qs], w_enc, b_enc, w_head, b_head, modes, None, pool_tokens=100)
    rp, ci = _csr_dev(fa, S, 128, 256)
    o_r = [torch.empty((B, S, Hq, d), dtype=torch.float32, device=DEV) for _ in range(L)]
    l_r = [torch.empty((B, Hq, S), dtype=torch.float32, device=DEV) for _ in range(L)]
    fa.flux_attn_prefill_layers_routed(modes, qs, ks, vs, o_r, l_r, block=64, sink_tokens=128, window_tokens=256,
                                       blk_row_ptr=rp, blk_col_idx=ci)
    o_h = [torch.empty_like(x) for x in o_r]
    l_h = [torch.empty_like(x) for x in l_r]
    fa.flux_attn_prefill_layers(plan, qs, ks, vs, o_h, l_h, block=64, sink_tokens=128, window_tokens=256,
                                blk_row_ptr=rp, blk_col_idx=ci)
    torch.cuda.synchronize()
    assert np.array_equal(modes.cpu().numpy(), plan)
    for l in range(L):
        assert torch.equal(o_r[l], o_h[l]) and torch.equal(l_r[l], l_h[l]), f"layer {l}"
        q, k, v = host[l]
        ref, ref_lse = oracle.attention(q, k, v, default_scale(d), causal=True, sparse=bool(plan[l]), block=64,
                                        sink_tokens=128, window_tokens=256)
        check_close(o_r[l].cpu().numpy(), ref, f"routed layer {l}")
        check_lse(l_r[l].cpu().numpy(), np.transpose(ref_lse, (0, 2, 1)), f"routed layer {l} lse")


def test_routed_dispatch_fp32_inputs(fa):
    """The fp32-input kernel reads the device mode too."""
    B, S, H, d = 1, 384, 2, 64
    say("routed dispatch fp32")
    q, k, v = synth.qkv_f32(B, S, H, H, d, seed=62)
    qd, kd, vd = (torch.from_numpy(x).to(DEV) for x in (q, k, v))
    rp, ci = _csr_dev(fa, S, 128, 128)
    for mode in (0, 1):
        modes = torch.tensor([mode], dtype=torch.int32, device=DEV)
        o = torch.empty((B, S, H, d), dtype=torch.float32, device=DEV)
        fa.flux_attn_prefill_layers_routed(modes, [qd], [kd], [vd], [o], None, block=64, sink_tokens=128,
                                           window_tokens=128, blk_row_ptr=rp, blk_col_idx=ci)
        torch.cuda.synchronize()
        ref, _ = oracle.attention(q, k, v, 1.0 / 8, causal=True, sparse=bool(mode), block=64, sink_tokens=128,
                                  window_tokens=128)
        check_close(o.cpu().numpy(), ref, f"routed fp32 mode {mode}")


# ------------------------------------------------------------------ soft routing (training-time forward)
def test_soft_weights_match_oracle(fa):
    rng = np.random.default_rng(71)
    L = 40
    logits = rng.normal(size=(L, 2)).astype(np.float32) * 2
    u = rng.uniform(0.001, 0.999, size=(L, 2)).astype(np.float32)
    w = torch.empty((L, 2), dtype=torch.float32, device=DEV)
    for tau in (5.0, 1.0, 0.1):
        say("soft weights", tau)
        fa.flux_route_soft_weights(torch.from_numpy(logits).to(DEV), torch.from_numpy(u).to(DEV), tau, w)
        torch.cuda.synchronize()
        ref = oracle.soft_weights(logits.astype(np.float64), u.astype(np.float64), tau)
        assert np.abs(w.cpu().numpy() - ref).max() < 2e-5


@pytest.mark.parametrize("B,S,Hq,Hkv,d,sink,window,w0,csr", [
    (1, 700, 4, 2, 128, 128, 256, 0.3, True),
    (2, 333, 8, 2, 64, 64, 128, 0.85, True),
    (1, 512, 2, 2, 128, 128, 128, 1.0, True),
    (1, 512, 2, 2, 128, 128, 128, 0.0, True),
    (1, 650, 3, 1, 128, 0, 64, 0.4, False),      # odd group (4 query blocks per unit), no sink, 1-block window
    (1, 1000, 6, 2, 128, 64, 192, 0.7, False),   # odd group, 1 sink block, 3-block window, ragged end
    (1, 100, 2, 2, 64, 128, 128, 0.5, False),    # every row inside its sink: both outputs equal
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_soft_prefill_matches_oracle(fa, B, S, Hq, Hkv, d, sink, window, w0, csr, out_dtype):
    """The fused soft pass (sink and window blocks first, each row's block-sparse output taken where its
    window ends) against w0 * dense + (1 - w0) * block-sparse from the oracle; with and without the CSR."""
    say("soft prefill", B, S, Hq, Hkv, d, sink, window, w0, csr, out_dtype)
    (q, k, v), (qd, kd, vd) = bf16_tensors(B, S, Hq, Hkv, d, seed=72 + S)
    rp, ci = _csr_dev(fa, S, sink, window) if csr else (None, None)
    wd = torch.tensor([w0, 1.0 - w0], dtype=torch.float32, device=DEV)
    o = torch.full((B, S, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
    fa.flux_attn_prefill_soft(qd, kd, vd, o, wd, sink_tokens=sink, window_tokens=window, blk_row_ptr=rp,
                              blk_col_idx=ci)
    torch.cuda.synchronize()
    ref = oracle.attention_soft(q, k, v, default_scale(d), (w0, 1.0 - w0), block=64, sink_tokens=sink,
                                window_tokens=window)
    check_close(o.float().cpu().numpy(), ref, "soft prefill", out_bf16=out_dtype == torch.bfloat16)


def test_soft_prefill_router_pipeline_s8192_sampled(fa):
    """Router logits -> Gumbel-softmax weights -> soft-routed layer at the Llama layer shape."""
    B, S, Hq, Hkv, d = 1, 8192, 32, 8, 128
    say("soft prefill S=8192")
    qd = synth.torch_normal((B, S, Hq, d), 1040, torch.bfloat16)
    kd = synth.torch_normal((B, S, Hkv, d), 1041, torch.bfloat16)
    vd = synth.torch_normal((B, S, Hkv, d), 1042, torch.bfloat16)
    w = synth.router_weights(1, Hq * d, 64, seed=1043)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w)
    logits = torch.empty((1, 2), dtype=torch.float32, device=DEV)
    modes = torch.empty(1, dtype=torch.int32, device=DEV)
    fa.flux_route_layers([qd[0]], w_enc, b_enc, w_head, b_head, modes, logits, pool_tokens=100)
    u = torch.tensor([[0.3, 0.6]], dtype=torch.float32, device=DEV)
    weights = torch.empty((1, 2), dtype=torch.float32, device=DEV)
    fa.flux_route_soft_weights(logits, u, 0.5, weights)
    rp, ci = _csr_dev(fa, S, 128, 2048)
    o = torch.full((B, S, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    fa.flux_attn_prefill_soft(qd, kd, vd, o, weights[0], blk_row_ptr=rp, blk_col_idx=ci)
    torch.cuda.synchronize()
    _assert_all_written(o)
    ref_w = oracle.soft_weights(logits.cpu().numpy().astype(np.float64), u.cpu().numpy().astype(np.float64), 0.5)
    assert np.abs(weights.cpu().numpy() - ref_w).max() < 2e-5
    rows = _wave_rows(B, Hq, S, 32, 1044)
    ref = oracle.attention_soft(dev_bits_to_host(qd), dev_bits_to_host(kd), dev_bits_to_host(vd), default_scale(d),
                                ref_w[0], block=64, sink_tokens=128, window_tokens=2048, rows=rows)
    o_h = o.cpu().numpy()
    check_close(np.stack([o_h[b, i, h] for b, h, i in rows]), ref, "soft prefill S=8192")


# ------------------------------------------------------------- scores far from N(0,1): the rescale path
def _large_score_inputs(pattern, B, S, Hq, Hkv, d, seed):
    """'sharp': Q, K scaled by 4 (scores of std ~16), so a row's running max jumps past the kernel's
    lazy-rescale slack many times; 'rising': Q and K share a direction along which K grows with the key
    position (about 6 score units per 64-key tile), so every tile raises every row's max."""
    q, k, v = (synth.bf16_bits_to_f32(x) for x in synth.qkv_bf16(B, S, Hq, Hkv, d, seed))
    if pattern == "sharp":
        q, k = 4.0 * q, 4.0 * k
    else:
        u = np.full(d, 1.0 / np.sqrt(d), np.float32)
        pos = (np.arange(S, dtype=np.float32) / 64.0 * 6.0 * np.sqrt(d) / 6.0)[None, :, None, None]
        q = 0.5 * q + 6.0 * u
        k = 0.5 * k + pos * u
    q, k, v = (synth.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)) for x in (q, k, v))
    return (q, k, v), tuple(synth.torch_bf16_from_bits(x) for x in (q, k, v))


@pytest.mark.parametrize("pattern", ["sharp", "rising"])
@pytest.mark.parametrize("mode", [0, 1])
def test_large_scores_rescale_path(fa, pattern, mode):
    """Output and LSE against the oracle when the online softmax must rescale O on most tiles."""
    B, S, Hq, Hkv, d = 1, 700, 4, 2, 128
    say("large scores", pattern, "mode", mode)
    (q, k, v), (qd, kd, vd) = _large_score_inputs(pattern, B, S, Hq, Hkv, d, seed=2601)
    o, lse = _run_prefill(fa, qd, kd, vd, torch.float32, mode, sink=64, window=128)
    ref, ref_lse = oracle.attention(q, k, v, default_scale(d), causal=True, sparse=bool(mode), block=64,
                                    sink_tokens=64, window_tokens=128)
    check_close(o.cpu().numpy(), ref, f"large scores {pattern}")
    check_lse(lse.cpu().numpy(), np.transpose(ref_lse, (0, 2, 1)), f"large scores {pattern} lse")


# ------------------------------------------------------------- graph capture of the routed step
def test_routed_step_graph_replay(fa):
    """Router + routed prefill of two layers (one routed dense, one sparse by the head bias) captured in a
    HIP graph: each replay, with eager work between replays, reproduces the eager outputs and modes bit
    for bit (the router resets its own counters with a kernel; nothing in the step issues a memset)."""
    B, S, Hq, Hkv, d, L = 1, 700, 4, 2, 128, 2
    say("routed step graph replay")
    qs = [synth.torch_normal((B, S, Hq, d), 801 + l, torch.bfloat16) for l in range(L)]
    ks = [synth.torch_normal((B, S, Hkv, d), 811 + l, torch.bfloat16) for l in range(L)]
    vs = [synth.torch_normal((B, S, Hkv, d), 821 + l, torch.bfloat16) for l in range(L)]
    os_ = [torch.empty((B, S, Hq, d), dtype=torch.float32, device=DEV) for _ in range(L)]
    w = synth.router_weights(L, Hq * d, 64, seed=831)
    w[3][0, 0] += 8.0    # layer 0 dense
    w[3][1, 1] += 8.0    # layer 1 sparse
    wd = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in w]
    modes = torch.empty(L, dtype=torch.int32, device=DEV)
    ws = torch.empty(fa.flux_route_workspace_size(L, Hq, d, 64), dtype=torch.uint8, device=DEV)
    rp, ci = _csr_dev(fa, S, 128, 256)

    def step():
        fa.flux_route_layers([q[0] for q in qs], *wd, modes, None, workspace=ws, pool_tokens=100)
        fa.flux_attn_prefill_layers_routed(modes, qs, ks, vs, os_, None, sink_tokens=128, window_tokens=256,
                                           blk_row_ptr=rp, blk_col_idx=ci)

    step()
    torch.cuda.synchronize()
    assert modes.cpu().tolist() == [0, 1]
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
        modes.fill_(-1)
        for o in os_:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert modes.cpu().tolist() == [0, 1], f"replay {rep} modes"
        for l in range(L):
            assert torch.equal(os_[l], eager[l]), f"replay {rep} layer {l}"
    del g
