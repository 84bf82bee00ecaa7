"""GPU check of flux_attn_decode_noalloc: the decode entry point that allocates nothing and keeps its split
partials in the library's fixed per-device scratch.  Through the C ABI it must reproduce flux_attn_decode
(same kernels, caller workspace) bit for bit, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's partials), and both must meet the oracle bar."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import check_close, check_lse, default_scale, dev_bits_to_host, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def fa():
    import long_context_attention_tiled_amd as fa
    assert torch.cuda.is_available()
    return fa


def _pair(fa, qd, kd, vd, mode, sink, window, num_splits, out_dtype):
    B, Hq, d = qd.shape
    L, Hkv = kd.shape[1], kd.shape[2]
    outs = []
    for noalloc in (True, False):
        o = torch.full((B, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        if noalloc:
            fa.flux_attn_decode_noalloc(qd, kd, vd, o, lse, mode=mode, sink_tokens=sink, window_tokens=window,
                                        num_splits=num_splits)
        else:
            ws = torch.empty(fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, mode, 64, sink, window, num_splits),
                             dtype=torch.uint8, device=DEV)
            fa.flux_attn_decode(qd, kd, vd, o, lse, mode=mode, sink_tokens=sink, window_tokens=window,
                                num_splits=num_splits, workspace=ws)
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o_n, l_n), (o_w, l_w) = outs
    assert torch.isfinite(o_n).all() and torch.isfinite(l_n).all(), "unwritten output"
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), "no-allocation decode differs from flux_attn_decode"
    return o_n, l_n


def test_decode_noalloc_two_calls_matches_workspace_decode(fa):
    # call 1: batch 8, 65536-token caches, 32/8 heads, dense, automatic splits (32 per sequence and KV head)
    B, L, Hq, Hkv, d = 8, 65536, 32, 8, 128
    say("noalloc decode call 1", B, L, Hq, Hkv, d, "dense")
    qd = synth.torch_normal((B, Hq, d), 6001, torch.bfloat16)
    kd = synth.torch_normal((B, L, Hkv, d), 6002, torch.bfloat16)
    vd = synth.torch_normal((B, L, Hkv, d), 6003, torch.bfloat16)
    assert fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, 0, 64, 128, 2048, 0) <= fa.FLUX_DECODE_SCRATCH_BYTES
    o, lse = _pair(fa, qd, kd, vd, fa.FLUX_MODE_DENSE, 128, 2048, 0, torch.float32)
    rows = np.array([(b, h) for b in (0, 7) for h in range(Hq)], np.int64)
    q_h = dev_bits_to_host(qd)
    for b in (0, 7):
        ref, ref_lse = oracle.decode(np.ascontiguousarray(q_h[b:b + 1]), dev_bits_to_host(kd[b:b + 1]),
                                     dev_bits_to_host(vd[b:b + 1]), default_scale(d))
        check_close(o[b:b + 1].cpu().numpy(), ref, f"noalloc call 1 b {b}")
        check_lse(lse[b:b + 1].cpu().numpy(), ref_lse, f"noalloc call 1 lse b {b}")
    del qd, kd, vd, rows
    torch.cuda.empty_cache()

    # call 2, smaller: batch 2, ragged 3000-token caches, 8/2 heads, block-sparse, 5 forced splits, bf16 output
    B, L, Hq, Hkv, d = 2, 3000, 8, 2, 128
    say("noalloc decode call 2", B, L, Hq, Hkv, d, "sparse")
    q = synth.normal_bf16_bits((B, Hq, d), 6004, 0, synth.TENSOR_Q)
    k = synth.normal_bf16_bits((B, L, Hkv, d), 6004, 0, synth.TENSOR_K)
    v = synth.normal_bf16_bits((B, L, Hkv, d), 6004, 0, synth.TENSOR_V)
    qd, kd, vd = (synth.torch_bf16_from_bits(x) for x in (q, k, v))
    o, lse = _pair(fa, qd, kd, vd, fa.FLUX_MODE_SPARSE, 128, 512, 5, torch.bfloat16)
    ref, ref_lse = oracle.decode(q, k, v, default_scale(d), sparse=True, block=64, sink_tokens=128, window_tokens=512)
    check_close(o.float().cpu().numpy(), ref, "noalloc call 2", out_bf16=True)
    check_lse(lse.cpu().numpy(), ref_lse, "noalloc call 2 lse")


def test_decode_noalloc_rejects_partials_over_scratch(fa):
    """Partials larger than the scratch: FLUX_ERR_CAPACITY before any launch, outputs untouched."""
    B, L, Hq, Hkv, d = 64, 4096, 32, 8, 128
    need = fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, 0, 64, 128, 2048, 64)
    assert need > fa.FLUX_DECODE_SCRATCH_BYTES
    qd = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    kd = torch.zeros((B, L, Hkv, d), dtype=torch.bfloat16, device=DEV)
    o = torch.full((B, Hq, d), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FluxError) as e:
        fa.flux_attn_decode_noalloc(qd, kd, kd, o, None, num_splits=64)
    assert e.value.status == fa.FLUX_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
