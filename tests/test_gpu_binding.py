"""The Python binding's argument checks on GPU tensors: shapes, dtypes and CSR sizes that do not fit
are refused before any pointer reaches the C ABI (which takes plain pointers and sizes and would read
past a short buffer).  Nothing is launched."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def fa():
    import long_context_attention_tiled_amd as fa
    assert torch.cuda.is_available()
    return fa


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def test_prefill_shape_and_dtype_checks(fa):
    B, S, Hq, Hkv, d = 1, 128, 4, 2, 64
    q, k, o = _t(B, S, Hq, d), _t(B, S, Hkv, d), _t(B, S, Hq, d, dtype=torch.float32)
    with pytest.raises(ValueError, match="k has shape"):
        fa.flux_attn_prefill(q, _t(B, S - 64, Hkv, d), k, o)                 # K shorter than Q
    with pytest.raises(TypeError, match="v has dtype"):
        fa.flux_attn_prefill(q, k, _t(B, S, Hkv, d, dtype=torch.float32), o)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.flux_attn_prefill(q, k, k, o, _t(B, S, Hq, dtype=torch.float32))  # [B,S,Hq] instead of [B,Hq,S]
    with pytest.raises(ValueError, match="o has shape"):
        fa.flux_attn_prefill(q, k, k, _t(B, S, Hkv, d))
    rp, ci = fa.flux_build_block_mask(2 * S, 2 * S, 64, 64, 64, 1, fa.FLUX_MODE_SPARSE)   # built for 2S
    with pytest.raises(ValueError, match="blk_row_ptr has shape"):
        fa.flux_attn_prefill(q, k, k, o, mode=fa.FLUX_MODE_SPARSE, sink_tokens=64, window_tokens=64,
                             blk_row_ptr=torch.from_numpy(rp).to(DEV), blk_col_idx=torch.from_numpy(ci).to(DEV))


def test_decode_and_backward_checks(fa):
    B, L, Hq, Hkv, d = 2, 256, 4, 2, 64
    q, kc, o = _t(B, Hq, d), _t(B, L, Hkv, d), _t(B, Hq, d, dtype=torch.float32)
    with pytest.raises(ValueError, match="v_cache has shape"):
        fa.flux_attn_decode(q, kc, _t(B, L // 2, Hkv, d), o)
    with pytest.raises(TypeError, match="workspace must be a uint8"):
        fa.flux_attn_decode(q, kc, kc, o, workspace=_t(16, dtype=torch.float32))
    S = 128
    qf, kf = _t(1, S, Hq, d), _t(1, S, Hkv, d)
    of, lse = _t(1, S, Hq, d, dtype=torch.float32), _t(1, Hq, S, dtype=torch.float32)
    with pytest.raises(TypeError, match="dk has dtype"):
        fa.flux_attn_backward(qf, kf, kf, of, qf, lse, of, kf, _t(1, S, Hkv, d, dtype=torch.float32))
    with pytest.raises(ValueError, match="lse"):
        fa.flux_attn_backward(qf, kf, kf, of, qf, None, of, of, of)


def test_router_checks(fa):
    S, Hq, d, H = 256, 4, 64, 32
    q = _t(S, Hq, d)
    f32 = dict(dtype=torch.float32)
    w_enc, b_enc, w_head, b_head = _t(1, H, Hq * d, **f32), _t(1, H, **f32), _t(1, 2, H, **f32), _t(1, 2, **f32)
    modes = _t(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="w_enc has shape"):
        fa.flux_route_layers([q], _t(1, H, Hq * d // 2, **f32), b_enc, w_head, b_head, modes)
    with pytest.raises(TypeError, match="modes_out has dtype"):
        fa.flux_route_layers([q], w_enc, b_enc, w_head, b_head, _t(1, **f32))
