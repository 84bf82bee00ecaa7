"""Host-side checks of the C ABI: symbols, block-mask builder, argument validation.

No GPU is needed: every call here either is host-only (the mask builder,
workspace sizing, status strings) or is rejected by validation before any HIP
call (the device pointers below are never dereferenced).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fa():
    import long_context_attention_tiled_amd as fa
    return fa


def test_library_exports_every_header_symbol(fa):
    with open(os.path.join(ROOT, "include", "flux_attn.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(flux_\w+)\s*\(", text, re.M))
    assert declared == set(fa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(fa.lib(), name), name
    assert fa.flux_version() == 100


def test_status_strings(fa):
    for code in range(6):
        s = fa.status_string(code)
        assert s.startswith("FLUX_")
    assert "unknown" in fa.status_string(99)


def _csr_to_bitmap(row_ptr, col_idx, nbk):
    nbq = len(row_ptr) - 1
    bm = np.zeros((nbq, nbk), np.uint8)
    for i in range(nbq):
        cols = col_idx[row_ptr[i]:row_ptr[i + 1]]
        assert np.all(np.diff(cols) > 0), "ascending, no duplicates"
        bm[i, cols] = 1
    return bm


MASK_CASES = [
    (512, 64, 128, 128), (512, 64, 128, 2048), (1000, 64, 128, 256), (97, 16, 0, 16), (64, 64, 128, 64),
    (65536, 64, 128, 2048), (131072, 64, 128, 2048), (8192, 64, 0, 64), (777, 32, 64, 96),
]


@pytest.mark.parametrize("S,block,sink,window", MASK_CASES)
def test_block_mask_bit_exact_vs_oracle(fa, S, block, sink, window):
    rp, ci = fa.flux_build_block_mask(S, S, block, sink, window, 1, fa.FLUX_MODE_SPARSE)
    nb = -(-S // block)
    assert rp[0] == 0 and rp[-1] == len(ci) and len(rp) == nb + 1
    bm = _csr_to_bitmap(rp, ci, nb)
    ref = oracle.block_mask(S, S, block, sink, window, causal=True, sparse=True)
    np.testing.assert_array_equal(bm, ref)


def test_block_mask_config_counts(fa):
    assert len(fa.flux_build_block_mask(512, 512, 64, 128, 128)[1]) == 26
    assert len(fa.flux_build_block_mask(65536, 65536, 64, 128, 2048)[1]) == 34255
    assert len(fa.flux_build_block_mask(131072, 131072, 64, 128, 2048)[1]) == 69071


@pytest.mark.parametrize("S,causal", [(1000, 1), (1000, 0), (64, 1), (65, 0)])
def test_dense_mask_bit_exact(fa, S, causal):
    rp, ci = fa.flux_build_block_mask(S, S, 64, 0, 0, causal, fa.FLUX_MODE_DENSE)
    nb = -(-S // 64)
    ref = oracle.block_mask(S, S, 64, 0, 0, causal=bool(causal), sparse=False)
    np.testing.assert_array_equal(_csr_to_bitmap(rp, ci, nb), ref)


def _mask_call(fa, S=512, block=64, sink=128, window=128, causal=1, mode=1, cap=None, want_arrays=True):
    nnz = ctypes.c_int64(-1)
    nb = -(-S // max(block, 1))
    rp = np.zeros(max(nb, 1) + 1, np.int32)
    cap = 10 ** 6 if cap is None else cap
    ci = np.zeros(max(cap, 1), np.int32)
    st = fa.lib().flux_build_block_mask(S, S, block, sink, window, causal, mode,
                                        rp.ctypes.data_as(ctypes.c_void_p) if want_arrays else None,
                                        ci.ctypes.data_as(ctypes.c_void_p) if want_arrays else None,
                                        cap if want_arrays else 0, ctypes.byref(nnz))
    return st, nnz.value


def test_block_mask_validation(fa):
    assert _mask_call(fa)[0] == fa.FLUX_OK
    assert _mask_call(fa, sink=100)[0] == fa.FLUX_ERR_INVALID_ARG       # sink not a multiple of block
    assert _mask_call(fa, window=100)[0] == fa.FLUX_ERR_INVALID_ARG     # window not a multiple of block
    assert _mask_call(fa, window=0)[0] == fa.FLUX_ERR_INVALID_ARG       # window < block in sparse mode
    assert _mask_call(fa, causal=0)[0] == fa.FLUX_ERR_INVALID_ARG       # sparse needs causal
    assert _mask_call(fa, mode=7)[0] == fa.FLUX_ERR_INVALID_ARG
    assert _mask_call(fa, block=0)[0] == fa.FLUX_ERR_INVALID_ARG
    assert _mask_call(fa, S=0)[0] == fa.FLUX_ERR_INVALID_ARG
    st, nnz = _mask_call(fa, cap=10)
    assert st == fa.FLUX_ERR_CAPACITY and nnz == 26
    st, nnz = _mask_call(fa, want_arrays=False)
    assert st == fa.FLUX_OK and nnz == 26
    assert "window" in fa.last_error_detail() or fa.last_error_detail() == ""


# ---------------------------------------------------------------- prefill validation
FAKE = 0x10000  # an aligned address that validation failures never dereference


def _prefill(fa, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, in_dtype=0, out_dtype=1, batch=1, seq=512, hq=4, hkv=2,
                d=128, scale=0.088, causal=1, mode=0, block=64, sink=128, window=128, rp=None, ci=None, nnz=0)
    args.update(kw)
    return fa.lib().flux_attn_prefill(args["q"], args["k"], args["v"], args["o"], args["lse"], args["in_dtype"],
                                      args["out_dtype"], args["batch"], args["seq"], args["hq"], args["hkv"],
                                      args["d"], args["scale"], args["causal"], args["mode"], args["block"],
                                      args["sink"], args["window"], args["rp"], args["ci"], args["nnz"], None)


def test_prefill_validation(fa):
    E, U = fa.FLUX_ERR_INVALID_ARG, fa.FLUX_ERR_UNSUPPORTED
    assert _prefill(fa, q=None) == E
    assert _prefill(fa, o=None) == E
    assert _prefill(fa, k=FAKE + 2) == E                    # misaligned
    assert _prefill(fa, lse=FAKE + 2) == E
    assert _prefill(fa, hq=6, hkv=4) == E                   # hq % hkv != 0
    assert _prefill(fa, hkv=0) == E
    assert _prefill(fa, seq=0) == E
    assert _prefill(fa, batch=0) == E
    assert _prefill(fa, scale=0.0) == E
    assert _prefill(fa, scale=float("inf")) == E
    assert _prefill(fa, scale=float("nan")) == E
    assert _prefill(fa, in_dtype=5) == E
    assert _prefill(fa, out_dtype=5) == E
    assert _prefill(fa, causal=2) == E
    assert _prefill(fa, mode=3) == E
    assert _prefill(fa, d=96) == U
    assert _prefill(fa, block=32) == U
    assert _prefill(fa, in_dtype=1, out_dtype=0) == U
    # sparse-mode rules
    assert _prefill(fa, mode=1, causal=0, rp=FAKE, ci=FAKE, nnz=26) == E
    assert _prefill(fa, mode=1, sink=100, rp=FAKE, ci=FAKE, nnz=26) == E
    assert _prefill(fa, mode=1, window=0, rp=FAKE, ci=FAKE, nnz=26) == E
    assert _prefill(fa, mode=1, window=96, rp=FAKE, ci=FAKE, nnz=26) == E
    assert _prefill(fa, mode=1, rp=None, ci=FAKE, nnz=26) == E
    assert _prefill(fa, mode=1, rp=FAKE, ci=FAKE, nnz=25) == E   # CSR does not match the pattern
    assert "blk_nnz" in fa.last_error_detail()


def test_prefill_layers_validation(fa):
    L = 2
    P = ctypes.POINTER(ctypes.c_void_p)
    ptrs = (ctypes.c_void_p * L)(FAKE, FAKE)
    pp = ctypes.cast(ptrs, P)
    modes = np.array([0, 7], np.int32)
    st = fa.lib().flux_attn_prefill_layers(L, modes.ctypes.data_as(ctypes.c_void_p), pp, pp, pp, pp, None, 0, 1, 1,
                                           512, 4, 2, 128, 0.088, 64, 128, 128, None, None, 0, None)
    assert st == fa.FLUX_ERR_INVALID_ARG and "layer 1" in fa.last_error_detail()
    st = fa.lib().flux_attn_prefill_layers(0, modes.ctypes.data_as(ctypes.c_void_p), pp, pp, pp, pp, None, 0, 1, 1,
                                           512, 4, 2, 128, 0.088, 64, 128, 128, None, None, 0, None)
    assert st == fa.FLUX_ERR_INVALID_ARG


def test_prefill_layers_routed_validation(fa):
    """Device-mode dispatch: every layer is checked as block-sparse (the CSR is required), the
    modes pointer must be present and aligned; all failures are reported before any launch."""
    L = 2
    P = ctypes.POINTER(ctypes.c_void_p)
    ptrs = (ctypes.c_void_p * L)(FAKE, FAKE)
    pp = ctypes.cast(ptrs, P)

    def call(n_layers=L, modes=FAKE, rp=FAKE, ci=FAKE, nnz=26, seq=512):
        return fa.lib().flux_attn_prefill_layers_routed(n_layers, modes, pp, pp, pp, pp, None, 0, 1, 1, seq, 4, 2,
                                                        128, 0.088, 64, 128, 128, rp, ci, nnz, None)
    E = fa.FLUX_ERR_INVALID_ARG
    assert call(n_layers=0) == E
    assert call(modes=None) == E
    assert call(modes=FAKE + 2) == E and "modes_device" in fa.last_error_detail()
    assert call(rp=None) == E and "layer 0" in fa.last_error_detail()
    assert call(nnz=25) == E and "blk_nnz" in fa.last_error_detail()


def test_window_cache_rows(fa):
    assert fa.flux_window_cache_rows(64, 128, 2048) == 2176
    assert fa.flux_window_cache_rows(64, 0, 64) == 64
    assert fa.flux_window_cache_rows(32, 128, 2048) == 0
    assert fa.flux_window_cache_rows(64, 100, 2048) == 0
    assert fa.flux_window_cache_rows(64, 128, 0) == 0


def _step(fa, **kw):
    args = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, out_dtype=1, batch=2, pos=100,
                rows=2176, layout=1, hq=8, hkv=2, d=128, scale=0.088, mode=1, block=64, sink=128, window=2048, ns=0,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return fa.lib().flux_decode_step(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["o"], a["lse"], a["out_dtype"],
                                     a["batch"], a["pos"], a["rows"], a["layout"], a["hq"], a["hkv"], a["d"],
                                     a["scale"], a["mode"], a["block"], a["sink"], a["window"], a["ns"], a["ws"],
                                     a["ws_bytes"], None)


def test_decode_step_validation(fa):
    E = fa.FLUX_ERR_INVALID_ARG
    assert _step(fa, kn=None) == E
    assert _step(fa, vn=FAKE + 4) == E                     # misaligned
    assert _step(fa, pos=-1) == E
    assert _step(fa, layout=2) == E
    assert _step(fa, mode=0) == E                          # the window cache holds sparse layers only
    assert _step(fa, rows=2175) == E and "2176" in fa.last_error_detail()
    assert _step(fa, layout=0, mode=0, rows=100, pos=100) == fa.FLUX_ERR_CAPACITY
    assert _step(fa, ws=None) == fa.FLUX_ERR_WORKSPACE
    assert _step(fa, ws_bytes=16) == fa.FLUX_ERR_WORKSPACE
    assert _step(fa, hq=6, hkv=4) == E                     # hq % hkv != 0
    assert _step(fa, hq=6) == fa.FLUX_ERR_UNSUPPORTED       # group of 3


def test_decode_step_layers_validation(fa):
    L = 2
    P = ctypes.POINTER(ctypes.c_void_p)
    ptrs = (ctypes.c_void_p * L)(FAKE, FAKE)
    pp = ctypes.cast(ptrs, P)

    def call(modes, dense_rows=4096, pos=100):
        m = np.array(modes, np.int32)
        return fa.lib().flux_decode_step_layers(L, m.ctypes.data_as(ctypes.c_void_p), pp, pp, pp, pp, pp, pp, None,
                                                1, 2, pos, dense_rows, 8, 2, 128, 0.088, 64, 128, 2048, FAKE, 1 << 30,
                                                None)
    assert call([0, 7]) == fa.FLUX_ERR_INVALID_ARG and "layer 1" in fa.last_error_detail()
    assert call([1, 0], dense_rows=50) == fa.FLUX_ERR_CAPACITY and "layer 1" in fa.last_error_detail()


def test_soft_routing_validation(fa):
    E = fa.FLUX_ERR_INVALID_ARG
    lib = fa.lib()
    assert lib.flux_route_soft_weights(None, FAKE, 1.0, 2, FAKE, None) == E
    assert lib.flux_route_soft_weights(FAKE, FAKE, 0.0, 2, FAKE, None) == E
    assert lib.flux_route_soft_weights(FAKE, FAKE, float("nan"), 2, FAKE, None) == E
    assert lib.flux_route_soft_weights(FAKE, FAKE, 1.0, 0, FAKE, None) == E
    assert fa.flux_prefill_soft_workspace_size(2, 100, 4, 64) == 2 * 100 * 4 * 64 * 4
    assert fa.flux_prefill_soft_workspace_size(0, 100, 4, 64) == 0

    def soft(**kw):
        a = dict(q=FAKE, o=FAKE + 4096, in_dtype=0, out_dtype=1, seq=512, rp=FAKE, ci=FAKE, nnz=26, w=FAKE,
                 ws=FAKE + 8192, ws_bytes=1 << 30)
        a.update(kw)
        return lib.flux_attn_prefill_soft(a["q"], FAKE, FAKE, a["o"], a["in_dtype"], a["out_dtype"], 1, a["seq"], 4,
                                          2, 128, 0.088, 64, 128, 128, a["rp"], a["ci"], a["nnz"], a["w"], a["ws"],
                                          a["ws_bytes"], None)
    assert soft(w=None) == E
    assert soft(in_dtype=1) == fa.FLUX_ERR_UNSUPPORTED
    assert soft(rp=None) == E                              # half a CSR
    assert soft(rp=None, ci=None, ws_bytes=100) == fa.FLUX_ERR_WORKSPACE   # no CSR: pattern from sink/window
    assert soft(rp=None, ci=None, seq=0) == E
    assert soft(nnz=25) == E
    assert soft(ws_bytes=100) == fa.FLUX_ERR_WORKSPACE
    assert soft(ws=FAKE + 4096) == E                       # aliases o
    assert soft(ws=FAKE + 4100) == E                       # misaligned workspace


def test_backward_workspace_size(fa):
    align = lambda x: (x + 255) // 256 * 256
    B, S, Hq, Hkv, d = 2, 1000, 8, 2, 128
    nqb = (S + 63) // 64
    stat = align(B * Hq * nqb * 128 * 4)

    def fp16_part(B, S):   # chunk maxima, exponents, fp16 copies of Q, K, V, dO
        q16, k16 = align(B * S * Hq * d * 2), align(B * S * Hkv * d * 2)
        return align(4 * B * Hkv * 128 * 4) + align(4 * B * Hkv * 4) + 2 * q16 + 2 * k16

    SP = fa.FLUX_MODE_SPARSE
    # dense: dK/dV units take a KV head's query heads in turn, no per-head buffers
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d) == stat + 256 + fp16_part(B, S)
    # block-sparse GQA: per-head buffers for the key pairs holding sink blocks (128 keys per pair)
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, SP, 64, 128) == \
        stat + 256 + 2 * align(B * 128 * Hq * d * 4) + fp16_part(B, S)
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, SP, 64, 192) == \
        stat + 256 + 2 * align(B * 256 * Hq * d * 4) + fp16_part(B, S)
    assert fa.flux_attn_backward_workspace_size(B, 100, Hq, Hkv, d, SP, 64, 192) == \
        align(B * Hq * 2 * 128 * 4) + 256 + 2 * align(B * 100 * Hq * d * 4) + fp16_part(B, 100)   # pairs clipped at seq
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, SP, 64, 0) == stat + 256 + fp16_part(B, S)   # no sink
    dense_mha = fa.flux_attn_backward_workspace_size(B, S, Hq, Hq, d)
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hq, d, SP, 64, 128) == dense_mha   # no grouping
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, 3, d) == 0                    # hq % hkv
    assert fa.flux_attn_backward_workspace_size(0, S, Hq, Hkv, d) == 0
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, SP, 64, 100) == 0     # sink not a block multiple
    assert fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, 5, 64, 0) == 0        # unknown mode


def test_backward_validation(fa):
    E, U = fa.FLUX_ERR_INVALID_ARG, fa.FLUX_ERR_UNSUPPORTED
    lib = fa.lib()

    def bwd(**kw):
        a = dict(q=FAKE, lse=FAKE, dq=FAKE + 4096, dk=FAKE + 8192, dv=FAKE + 12288, in_dtype=0, o_dtype=0, seq=512, hq=4, hkv=2,
                 d=128, scale=0.088, causal=1, mode=0, block=64, sink=128, window=128, ws=FAKE + 16384,
                 ws_bytes=1 << 30)
        a.update(kw)
        return lib.flux_attn_backward(a["q"], FAKE, FAKE, FAKE, FAKE, a["lse"], a["dq"], a["dk"], a["dv"],
                                      a["in_dtype"], a["o_dtype"], 1, a["seq"], a["hq"], a["hkv"], a["d"], a["scale"], a["causal"],
                                      a["mode"], a["block"], a["sink"], a["window"], a["ws"], a["ws_bytes"], None)
    assert bwd(q=None) == E
    assert bwd(lse=None) == E
    assert bwd(dq=FAKE + 4100) == E                        # misaligned
    assert bwd(lse=FAKE + 2) == E
    assert bwd(seq=0) == E
    assert bwd(hkv=3) == E
    assert bwd(scale=0.0) == E
    assert bwd(scale=float("inf")) == E
    assert bwd(in_dtype=7) == E
    assert bwd(causal=2) == E
    assert bwd(mode=1, causal=0) == E                      # sparse needs causal
    assert bwd(mode=1, sink=100) == E
    assert bwd(mode=1, window=0) == E
    assert bwd(o_dtype=2) == E
    assert bwd(d=96) == U
    assert bwd(block=32) == U
    assert bwd(ws_bytes=100) == fa.FLUX_ERR_WORKSPACE
    assert bwd(ws=None) == fa.FLUX_ERR_WORKSPACE
    assert bwd(ws=FAKE + 16388) == E                       # misaligned workspace
    assert bwd(dk=FAKE + 4096) == E                        # dq aliases dk
    assert "distinct" in fa.last_error_detail()


# ---------------------------------------------------------------- decode validation / workspace
def test_decode_workspace_size(fa):
    B, Hq, Hkv, L, d = 8, 32, 8, 262144, 128
    ws = fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, fa.FLUX_MODE_DENSE)
    assert ws > 0 and ws % 256 == 0
    # explicit split count: [B,Hq,n,d] + [B,Hq,n] floats, each part 256-aligned
    ws7 = fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, fa.FLUX_MODE_DENSE, num_splits=7)
    rows = B * Hq * 7
    align = lambda x: (x + 255) // 256 * 256
    assert ws7 == align(rows * d * 4) + align(rows * 4)
    assert fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, fa.FLUX_MODE_SPARSE, 64, 128, 2048) > 0
    assert fa.flux_decode_workspace_size(B, Hq, 5, L, d) == 0          # hq % hkv
    assert fa.flux_decode_workspace_size(B, Hq, Hkv, L, 96) == 0       # unsupported head_dim
    assert fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, fa.FLUX_MODE_SPARSE, 64, 100, 2048) == 0


def _decode(fa, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, in_dtype=0, out_dtype=1, batch=2, kv_len=4096, cap=0,
                hq=8, hkv=2, d=128, scale=0.088, mode=0, block=64, sink=128, window=2048, ns=0, ws=FAKE,
                ws_bytes=1 << 30)
    args.update(kw)
    return fa.lib().flux_attn_decode(args["q"], args["k"], args["v"], args["o"], args["lse"], args["in_dtype"],
                                     args["out_dtype"], args["batch"], args["kv_len"], args["cap"], args["hq"],
                                     args["hkv"], args["d"], args["scale"], args["mode"], args["block"],
                                     args["sink"], args["window"], args["ns"], args["ws"], args["ws_bytes"], None)


def test_decode_validation(fa):
    E, U, W = fa.FLUX_ERR_INVALID_ARG, fa.FLUX_ERR_UNSUPPORTED, fa.FLUX_ERR_WORKSPACE
    assert _decode(fa, q=None) == E
    assert _decode(fa, v=FAKE + 8) == E
    assert _decode(fa, hq=8, hkv=3) == E
    assert _decode(fa, hq=32, hkv=2) == U                   # group of 16 heads
    assert _decode(fa, kv_len=0) == E
    assert _decode(fa, cap=100) == E                        # capacity < kv_len
    assert _decode(fa, ns=-1) == E
    assert _decode(fa, scale=-1.0) == E
    assert _decode(fa, mode=1, window=0) == E
    assert _decode(fa, mode=1, sink=64 + 3) == E
    assert _decode(fa, d=80) == U
    assert _decode(fa, in_dtype=1) == U
    assert _decode(fa, ws=None) == W
    assert _decode(fa, ws_bytes=16) == W
    assert _decode(fa, ws=FAKE + 64) == E                   # workspace alignment


def _decode_noalloc(fa, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, in_dtype=0, out_dtype=1, batch=2, kv_len=4096, cap=0,
                hq=8, hkv=2, d=128, scale=0.088, mode=0, block=64, sink=128, window=2048, ns=0)
    args.update(kw)
    return fa.lib().flux_attn_decode_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                             args["in_dtype"], args["out_dtype"], args["batch"], args["kv_len"],
                                             args["cap"], args["hq"], args["hkv"], args["d"], args["scale"],
                                             args["mode"], args["block"], args["sink"], args["window"], args["ns"],
                                             None)


def test_decode_noalloc_validation(fa):
    """The no-allocation decode validates like flux_attn_decode, and rejects split partials larger than its
    fixed scratch (FLUX_DECODE_SCRATCH_BYTES) with FLUX_ERR_CAPACITY, all before its first HIP call."""
    E, U, C = fa.FLUX_ERR_INVALID_ARG, fa.FLUX_ERR_UNSUPPORTED, fa.FLUX_ERR_CAPACITY
    assert _decode_noalloc(fa, q=None) == E
    assert _decode_noalloc(fa, o=FAKE + 4) == E
    assert _decode_noalloc(fa, hq=8, hkv=3) == E
    assert _decode_noalloc(fa, hq=32, hkv=2) == U
    assert _decode_noalloc(fa, cap=100) == E
    assert _decode_noalloc(fa, scale=float("nan")) == E
    assert _decode_noalloc(fa, mode=1, window=0) == E
    assert _decode_noalloc(fa, d=80) == U
    assert _decode_noalloc(fa, in_dtype=1) == U
    # partials over the scratch: batch 64 x 32 heads x 64 splits x 129 floats
    big = dict(batch=64, hq=32, hkv=8, ns=64)
    need = fa.flux_decode_workspace_size(64, 32, 8, 4096, 128, 0, 64, 128, 2048, 64)
    assert need > fa.FLUX_DECODE_SCRATCH_BYTES
    assert _decode_noalloc(fa, **big) == C
    assert "scratch" in fa.last_error_detail()
    # the decode workload's shape (batch 8, 32/8 heads, 262144-token cache, automatic splits) fits
    assert fa.flux_decode_workspace_size(8, 32, 8, 262144, 128, 0, 64, 128, 2048, 0) <= fa.FLUX_DECODE_SCRATCH_BYTES


def test_decode_scratch_constant_matches_header(fa):
    with open(os.path.join(ROOT, "include", "flux_attn.h")) as f:
        m = re.search(r"#define FLUX_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FLUX_DECODE_SCRATCH_BYTES


def test_route_workspace_size(fa):
    align = lambda x: (x + 255) // 256 * 256
    assert fa.flux_route_workspace_size(36, 32, 128, 256) == align(36 * 4096 * 4) + align(36 * 256 * 4) + align(36 * 4)
    assert fa.flux_route_workspace_size(0, 32, 128, 256) == 0


def test_route_validation(fa):
    P = ctypes.POINTER(ctypes.c_void_p)
    ptrs = (ctypes.c_void_p * 2)(FAKE, None)
    pp = ctypes.cast(ptrs, P)
    lib = fa.lib()
    big = 1 << 30
    st = lib.flux_route_layers(pp, 2, 1000, 32, 128, 0, 100, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, big, None)
    assert st == fa.FLUX_ERR_INVALID_ARG and "q_layers[1]" in fa.last_error_detail()
    ptrs2 = (ctypes.c_void_p * 1)(FAKE)
    pp2 = ctypes.cast(ptrs2, P)
    call = lambda *a: lib.flux_route_layers(pp2, 1, *a, None)
    assert call(1000, 32, 128, 0, 100, None, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, big) == fa.FLUX_ERR_INVALID_ARG
    assert call(1000, 32, 128, 0, 0, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, big) == fa.FLUX_ERR_INVALID_ARG
    assert call(1000, 3, 3, 0, 100, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, big) == fa.FLUX_ERR_UNSUPPORTED
    assert call(1000, 32, 128, 2, 100, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, big) == fa.FLUX_ERR_INVALID_ARG
    assert call(1000, 32, 128, 0, 100, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, None, big) == fa.FLUX_ERR_WORKSPACE
    assert call(1000, 32, 128, 0, 100, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, 100) == fa.FLUX_ERR_WORKSPACE
    assert call(1000, 32, 128, 0, 100, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE + 16, big) == \
        fa.FLUX_ERR_INVALID_ARG


# ------------------------------------------------------------------ the Python binding's own checks
def test_binding_refuses_host_tensors(fa):
    """The C ABI cannot tell a host pointer from a device pointer; the binding refuses tensors that are
    not on a GPU before any pointer crosses it (the kernels would otherwise fault on them)."""
    import torch
    B, S, Hq, Hkv, d = 1, 64, 2, 1, 64
    q = torch.zeros((B, S, Hq, d), dtype=torch.bfloat16)
    k = torch.zeros((B, S, Hkv, d), dtype=torch.bfloat16)
    o = torch.zeros((B, S, Hq, d), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flux_attn_prefill(q, k, k, o)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flux_attn_decode(q[:, 0], k, k, o[:, 0])
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flux_attn_backward(q, k, k, o, q, torch.zeros((B, Hq, S)), o, o[:, :, :1].contiguous(),
                              o[:, :, :1].contiguous())
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flux_route_soft_weights(torch.zeros((1, 2)), torch.zeros((1, 2)), 1.0, torch.zeros((1, 2)))
    with pytest.raises(TypeError, match="torch.Tensor"):
        fa.flux_attn_prefill(np.zeros((B, S, Hq, d), np.float32), k, k, o)


def test_binding_shape_checks_order(fa):
    """Shape and rank errors are reported as such (ValueError) for malformed inputs."""
    import torch
    with pytest.raises(ValueError, match="batch, seq, heads, head_dim"):
        fa.flux_attn_prefill(torch.zeros((64, 2, 64)), torch.zeros((64, 2, 64)), torch.zeros((64, 2, 64)),
                             torch.zeros((64, 2, 64)))
    with pytest.raises(ValueError, match="one mode per layer"):
        fa.flux_attn_prefill_layers([0, 1], [torch.zeros((1, 64, 2, 64))], [None], [None], [None])
