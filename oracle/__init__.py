"""fp64 CPU oracle for the tiled attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
and never imports it.  The arithmetic lives in ``flux_oracle.c`` (plain C,
double precision, two-pass max-subtracted softmax); this module only marshals
numpy arrays into it.

Every function here follows its C counterpart's definition; the citations are
in ``flux_oracle.c``.  Inputs are float32 arrays or bfloat16 bit patterns
(uint16 arrays); both widen to double exactly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

KIND_F32, KIND_BF16 = 0, 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: F401  (oracle/build.py)
        _b.build(verbose=False)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_attention_rows.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, i32, dbl, i32, i32, i32,
                                          i32, i32, vp, i64, i32, vp, vp]
    lib.oracle_attention_rows.restype = i32
    lib.oracle_attention_backward.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, dbl, i32, i32, i32, i32,
                                              i32, i32, vp, vp, vp]
    lib.oracle_attention_backward.restype = i32
    lib.oracle_attention_backward_keys.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, dbl, i32, i32,
                                                   i32, i32, i32, vp, i64, i32, vp, vp]
    lib.oracle_attention_backward_keys.restype = i32
    lib.oracle_soft_weights.argtypes = [vp, vp, dbl, i32, vp]
    lib.oracle_soft_weights.restype = i32
    lib.oracle_mix.argtypes = [vp, vp, dbl, dbl, i64, vp]
    lib.oracle_mix.restype = None
    lib.oracle_decode.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, dbl, i32, i32, i32, i32, vp, i64,
                                  i32, vp, vp]
    lib.oracle_decode.restype = i32
    lib.oracle_block_mask.argtypes = [i64, i64, i32, i32, i32, i32, i32, vp]
    lib.oracle_block_mask.restype = i64
    lib.oracle_count_pairs.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32]
    lib.oracle_count_pairs.restype = i64
    lib.oracle_route.argtypes = [vp, i32, i32, i64, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.oracle_route.restype = i32
    _lib = lib
    return lib


def _kind_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return KIND_F32
    if a.dtype == np.uint16:
        return KIND_BF16
    raise TypeError(f"oracle inputs must be float32 or bfloat16 bits (uint16), got {a.dtype}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def attention(q, k, v, scale, causal=True, sparse=False, block=64, sink_tokens=0, window_tokens=0,
              rows=None, n_threads=0):
    """Attention rows in fp64.

    q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d] (float32 or bf16 bits).  rows: int array [n,3] of
    (b, h, i) or None for all rows.  Returns (out, lse): out [B,Sq,Hq,d] (all rows) or
    [n,d]; lse [B,Sq,Hq] or [n].
    """
    q = np.ascontiguousarray(q); k = np.ascontiguousarray(k); v = np.ascontiguousarray(v)
    kind = _kind_of(q)
    assert _kind_of(k) == kind and _kind_of(v) == kind
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, dk = k.shape
    assert dk == d and v.shape == k.shape and k.shape[0] == B
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        out = np.empty((n, d), np.float64); lse = np.empty((n,), np.float64)
    else:
        n = B * Sq * Hq
        out = np.empty((B, Sq, Hq, d), np.float64); lse = np.empty((B, Sq, Hq), np.float64)
    rc = _load().oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), kind, B, Sq, Sk, Hq, Hkv, d, float(scale),
                                       int(causal), int(sparse), int(block), int(sink_tokens),
                                       int(window_tokens), _ptr(rows), n, int(n_threads), _ptr(out),
                                       _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attention_rows failed ({rc})")
    return out, lse


def decode(q, k_cache, v_cache, scale, sparse=False, block=64, sink_tokens=0, window_tokens=0,
           rows=None, n_threads=0):
    """Single-token decode at position L-1.  q [B,Hq,d], caches [B,L,Hkv,d].

    rows: int array [n,2] of (b, h) or None.  Returns (out, lse).
    """
    q = np.ascontiguousarray(q); k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    kind = _kind_of(q)
    B, Hq, d = q.shape
    _, L, Hkv, _ = k_cache.shape
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
        n = rows.shape[0]
        out = np.empty((n, d), np.float64); lse = np.empty((n,), np.float64)
    else:
        n = B * Hq
        out = np.empty((B, Hq, d), np.float64); lse = np.empty((B, Hq), np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), kind, B, L, Hq, Hkv, d, float(scale),
                               int(sparse), int(block), int(sink_tokens), int(window_tokens), _ptr(rows), n,
                               int(n_threads), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out, lse


def block_mask(seq_q, seq_k, block, sink_tokens, window_tokens, causal=True, sparse=True):
    """Dense bitmap [nbq, nbk] (uint8) of active block pairs."""
    nbq = -(-seq_q // block); nbk = -(-seq_k // block)
    bm = np.zeros((nbq, nbk), np.uint8)
    cnt = _load().oracle_block_mask(seq_q, seq_k, block, sink_tokens, window_tokens, int(causal), int(sparse),
                                    _ptr(bm))
    if cnt < 0:
        raise ValueError("oracle_block_mask: bad arguments")
    return bm


def count_pairs(seq_q, seq_k, causal=True, sparse=False, block=64, sink_tokens=0, window_tokens=0,
                n_threads=0):
    c = _load().oracle_count_pairs(seq_q, seq_k, int(causal), int(sparse), int(block), int(sink_tokens),
                                   int(window_tokens), int(n_threads))
    if c < 0:
        raise ValueError("oracle_count_pairs: bad arguments")
    return int(c)


def route(xq_layers, w_enc, b_enc, w_head, b_head, pool_tokens=100):
    """Router per layer.  xq_layers: list of [S,Hq,d] arrays (float32 or bf16 bits).

    Returns (pooled [L, Hq*d], logits [L,2], modes [L] int32).
    """
    xs = [np.ascontiguousarray(x) for x in xq_layers]
    kind = _kind_of(xs[0])
    S, Hq, d = xs[0].shape
    L = len(xs)
    hidden = w_enc.shape[1]
    assert w_enc.shape == (L, hidden, Hq * d) and b_enc.shape == (L, hidden)
    assert w_head.shape == (L, 2, hidden) and b_head.shape == (L, 2)
    w_enc = np.ascontiguousarray(w_enc, np.float32); b_enc = np.ascontiguousarray(b_enc, np.float32)
    w_head = np.ascontiguousarray(w_head, np.float32); b_head = np.ascontiguousarray(b_head, np.float32)
    ptrs = (ctypes.c_void_p * L)(*[x.ctypes.data for x in xs])
    pooled = np.empty((L, Hq * d), np.float64)
    logits = np.empty((L, 2), np.float64)
    modes = np.empty((L,), np.int32)
    rc = _load().oracle_route(ctypes.cast(ptrs, ctypes.c_void_p), kind, L, S, Hq, d, int(pool_tokens),
                              _ptr(w_enc), _ptr(b_enc), hidden, _ptr(w_head), _ptr(b_head), _ptr(pooled),
                              _ptr(logits), _ptr(modes))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return pooled, logits, modes


def soft_weights(logits, uniforms, tau):
    """Gumbel-softmax routing weights [L,2] from logits [L,2] and uniforms [L,2] in (0,1)."""
    logits = np.ascontiguousarray(logits, np.float64)
    uniforms = np.ascontiguousarray(uniforms, np.float64)
    L = logits.shape[0]
    assert logits.shape == (L, 2) and uniforms.shape == (L, 2)
    w = np.empty((L, 2), np.float64)
    if _load().oracle_soft_weights(_ptr(logits), _ptr(uniforms), float(tau), L, _ptr(w)) != 0:
        raise ValueError("oracle_soft_weights: bad argument")
    return w


def attention_soft(q, k, v, scale, weights, block=64, sink_tokens=0, window_tokens=0, rows=None, n_threads=0):
    """Soft-routed layer output: weights[0] * full causal attention + weights[1] * block-sparse attention."""
    o_full, _ = attention(q, k, v, scale, causal=True, sparse=False, rows=rows, n_threads=n_threads)
    o_sparse, _ = attention(q, k, v, scale, causal=True, sparse=True, block=block, sink_tokens=sink_tokens,
                            window_tokens=window_tokens, rows=rows, n_threads=n_threads)
    o_full = np.ascontiguousarray(o_full, np.float64)
    o_sparse = np.ascontiguousarray(o_sparse, np.float64)
    out = np.empty_like(o_full)
    _load().oracle_mix(_ptr(o_full), _ptr(o_sparse), float(weights[0]), float(weights[1]), o_full.size, _ptr(out))
    return out


def attention_backward(q, k, v, d_o, scale, causal=True, sparse=False, block=64, sink_tokens=0, window_tokens=0,
                       n_threads=0):
    """Gradients (dq [B,S,Hq,d], dk, dv [B,S,Hkv,d], float64) of O = attention(q, k, v) for output gradient d_o."""
    q, k, v, d_o = (np.ascontiguousarray(x) for x in (q, k, v, d_o))
    kind = _kind_of(q)
    assert _kind_of(k) == kind and _kind_of(v) == kind and _kind_of(d_o) == kind
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    dq = np.empty((B, S, Hq, d), np.float64)
    dk = np.empty((B, S, Hkv, d), np.float64)
    dv = np.empty((B, S, Hkv, d), np.float64)
    rc = _load().oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(d_o), kind, B, S, Hq, Hkv, d, float(scale),
                                           int(causal), int(sparse), int(block), int(sink_tokens), int(window_tokens),
                                           int(n_threads), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError(f"oracle_attention_backward failed ({rc})")
    return dq, dk, dv


def attention_backward_keys(q, k, v, d_o, scale, keys, causal=True, sparse=False, block=64, sink_tokens=0,
                            window_tokens=0, n_threads=0):
    """dK, dV ([n, d] float64 each) of the requested keys only: keys is an int array [n, 3] of
    (b, kv head g, key position j).  Same gradients as attention_backward at those rows."""
    q, k, v, d_o = (np.ascontiguousarray(x) for x in (q, k, v, d_o))
    kind = _kind_of(q)
    assert _kind_of(k) == kind and _kind_of(v) == kind and _kind_of(d_o) == kind
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    keys = np.ascontiguousarray(np.asarray(keys, dtype=np.int64).reshape(-1, 3))
    n = keys.shape[0]
    dk = np.empty((n, d), np.float64)
    dv = np.empty((n, d), np.float64)
    rc = _load().oracle_attention_backward_keys(_ptr(q), _ptr(k), _ptr(v), _ptr(d_o), kind, B, S, Hq, Hkv, d,
                                                float(scale), int(causal), int(sparse), int(block),
                                                int(sink_tokens), int(window_tokens), _ptr(keys), n,
                                                int(n_threads), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError(f"oracle_attention_backward_keys failed ({rc})")
    return dk, dv
