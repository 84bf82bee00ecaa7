"""Helpers shared by the GPU parity tests (inputs, comparisons, sampled rows)."""
from __future__ import annotations

import math

import numpy as np

import synth

MAX_ABS = 1e-2    # parity bar: max-abs error vs the fp64 oracle (fp32 outputs)
MEAN_ABS = 1e-3   # parity bar: mean-abs error


def say(*a):
    print("[case]", *a, flush=True)


def dev_bits_to_host(t) -> np.ndarray:
    """Device bf16 tensor -> host uint16 bit pattern (exact)."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_tensors(B, S, Hq, Hkv, d, seed, layer=0):
    q, k, v = synth.qkv_bf16(B, S, Hq, Hkv, d, seed, layer)
    return (q, k, v), tuple(synth.torch_bf16_from_bits(x) for x in (q, k, v))


def check_close(gpu, ref, what, out_bf16=False):
    """Element-wise comparison to the oracle.  fp32 outputs: max-abs <= 1e-2, mean-abs <= 1e-3.
    bf16 outputs additionally allow half a bf16 ulp of the reference value (output rounding)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    if out_bf16:
        mag = np.maximum(np.abs(ref), 1e-30)
        half_ulp = 0.5 * np.exp2(np.floor(np.log2(mag)) - 7)
        bound = MAX_ABS + half_ulp
        bad = err > bound
        assert not bad.any(), f"{what}: {bad.sum()} elements over bf16 bound, max err {err.max():.3e}"
        assert err.mean() <= MEAN_ABS + np.mean(half_ulp), f"{what}: mean-abs {err.mean():.3e}"
    else:
        assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
        assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    return float(err.max()), float(err.mean())


def check_lse(gpu, ref, what, tol=1e-3):
    """Row log-sum-exp: the kernels accumulate the row sum in fp32 from unrounded
    probabilities, so max-abs 1e-3 (natural log) is well above their rounding."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    assert err.max() <= tol, f"{what}: lse max-abs {err.max():.3e}"


def sample_positions(S, n_random, seed):
    fixed = [0, 1, 2, 63, 64, 65, 127, 128, 129, 2047, 2048, 2049, S // 2, S - 65, S - 64, S - 2, S - 1]
    rnd = np.random.default_rng(seed).integers(0, S, n_random).tolist()
    return sorted({p for p in fixed + rnd if 0 <= p < S})


def sample_rows(B, Hq, S, n_random, seed):
    """(b, h, i) triples: every head at the fixed edge positions plus random (b, h, i)."""
    rng = np.random.default_rng(seed + 1)
    rows = []
    for i in sample_positions(S, 0, seed):
        for h in range(Hq):
            rows.append((int(rng.integers(0, B)), h, i))
    for _ in range(n_random):
        rows.append((int(rng.integers(0, B)), int(rng.integers(0, Hq)), int(rng.integers(0, S))))
    return np.array(sorted(set(rows)), np.int64)


def default_scale(d):
    return 1.0 / math.sqrt(d)
