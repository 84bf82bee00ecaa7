"""Benchmark of the tiled-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs LIST] [--no-cpu-baseline]

Headline workload (one step): a Qwen3-8B-shaped 36-layer attention stack prefill
at seq 131072 (batch 1, 32 query heads, 8 KV heads, head_dim 128, bf16, per-layer
Q/K/V iid N(0,1)).  The layer router reads every layer's queries (first/last 100
tokens -> MLP -> argmax) and leaves the 36 modes on the device; each layer's
routed prefill kernel reads its own mode and runs dense causal attention or
64x64 block-sparse attention (sink 128 tokens, causal window 2048 tokens).  The
seeded plan (12 dense layers, 24 sparse) is encoded in the router's head bias, so
the router's argmax reproduces it while all router arithmetic still runs.
`value` = useful prefill TFLOP/s (4*B*Hq*d per allowed query-key pair) of the
whole step.  The same 36 layers run all dense beside it, for the ratio the
Flux Attention pages quote as "up to 2.8x prefill at 256K context" (hardware not
stated there).

The roofline object is for the dominant kernel, the routed prefill kernel (every
layer's launch), timed with HIP events on the stream it runs on, with the dense
and sparse launches also given separately.  cpu_baseline times the fp64 CPU
oracle on a bounded sample of the same workload (rank 0, N=1 only), extrapolated
to the whole stack by allowed-pair counts, plus oracle samples of the other
configurations.

Secondary legs (same JSON line, "legs"): the routed Llama-3.1-8B layer at seq
8192 (router + dense-causal prefill), block-sparse prefill at seq 65536, GQA
decode over a 262144-token bf16 cache (dense and sparse; HBM GB/s and tok/s), the
routed decode loop, soft-routed prefill, the attention backward (seq 8192 dense,
seq 65536 sparse) and device ceilings.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "prefill useful TFLOP/s + decode HBM GB/s (tok/s), % of roofline, 1 MI355X"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def causal_pairs(S: int) -> int:
    return S * (S + 1) // 2


def csr_pairs(row_ptr, col_idx, S: int, block: int = 64) -> int:
    """Allowed (query, key) pairs of a causal block mask: full off-diagonal blocks, triangular diagonal."""
    total = 0
    for I in range(len(row_ptr) - 1):
        qn = min(S, (I + 1) * block) - I * block
        for J in col_idx[row_ptr[I]:row_ptr[I + 1]]:
            kn = min(S, (int(J) + 1) * block) - int(J) * block
            total += qn * (qn + 1) // 2 if J == I else qn * kn
    return total


class KernelTimer:
    """HIP events around each launch on the current stream; mean duration in ms."""

    def __init__(self):
        self.pairs = []

    def record(self, fn):
        import torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs])) if self.pairs else float("nan")

    def pct_ms(self):
        """(p10, median, p90) of the recorded launch durations."""
        d = np.array([s.elapsed_time(e) for s, e in self.pairs])
        return tuple(round(float(np.percentile(d, q)), 4) for q in (10, 50, 90))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_dense_causal_s8192_traffic.txt")
STACK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_routed_stack_s131072_traffic.txt")
PREFILL_SRCS = [os.path.join(ROOT, "long_context_attention_tiled_amd", "csrc", f)
                for f in ("prefill_bf16.hip", "tile_common.h")]


def prefill_source_hash() -> str:
    """sha256 over the prefill kernel's sources (kernel file, then its tile helper header)."""
    import hashlib
    h = hashlib.sha256()
    for f in PREFILL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of a prefill kernel from a committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the summary was taken on another
    version of the kernel source."""
    try:
        kv = {}
        for line in open(path):
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
        if kv.get("prefill_source_sha256") != prefill_source_hash():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def time_steps(step, steps, warmup, warm_ms=100.0):
    """Wall-clock ms per call over `steps` calls, after `warmup` calls and then more until `warm_ms` of
    warm-up have passed (kernel times settle over the first tens of ms on a freshly busy device)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def call_percentiles(step, reps):
    """(p10, median, p90) in ms of single calls, each bracketed by HIP events on the current stream."""
    import torch
    t = KernelTimer()
    for _ in range(reps):
        t.record(step)
    torch.cuda.synchronize()
    return t.pct_ms()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="layer8k,sparse,decode,decode_loop,soft,backward,peaks",
                    help="comma list of secondary legs: layer8k, sparse, dense64k, decode, decode_loop, soft, backward, "
                         "peaks (or 'none')")
    ap.add_argument("--no-legs", dest="legs", action="store_const", const="none")
    ap.add_argument("--no-headline", dest="headline", action="store_false", default=True,
                    help="skip the headline step (profiling a single leg)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run one plain device-to-device copy of MIB MiB (HBM counter calibration)")
    ap.add_argument("--sustain", nargs=2, metavar=("DATA", "SECONDS"), default=None,
                    help="only run the seq-65536 dense-causal prefill back to back for SECONDS with DATA = randn "
                         "(N(0,1) inputs) or const (constant inputs), for reading clocks with rocm-smi meanwhile")
    ap.add_argument("--dense-steps", type=int, default=2,
                    help="timed steps of the all-dense 36-layer comparison (0 skips it)")
    ap.add_argument("--steps-leg", type=int, default=20, help="timed repetitions per secondary leg")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false", default=True)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the kernels run on one "
              "GPU's share; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_attention_tiled_amd as fa
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n}), flush=True)
        return
    if args.sustain:
        run_sustain(fa, synth, torch, args.sustain[0], float(args.sustain[1]))
        return
    legs_sel = set() if args.legs == "none" else set(x for x in args.legs.split(",") if x)
    result = {}
    if args.headline:
        result = headline(args, fa, synth, torch, dev)
    legs = run_legs(fa, synth, torch, dev, legs_sel, args.steps_leg, args.warmup)
    if legs:
        result["legs"] = legs
        if "decode_dense_L262144" in legs:
            dd = legs["decode_dense_L262144"]
            result["decode"] = {"GB/s": dd["GB/s"], "tok/s": dd["tok/s"], "frac_hbm": dd["frac"]}
    if args.cpu_baseline and args.headline:
        result["cpu_baseline"] = cpu_baseline(synth, result.pop("_oracle_inputs"))
    result.pop("_oracle_inputs", None)
    print(json.dumps(result), flush=True)


def run_sustain(fa, synth, torch, data, seconds):
    """The seq-65536 dense-causal prefill (32/8 heads, d 128) back to back for `seconds`; N(0,1) or constant
    inputs.  Prints the mean time per call (the clock the chip settles at depends on the data)."""
    B, S, Hq, Hkv, d = 1, 65536, 32, 8, 128
    q = synth.torch_normal((B, S, Hq, d), 1102, torch.bfloat16)
    k = synth.torch_normal((B, S, Hkv, d), 1103, torch.bfloat16)
    v = synth.torch_normal((B, S, Hkv, d), 1104, torch.bfloat16)
    if data == "const":
        q.fill_(0.01)
        k.fill_(0.02)
        v.fill_(0.5)
    o = torch.empty_like(q)
    log(f"sustained prefill, {data} inputs, {seconds} s")
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        fa.flux_attn_prefill(q, k, v, o, None, causal=1, mode=fa.FLUX_MODE_DENSE)
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(json.dumps({"sustain": data, "calls": n, "seconds": round(dt, 2), "ms_per_call": round(dt / n * 1e3, 3)}),
          flush=True)


def host_bits(t) -> np.ndarray:
    """Device bf16 tensor -> host uint16 bit pattern (exact copy)."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sparse_row_pairs(i: int, block: int = 64, sink: int = 128, window: int = 2048) -> int:
    """Keys the block-sparse causal rule allows to query position i: the row's window blocks up to i, plus the
    sink keys before the window."""
    w0 = max(0, (i // block - window // block + 1) * block)
    return (i - w0 + 1) + min((sink // block) * block, w0)


def headline(args, fa, synth, torch, dev):

    # ---------------------------------------------------------------- headline: 36-layer routed stack, S=131072
    L, S, Hq, Hkv, d = 36, 131072, 32, 8, 128
    sink, window = 128, 2048
    log("generating headline inputs (36 layers, seq 131072)")
    plan = synth.layer_mode_draw(L, 12, seed=1004)
    qs = [synth.torch_normal((1, S, Hq, d), 2000 + 3 * l, torch.bfloat16) for l in range(L)]
    ks = [synth.torch_normal((1, S, Hkv, d), 2001 + 3 * l, torch.bfloat16) for l in range(L)]
    vs = [synth.torch_normal((1, S, Hkv, d), 2002 + 3 * l, torch.bfloat16) for l in range(L)]
    o = torch.empty((1, S, Hq, d), dtype=torch.bfloat16, device=dev)   # one output buffer reused by every layer
    w = synth.router_weights(L, Hq * d, 256, seed=1006)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in w)
    for l in range(L):
        b_head[l, int(plan[l])] += 8.0   # the seeded plan, reproduced by the router's own argmax
    rp, ci = fa.flux_build_block_mask(S, S, 64, sink, window, 1, fa.FLUX_MODE_SPARSE)
    rpd, cid = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
    modes_dev = torch.empty(L, dtype=torch.int32, device=dev)
    route_ws = torch.empty(fa.flux_route_workspace_size(L, Hq, d, 256), dtype=torch.uint8, device=dev)
    flops_dense = 4.0 * Hq * d * causal_pairs(S)
    flops_sparse = 4.0 * Hq * d * csr_pairs(rp, ci, S)
    layer_flops = [flops_dense if plan[l] == 0 else flops_sparse for l in range(L)]
    useful = float(sum(layer_flops))
    useful_all_dense = L * flops_dense
    algo_bytes = 2 * S * (2 * Hq + 2 * Hkv) * d   # per layer launch: Q, K, V read once and O written once, bf16
    timers = [KernelTimer() for _ in range(L)]

    def layer_call(l):
        # no CSR: a sparse layer's kernel derives its key blocks from (sink, window)
        fa.flux_attn_prefill_layers_routed(modes_dev[l:l + 1], [qs[l]], [ks[l]], [vs[l]], [o], None, block=64,
                                           sink_tokens=sink, window_tokens=window)

    def step(record=False):
        # router -> 36 device modes -> each layer's prefill kernel reads its own mode: no host round trip
        fa.flux_route_layers([x[0] for x in qs], w_enc, b_enc, w_head, b_head, modes_dev, None, workspace=route_ws,
                             pool_tokens=100)
        for l in range(L):
            if record:
                timers[l].record(lambda l=l: layer_call(l))
            else:
                layer_call(l)

    log("timing headline")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    assert np.array_equal(modes_dev.cpu().numpy(), plan), "router modes differ from the plan"
    layer_ms = [t.mean_ms() for t in timers]
    dense_ms = float(np.mean([layer_ms[l] for l in range(L) if plan[l] == 0]))
    sparse_ms = float(np.mean([layer_ms[l] for l in range(L) if plan[l] == 1]))
    kern_ms_total = float(np.sum(layer_ms))
    achieved = useful / (kern_ms_total * 1e-3) / 1e12
    value = useful / (ms_per_step * 1e-3) / 1e12

    # the same 36 layers, every one dense causal (host-mode dispatch): the pages' "versus full attention"
    dense_cmp = None
    if args.dense_steps > 0:
        log("timing the all-dense stack")
        all_dense = lambda: fa.flux_attn_prefill_layers(np.zeros(L, np.int32), qs, ks, vs, [o] * L, None, block=64,
                                                        sink_tokens=sink, window_tokens=window, blk_row_ptr=rpd,
                                                        blk_col_idx=cid)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.dense_steps):
            all_dense()
        torch.cuda.synchronize()
        ms_dense = (time.perf_counter() - t0) * 1e3 / args.dense_steps
        dense_cmp = {"routed_ms_per_step": round(ms_per_step, 2), "all_dense_ms_per_step": round(ms_dense, 2),
                     "all_dense_TFLOP/s": round(useful_all_dense / ms_dense / 1e9, 2),
                     "speedup": round(ms_dense / ms_per_step, 3),
                     "useful_flop_ratio": round(useful_all_dense / useful, 3), "steps": args.dense_steps,
                     "pages_context": "Flux Attention page (aitrends.kr), speed paragraph: up to 2.8x prefill and "
                                      "2.0x decode speedup versus full attention at 256K context; hardware not "
                                      "stated there"}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: per-layer iid N(0,1) Q/K/V rounded to bf16; seeded random router weights whose head "
                "bias encodes a seeded 12-dense / 24-sparse plan",
        "config": {"workload": "qwen3-8b-shaped 36-layer routed attention stack prefill (router + 12 dense-causal "
                               "+ 24 block-sparse layers)",
                   "batch": 1, "seq_len": S, "layers": L, "dense_layers": int((plan == 0).sum()), "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "block": 64, "sink_tokens": sink, "window_tokens": window,
                   "out_dtype": "bf16", "useful_flops_per_step": useful, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(STACK_TRAFFIC_FILE),
                     "algorithmic_bytes": algo_bytes,
                     "kernel": "prefill_bf16_kernel<128, routed, bf16 out>: all 36 layer launches of a step",
                     "kernel_ms_mean": round(kern_ms_total / L, 4),
                     "useful_flops_per_launch_mean": useful / L,
                     "dense_layer": {"ms": round(dense_ms, 3), "TFLOP/s": round(flops_dense / dense_ms / 1e9, 2),
                                     "frac": round(flops_dense / dense_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                     "useful_flops": flops_dense},
                     "sparse_layer": {"ms": round(sparse_ms, 3), "TFLOP/s": round(flops_sparse / sparse_ms / 1e9, 2),
                                      "frac": round(flops_sparse / sparse_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                      "useful_flops": flops_sparse, "nnz_blocks": int(len(ci))}},
    }
    if dense_cmp:
        result["vs_all_dense"] = dense_cmp
    # the oracle baseline samples one dense and one sparse layer of this stack: keep their bits on the host
    ld, ls_ = int(np.argmax(plan == 0)), int(np.argmax(plan == 1))
    result["_oracle_inputs"] = {"plan": plan, "flops_dense": flops_dense, "flops_sparse": flops_sparse,
                                "useful": useful,
                                "dense": tuple(host_bits(x[ld]) for x in (qs, ks, vs)),
                                "sparse": tuple(host_bits(x[ls_]) for x in (qs, ks, vs))}
    del qs, ks, vs, o
    torch.cuda.empty_cache()
    return result


def run_layer8k(fa, synth, torch, dev, reps, warmup):
    """The routed Llama-3.1-8B layer at seq 8192 (batch 1, 32/8 heads, head_dim 128, bf16): router on the layer's
    queries -> device mode (the head bias selects dense causal, the workload's mode) -> routed prefill kernel."""
    B, S, Hq, Hkv, d = 1, 8192, 32, 8, 128
    log("leg: routed layer S=8192")
    q = synth.torch_normal((B, S, Hq, d), 1002, torch.bfloat16)
    k = synth.torch_normal((B, S, Hkv, d), 1003, torch.bfloat16)
    v = synth.torch_normal((B, S, Hkv, d), 1004, torch.bfloat16)
    o = torch.empty((B, S, Hq, d), dtype=torch.bfloat16, device=dev)
    w = synth.router_weights(1, Hq * d, 256, seed=1005)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in w)
    b_head[0, 0] += 8.0
    modes_dev = torch.empty(1, dtype=torch.int32, device=dev)
    route_ws = torch.empty(fa.flux_route_workspace_size(1, Hq, d, 256), dtype=torch.uint8, device=dev)
    timer = KernelTimer()
    useful = 4.0 * B * Hq * d * causal_pairs(S)

    def step(record=False):
        fa.flux_route_layers([q[0]], w_enc, b_enc, w_head, b_head, modes_dev, None, workspace=route_ws,
                             pool_tokens=100)
        call = lambda: fa.flux_attn_prefill_layers_routed(modes_dev, [q], [k], [v], [o], None, block=64,
                                                          sink_tokens=128, window_tokens=2048)
        if record:
            timer.record(call)
        else:
            call()

    for _ in range(max(warmup, 5)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = max(reps, 20)
    for _ in range(n):
        step(record=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    assert int(modes_dev.cpu()[0]) == fa.FLUX_MODE_DENSE
    kern_ms = timer.mean_ms()
    res = {"ms_per_step": round(ms, 4), "step_TFLOP/s": round(useful / ms / 1e9, 2),
           "kernel_ms": round(kern_ms, 4), "kernel_ms_p10_p50_p90": timer.pct_ms(),
           "TFLOP/s": round(useful / kern_ms / 1e9, 2), "frac": round(useful / kern_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "useful_flops": useful, "traffic": measured_traffic(TRAFFIC_FILE),
           "algorithmic_bytes": 2 * B * S * (2 * Hq + 2 * Hkv) * d}
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def run_legs(fa, synth, torch, dev, sel, reps, warmup):
    legs = {}
    if "layer8k" in sel:
        legs["routed_layer_s8192"] = run_layer8k(fa, synth, torch, dev, reps, warmup)
    if {"sparse", "dense64k"} & sel:
        # ---- block-sparse prefill, seq 65536 (and optionally dense at the same length)
        B, S, Hq, Hkv, d = 1, 65536, 32, 8, 128
        log("leg: prefill S=65536")
        q = synth.torch_normal((B, S, Hq, d), 1102, torch.bfloat16)
        k = synth.torch_normal((B, S, Hkv, d), 1103, torch.bfloat16)
        v = synth.torch_normal((B, S, Hkv, d), 1104, torch.bfloat16)
        o = torch.empty((B, S, Hq, d), dtype=torch.bfloat16, device=dev)
        rp, ci = fa.flux_build_block_mask(S, S, 64, 128, 2048, 1, fa.FLUX_MODE_SPARSE)
        rpd, cid = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
        if "sparse" in sel:
            useful = 4.0 * B * Hq * d * csr_pairs(rp, ci, S)
            # key blocks derived from (sink, window) in the kernel; the CSR walk timed beside it
            call = lambda: fa.flux_attn_prefill(q, k, v, o, None, causal=1, mode=fa.FLUX_MODE_SPARSE,
                                                sink_tokens=128, window_tokens=2048)
            call_csr = lambda: fa.flux_attn_prefill(q, k, v, o, None, causal=1, mode=fa.FLUX_MODE_SPARSE,
                                                    sink_tokens=128, window_tokens=2048, blk_row_ptr=rpd,
                                                    blk_col_idx=cid)
            ms = time_steps(call, reps, 3)
            ms_csr = time_steps(call_csr, reps, 3)
            legs["sparse_prefill_s65536"] = {"ms": round(ms, 4), "ms_p10_p50_p90": call_percentiles(call, reps),
                                             "useful_flops": useful, "nnz_blocks": int(len(ci)),
                                             "TFLOP/s": round(useful / ms / 1e9, 2),
                                             "frac": round(useful / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                             "csr_walk_ms": round(ms_csr, 4),
                                             "csr_walk_TFLOP/s": round(useful / ms_csr / 1e9, 2)}
        if "dense64k" in sel:
            calld = lambda: fa.flux_attn_prefill(q, k, v, o, None, causal=1, mode=fa.FLUX_MODE_DENSE)
            msd = time_steps(calld, 3, 1)
            usefuld = 4.0 * B * Hq * d * causal_pairs(S)
            legs["dense_prefill_s65536"] = {"ms": round(msd, 4), "TFLOP/s": round(usefuld / msd / 1e9, 2),
                                            "frac": round(usefuld / msd / 1e9 / PEAK_BF16_TFLOPS, 4)}
            if "sparse_prefill_s65536" in legs:
                legs["dense_prefill_s65536"]["sparse_speedup"] = round(msd / legs["sparse_prefill_s65536"]["ms"], 3)
        del q, k, v, o
        torch.cuda.empty_cache()

    if "decode" in sel:
        # ---- decode, B=8, L=262144
        B, L, Hq, Hkv, d = 8, 262144, 32, 8, 128
        log("leg: decode L=262144")
        qd = synth.torch_normal((B, Hq, d), 1202, torch.bfloat16)
        kc = synth.torch_normal((B, L, Hkv, d), 1203, torch.bfloat16)
        vc = synth.torch_normal((B, L, Hkv, d), 1204, torch.bfloat16)
        od = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
        for mode, name in ((fa.FLUX_MODE_DENSE, "decode_dense_L262144"),
                           (fa.FLUX_MODE_SPARSE, "decode_sparse_L262144")):
            wsb = fa.flux_decode_workspace_size(B, Hq, Hkv, L, d, mode, 64, 128, 2048, 0)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
            n_keys = L if mode == fa.FLUX_MODE_DENSE else 128 + 2048
            nbytes = B * Hkv * n_keys * d * 2 * 2 + 2 * B * Hq * d * 2
            timer = KernelTimer()
            call = lambda: fa.flux_attn_decode(qd, kc, vc, od, None, mode=mode, sink_tokens=128, window_tokens=2048,
                                               workspace=ws)
            ms = time_steps(call, reps if mode == 0 else 5 * reps, 3)
            gbs = nbytes / ms / 1e6
            legs[name] = {"ms": round(ms, 4), "ms_p10_p50_p90": call_percentiles(call, reps), "bytes": nbytes,
                          "GB/s": round(gbs, 1),
                          "frac": round(gbs / PEAK_HBM_GBS, 4), "tok/s": round(B / (ms * 1e-3), 1)}
        legs["decode_sparse_L262144"]["speedup_vs_dense"] = round(
            legs["decode_dense_L262144"]["ms"] / legs["decode_sparse_L262144"]["ms"], 2)
        del qd, kc, vc, od
        torch.cuda.empty_cache()

    if "soft" in sel:
        legs["soft_routed_prefill_s8192"] = run_soft(fa, synth, torch, dev, reps)
    if "backward" in sel:
        legs.update(run_backward(fa, synth, torch, dev, reps))
    if "decode_loop" in sel:
        legs["decode_loop_36l_L262144"] = run_decode_loop(fa, synth, torch, dev)
    if "peaks" in sel:
        legs["device_ceilings"] = run_peaks(torch, dev)
    return legs


def run_soft(fa, synth, torch, dev, reps):
    """Training-time soft routing at the headline layer shape (seq 8192, 32/8 heads, head_dim 128):
    router logits -> Gumbel-softmax weights -> w_FA * dense + w_SA * sparse attention, timed against
    the dense layer alone."""
    B, S, Hq, Hkv, d = 1, 8192, 32, 8, 128
    log("leg: soft-routed prefill")
    q = synth.torch_normal((B, S, Hq, d), 1302, torch.bfloat16)
    k = synth.torch_normal((B, S, Hkv, d), 1303, torch.bfloat16)
    v = synth.torch_normal((B, S, Hkv, d), 1304, torch.bfloat16)
    o = torch.empty((B, S, Hq, d), dtype=torch.bfloat16, device=dev)
    w = synth.router_weights(1, Hq * d, 256, seed=1305)
    w_enc, b_enc, w_head, b_head = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in w)
    logits = torch.empty((1, 2), dtype=torch.float32, device=dev)
    modes = torch.empty(1, dtype=torch.int32, device=dev)
    u = torch.tensor([[0.37, 0.61]], dtype=torch.float32, device=dev)
    weights = torch.empty((1, 2), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.flux_prefill_soft_workspace_size(B, S, Hq, d), dtype=torch.uint8, device=dev)
    route_ws = torch.empty(fa.flux_route_workspace_size(1, Hq, d, 256), dtype=torch.uint8, device=dev)
    rp, ci = fa.flux_build_block_mask(S, S, 64, 128, 2048, 1, fa.FLUX_MODE_SPARSE)
    rpd, cid = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)

    def soft():
        fa.flux_route_layers([q[0]], w_enc, b_enc, w_head, b_head, modes, logits, workspace=route_ws,
                             pool_tokens=100)
        fa.flux_route_soft_weights(logits, u, 1.0, weights)
        fa.flux_attn_prefill_soft(q, k, v, o, weights[0], blk_row_ptr=rpd, blk_col_idx=cid, workspace=ws)
    ms = time_steps(soft, reps, 3)
    dense = lambda: fa.flux_attn_prefill(q, k, v, o, None, causal=1, mode=fa.FLUX_MODE_DENSE)
    ms_d = time_steps(dense, reps, 3)
    res = {"ms": round(ms, 4), "dense_only_ms": round(ms_d, 4), "overhead_vs_dense": round(ms / ms_d, 3),
           "weights": [round(float(x), 4) for x in weights[0].cpu()]}
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return res


def run_backward(fa, synth, torch, dev, reps):
    """Attention backward (dQ, dK, dV in fp32) at the headline layer shape (seq 8192, 32/8 heads, head_dim 128,
    dense causal) and at seq 65536 block-sparse (sink 128, window 2048).  O (bf16) and LSE come from one forward
    launch outside the timed region.  Algorithmic FLOPs: the five products S, dP, dV, dK, dQ, 2*d each per
    visible query-key pair and head (2.5x the forward's useful FLOPs)."""
    out = {}
    for S, mode, name in ((8192, fa.FLUX_MODE_DENSE, "backward_dense_s8192"),
                          (65536, fa.FLUX_MODE_SPARSE, "backward_sparse_s65536")):
        B, Hq, Hkv, d = 1, 32, 8, 128
        sink, window = (128, 2048) if mode == fa.FLUX_MODE_SPARSE else (0, 0)
        log(f"leg: backward S={S} mode={mode}")
        q = synth.torch_normal((B, S, Hq, d), 1402, torch.bfloat16)
        k = synth.torch_normal((B, S, Hkv, d), 1403, torch.bfloat16)
        v = synth.torch_normal((B, S, Hkv, d), 1404, torch.bfloat16)
        g = synth.torch_normal((B, S, Hq, d), 1405, torch.bfloat16)
        o = torch.empty((B, S, Hq, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        rpd = cid = None
        if mode == fa.FLUX_MODE_SPARSE:
            rp, ci = fa.flux_build_block_mask(S, S, 64, sink, window, 1, fa.FLUX_MODE_SPARSE)
            rpd, cid = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
            pairs = csr_pairs(rp, ci, S)
        else:
            pairs = causal_pairs(S)
        fa.flux_attn_prefill(q, k, v, o, lse, causal=1, mode=mode, sink_tokens=sink, window_tokens=window,
                             blk_row_ptr=rpd, blk_col_idx=cid)
        dq = torch.empty((B, S, Hq, d), dtype=torch.float32, device=dev)
        dk = torch.empty((B, S, Hkv, d), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)
        ws = torch.empty(fa.flux_attn_backward_workspace_size(B, S, Hq, Hkv, d, mode, 64, sink), dtype=torch.uint8,
                         device=dev)
        call = lambda: fa.flux_attn_backward(q, k, v, o, g, lse, dq, dk, dv, causal=True, mode=mode,
                                             sink_tokens=sink, window_tokens=window, workspace=ws)
        ms = time_steps(call, reps, 2)
        flops = 10.0 * B * Hq * d * pairs
        out[name] = {"ms": round(ms, 4), "ms_p10_p50_p90": call_percentiles(call, reps), "algorithmic_flops": flops, "TFLOP/s": round(flops / ms / 1e9, 2),
                     "frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, g, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return out


def run_decode_loop(fa, synth, torch, dev, steps=5):
    """One decode step of a 36-layer routed stack at position 262143 (batch 8, 32/8 heads, head_dim 128):
    each layer appends its new token and attends from it (flux_decode_step_layers); the 12 dense layers
    (seeded plan) stream a full 262144-row cache, the 24 sparse layers a 2176-row window cache.
    Compared with the same step when every layer is dense, and also timed as one HIP-graph replay of
    the routed step (the 108 launches captured once).  The all-dense run reuses the 12 dense
    caches three times each (36 distinct 8.6 GB caches would not fit in HBM); every layer call still
    streams its whole cache from HBM."""
    L, B, Hq, Hkv, d, S = 36, 8, 32, 8, 128, 262144
    sink, window = 128, 2048
    log("leg: routed decode loop, generating caches")
    plan = synth.layer_mode_draw(L, 12, seed=1004)
    wrows = fa.flux_window_cache_rows(64, sink, window)
    dense_k = [synth.torch_normal((B, S, Hkv, d), 3000 + 2 * i, torch.bfloat16) for i in range(12)]
    dense_v = [synth.torch_normal((B, S, Hkv, d), 3001 + 2 * i, torch.bfloat16) for i in range(12)]
    win_k = [synth.torch_normal((B, wrows, Hkv, d), 3100 + 2 * i, torch.bfloat16) for i in range(24)]
    win_v = [synth.torch_normal((B, wrows, Hkv, d), 3101 + 2 * i, torch.bfloat16) for i in range(24)]
    qs = [synth.torch_normal((B, Hq, d), 3200 + l, torch.bfloat16) for l in range(L)]
    kn = [synth.torch_normal((B, Hkv, d), 3300 + l, torch.bfloat16) for l in range(L)]
    vn = [synth.torch_normal((B, Hkv, d), 3400 + l, torch.bfloat16) for l in range(L)]
    os_ = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ws = torch.empty(fa.flux_decode_workspace_size(B, Hq, Hkv, S, d, 0, 64, sink, window), dtype=torch.uint8,
                     device=dev)
    kc, vc, di, wi = [], [], 0, 0
    for l in range(L):
        if plan[l] == 0:
            kc.append(dense_k[di]); vc.append(dense_v[di]); di += 1
        else:
            kc.append(win_k[wi]); vc.append(win_v[wi]); wi += 1
    routed = lambda: fa.flux_decode_step_layers(plan, qs, kn, vn, kc, vc, os_, None, pos=S - 1, dense_cache_rows=S,
                                                sink_tokens=sink, window_tokens=window, workspace=ws)
    ms_r = time_steps(routed, steps, 1)
    # the same step captured once in a HIP graph and replayed (no per-launch host work)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        routed()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        routed()
    ms_g = time_steps(graph.replay, steps, 1)
    del graph
    dense_kc = [dense_k[l % 12] for l in range(L)]
    dense_vc = [dense_v[l % 12] for l in range(L)]
    all_dense = lambda: fa.flux_decode_step_layers(np.zeros(L, np.int32), qs, kn, vn, dense_kc, dense_vc, os_, None,
                                                   pos=S - 1, dense_cache_rows=S, sink_tokens=sink,
                                                   window_tokens=window, workspace=ws)
    ms_d = time_steps(all_dense, steps, 1)
    bytes_r = int(12 * B * Hkv * S * d * 4 + 24 * B * Hkv * (sink + window) * d * 4)
    res = {"routed_ms": round(ms_r, 3), "routed_tok/s": round(B / (ms_r * 1e-3), 1),
           "routed_graph_ms": round(ms_g, 3), "routed_graph_tok/s": round(B / (ms_g * 1e-3), 1),
           "all_dense_ms": round(ms_d, 3), "all_dense_tok/s": round(B / (ms_d * 1e-3), 1),
           "speedup": round(ms_d / ms_r, 3), "speedup_graph": round(ms_d / ms_g, 3),
           "dense_layers": int((plan == 0).sum()),
           "routed_kv_GB/s": round(bytes_r / ms_r / 1e6, 1)}
    del dense_k, dense_v, win_k, win_v, kc, vc, dense_kc, dense_vc
    torch.cuda.empty_cache()
    return res


def run_peaks(torch, dev):
    """Context for the roofline fractions: what this device reaches outside the attention path.
    Library kernels on random N(0,1) bf16 data -- a bf16 GEMM (hipBLASLt via torch.matmul), a
    device-to-device copy, a read-only reduction (torch.sum) -- and the micro-benchmarks of
    ceilings/ceilings.hip: a pure MFMA loop, 32x32x16 and 16x16x32 (operands N(0,1) bf16, then the
    constant 1.0), a
    streaming read of 8 GiB, and the split-KV decode's own read pattern over its 2 x 4 GiB caches
    (32 splits, the split count the decode picks at batch 8 x 8 KV heads); plus the CU count and
    the peak engine clock the runtime reports."""
    log("leg: device ceilings")
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    gemm = lambda: torch.matmul(a, b)
    ms_g = time_steps(gemm, 20, 3)
    x = torch.full((1 << 31,), 1, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    copy = lambda: y.copy_(x)
    ms_c = time_steps(copy, 20, 3)
    xf = x.view(torch.float32)
    read = lambda: torch.sum(xf)
    ms_r = time_steps(read, 20, 3)
    res = {"gemm_bf16_8192_TFLOP/s": round(2.0 * n ** 3 / ms_g / 1e9, 1),
           "copy_2GiB_GB/s_read_plus_write": round(2.0 * x.numel() / ms_c / 1e6, 1),
           "sum_2GiB_GB/s_read": round(x.numel() / ms_r / 1e6, 1)}
    del a, b, x, y, xf
    torch.cuda.empty_cache()
    try:
        res.update(run_microbench(torch, dev))
    except RuntimeError as e:   # library not built: the attention legs stand without this context
        res["microbench_error"] = str(e)
    return res


def run_microbench(torch, dev):
    import ctypes

    import ceilings
    lib = ceilings.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cu, clk = ctypes.c_int(0), ctypes.c_int(0)
    ceilings.check(lib.ceil_device_info(ctypes.byref(cu), ctypes.byref(clk)), "ceil_device_info")
    out = {"compute_units": cu.value, "peak_clock_MHz": round(clk.value / 1e3)}

    def median_ms(fn, reps=10, warm=2):
        for _ in range(warm):
            fn()
        return call_percentiles(fn, reps)[1]

    wgs, iters = 4 * cu.value, 2000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    flops = lib.ceil_mfma_loop_flops(wgs, iters)
    for shape, sname in ((0, ""), (1, "16x16x32_")):
        for tag, ops in (("randn", torch.randn(1 << 18, device=dev).to(torch.bfloat16)),
                         ("const", torch.ones(1 << 18, device=dev, dtype=torch.bfloat16))):
            n_ops = ops.numel() // 8
            call = lambda: ceilings.check(lib.ceil_mfma_loop(ops.data_ptr(), n_ops, sink.data_ptr(), sink.numel(),
                                                             wgs, iters, shape, stream), "ceil_mfma_loop")
            out[f"mfma_loop_bf16_{sname}{tag}_TFLOP/s"] = round(flops / median_ms(call) / 1e9, 1)
    del sink

    sink = torch.empty(256, dtype=torch.float32, device=dev)
    nbytes = 8 << 30
    buf = torch.full((nbytes,), 1, dtype=torch.uint8, device=dev)
    call = lambda: ceilings.check(lib.ceil_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel(),
                                                       16 * cu.value, stream), "ceil_read_stream")
    out["read_stream_8GiB_GB/s"] = round(nbytes / median_ms(call) / 1e6, 1)
    B, L, H = 8, 262144, 8
    kc = buf[: nbytes // 2].view(torch.bfloat16).view(B, L, H, 128)
    vc = buf[nbytes // 2:].view(torch.bfloat16).view(B, L, H, 128)
    call = lambda: ceilings.check(lib.ceil_read_decode(kc.data_ptr(), vc.data_ptr(), B, L, H, 32, sink.data_ptr(),
                                                       sink.numel(), stream), "ceil_read_decode")
    out["read_decode_pattern_32_splits_GB/s"] = round(nbytes / median_ms(call) / 1e6, 1)
    del buf, kc, vc
    torch.cuda.empty_cache()

    # issue cost of the prefill's direct HBM -> LDS loads: cycles (s_memtime) a wave spends issuing them
    wgs = cu.value
    src = torch.zeros(wgs * 65536, dtype=torch.uint8, device=dev)
    cyc = torch.zeros(wgs * 16, dtype=torch.int64, device=dev)

    def issue_cycles(n_inst, active):
        for _ in range(3):
            ceilings.check(lib.ceil_lds_dma_issue(src.data_ptr(), src.numel(), cyc.data_ptr(), cyc.numel(), wgs,
                                                  n_inst, active, stream), "ceil_lds_dma_issue")
        torch.cuda.synchronize()
        return float(np.median(cyc.view(wgs, 8, 2)[:, :active, 0].cpu().numpy()))
    one, eight = issue_cycles(1, 1), issue_cycles(8, 1)
    out["lds_dma_issue_cycles_per_load_1_wave"] = round((eight - one) / 7, 1)
    out["lds_dma_issue_cycles_4_loads_x_8_waves"] = issue_cycles(4, 8)
    for _ in range(3):   # the same four loads per wave as one run with M0 set once (the prefill's form)
        ceilings.check(lib.ceil_lds_dma_issue4(src.data_ptr(), src.numel(), cyc.data_ptr(), cyc.numel(), wgs, 1, 8,
                                               None, 0, stream), "ceil_lds_dma_issue4")
    torch.cuda.synchronize()
    out["lds_dma_issue_cycles_4_loads_x_8_waves_one_m0_write"] = float(np.median(cyc.view(wgs, 8, 2)[:, :, 0].cpu().numpy()))
    del src, cyc

    # LDS read rate per CU (bytes per shader clock): one 8-wave workgroup per CU, and two sharing each CU
    sink = torch.zeros(512, dtype=torch.int32, device=dev)
    for per_cu in (1, 2):
        n = cu.value * per_cu
        o = torch.zeros(n * 16, dtype=torch.int64, device=dev)
        for form, name in ((0, "b128"), (1, "b64_tr_b16")):
            for _ in range(2):
                ceilings.check(lib.ceil_lds_read(o.data_ptr(), o.numel(), sink.data_ptr(), sink.numel(), n, form,
                                                 2000, stream), "ceil_lds_read")
            torch.cuda.synchronize()
            t = o.view(n, 8, 2).cpu().numpy()
            bw = t[:, :, 1].sum(axis=1) / t[:, :, 0].max(axis=1)
            out[f"lds_read_{name}_B_per_clk_per_cu_{per_cu}_wg"] = round(float(np.median(bw)) * per_cu, 1)
        del o
    return out


def cpu_baseline(synth, stack):
    """The fp64 CPU oracle (plain two-pass softmax, OpenMP over rows) on bounded samples, timed on the host's
    cores (the CPU share of this process: OMP_NUM_THREADS, else its affinity set).

    Headline (value): the 36-layer stack at seq 131072, sampled as 64 query positions x 32 heads of one dense
    and one sparse layer of the benchmarked stack (first/last rows, both sides of the sink and window edges,
    seeded random rows), each layer's time extrapolated by allowed query-key pairs to the whole layer, then to
    12 dense + 24 sparse layers (labelled extrapolated).  Beside it: the seq-8192 dense layer (every 4th row of
    all heads), the seq-65536 block-sparse layer (one row per 256 of all heads) and the batch-8, 262144-token
    decode (sequence 0, all heads, dense and sparse), each as a rate on the sample."""
    import torch

    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    visible = len(os.sched_getaffinity(0))
    Hq, d = 32, 128
    scale = 1.0 / math.sqrt(d)
    rng = np.random.default_rng(1007)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # ---- headline stack: one dense and one sparse layer, sampled rows
    S = 131072
    pos = sorted({0, 1, 127, 128, 129, 2047, 2048, 2049, S // 2, S - 2049, S - 2048, S - 65, S - 64, S - 2, S - 1}
                 | set(rng.integers(0, S, 64).tolist()))[:64]
    rows = np.array([(0, h, i) for i in pos for h in range(Hq)], np.int64)
    log(f"cpu baseline: stack sample, {len(rows)} rows per layer on {cores} threads")
    sec, pairs_s = {}, {}
    for name, sparse in (("dense", False), ("sparse", True)):
        q, k, v = stack[name]
        sec[name] = timed(lambda: oracle.attention(q, k, v, scale, causal=True, sparse=sparse, block=64,
                                                   sink_tokens=128, window_tokens=2048, rows=rows, n_threads=cores))
        pairs_s[name] = Hq * sum((sparse_row_pairs(i) if sparse else i + 1) for i in pos)
    layer_pairs = {"dense": stack["flops_dense"] / (4.0 * d), "sparse": stack["flops_sparse"] / (4.0 * d)}
    layer_sec = {m: sec[m] * layer_pairs[m] / pairs_s[m] for m in sec}
    n_dense = int((stack["plan"] == 0).sum())
    stack_sec = n_dense * layer_sec["dense"] + (len(stack["plan"]) - n_dense) * layer_sec["sparse"]
    out = {"value": round(stack["useful"] / stack_sec / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
           "host_cpus_visible": visible, "kind": "oracle",
           "sample": f"36-layer seq-131072 stack, extrapolated: {len(pos)} query positions x {Hq} heads of one dense "
                     f"layer ({sec['dense']:.2f} s) and one block-sparse layer ({sec['sparse']:.2f} s) of the "
                     f"benchmarked stack, scaled by allowed query-key pairs to 12 dense + 24 sparse layers = "
                     f"{stack_sec:.0f} s per step on the CPU"}
    sub = {}

    # ---- seq-8192 dense layer
    q, k, v = synth.qkv_bf16(1, 8192, Hq, 8, d, seed=1002)
    rows = np.array([(0, h, i) for i in range(3, 8192, 4) for h in range(Hq)], np.int64)
    t = timed(lambda: oracle.attention(q, k, v, scale, causal=True, rows=rows, n_threads=cores))
    fl = 4.0 * d * Hq * sum(i + 1 for i in range(3, 8192, 4))
    sub["layer_s8192_dense"] = {"TFLOP/s": round(fl / t / 1e12, 6), "seconds": round(t, 2),
                                "sample": f"every 4th query row x {Hq} heads ({len(rows)} rows, {fl:.3e} useful flop)"}

    # ---- seq-65536 block-sparse layer
    S = 65536
    qd = synth.torch_normal((1, S, Hq, d), 1102, torch.bfloat16)
    kd = synth.torch_normal((1, S, 8, d), 1103, torch.bfloat16)
    vd = synth.torch_normal((1, S, 8, d), 1104, torch.bfloat16)
    q, k, v = (host_bits(x) for x in (qd, kd, vd))
    del qd, kd, vd
    prow = list(range(255, S, 256))
    rows = np.array([(0, h, i) for i in prow for h in range(Hq)], np.int64)
    t = timed(lambda: oracle.attention(q, k, v, scale, causal=True, sparse=True, block=64, sink_tokens=128,
                                       window_tokens=2048, rows=rows, n_threads=cores))
    fl = 4.0 * d * Hq * sum(sparse_row_pairs(i) for i in prow)
    sub["layer_s65536_sparse"] = {"TFLOP/s": round(fl / t / 1e12, 6), "seconds": round(t, 2),
                                  "sample": f"every 256th query row x {Hq} heads ({len(rows)} rows, {fl:.3e} useful "
                                            f"flop)"}
    del q, k, v

    # ---- decode, batch 8 x 262144-token cache: sequence 0, all 32 heads
    L = 262144
    qd = synth.torch_normal((8, Hq, d), 1202, torch.bfloat16)
    kd = synth.torch_normal((8, L, 8, d), 1203, torch.bfloat16)
    vd = synth.torch_normal((8, L, 8, d), 1204, torch.bfloat16)
    q0, k0, v0 = host_bits(qd[:1]), host_bits(kd[:1]), host_bits(vd[:1])
    del qd, kd, vd
    torch.cuda.empty_cache()
    for mode, keys in (("dense", L), ("sparse", 128 + 2048)):
        t = timed(lambda: oracle.decode(q0, k0, v0, scale, sparse=mode == "sparse", block=64, sink_tokens=128,
                                        window_tokens=2048, n_threads=cores))
        nbytes = 8 * keys * d * 2 * 2 + 2 * Hq * d * 2     # K+V of the allowed keys of one sequence, q and o
        sub[f"decode_L262144_{mode}"] = {"GB/s": round(nbytes / t / 1e9, 4), "tok/s": round(1.0 / t, 3),
                                         "seconds": round(t, 3),
                                         "sample": f"sequence 0 of 8, all {Hq} heads ({nbytes} algorithmic bytes)"}
    out["other_configs"] = sub
    return out


if __name__ == "__main__":
    main()
