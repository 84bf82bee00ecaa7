"""Phase timeline of the prefill's steady tile loop (measurement tool; the attention path never uses it).

    python ceilings/phase_trace.py build     # on the CPU: instrumented copy of the library, compiled for gfx950
    python ceilings/phase_trace.py run [DIR] # on an MI355X: per-wave phase durations, one JSON line
                                             # (with DIR, also the raw stamps as .npy files there)

`build` copies long_context_attention_tiled_amd/ into ceilings/phase_trace_pkg/ and adds, in the copy only,
s_memtime stamps to every steady step of prefill_bf16.hip's tile loop (step start; end of the first-phase
work; after the mid-step barrier; end of the second-phase work; after the wait for this step's loads) for
three workgroups (blockIdx 0, 97, 203) over the first 64 steps of their first work unit, with an
s_memrealtime stamp (a constant 100 MHz count) at each step start to give the rate s_memtime counts at
during the kernel, plus an entry point
flux_probe_set_trace() that hands the kernel a device buffer for them.  The arithmetic, the loads and the
schedule are those of the library; results stay exact (the parity of the copy is checked by `run`).

`run` times the copy with and without the stamps and reports, per wave (waves 0-3 form the group that runs
matrix work in the first phase, waves 4-7 the other), the median cycles of each segment over steps 2..63,
for the seq-8192 dense layer and the seq-131072 dense and block-sparse layers (32/8 heads, head_dim 128, bf16).
At seq 8192 the traced copy's output is compared with the library's own (loaded beside it): the stamps
change no arithmetic, so the two agree to within the rounding of the bf16 output.
"""
from __future__ import annotations

import ctypes
import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG_PARENT = os.path.join(HERE, "phase_trace_pkg")
PKG = os.path.join(PKG_PARENT, "long_context_attention_tiled_amd")
N_SLOTS, N_WAVES, N_STEPS, N_STAMPS = 3, 8, 64, 7


def _edit(path, old, new):
    s = open(path).read()
    if old not in s:
        raise RuntimeError(f"{os.path.basename(path)}: pattern not found: {old[:60]!r}")
    open(path, "w").write(s.replace(old, new, 1))


def build() -> str:
    if os.path.exists(PKG_PARENT):
        shutil.rmtree(PKG_PARENT)
    shutil.copytree(os.path.join(ROOT, "long_context_attention_tiled_amd"), PKG,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "_build"))
    c = os.path.join(PKG, "csrc")
    inc = os.path.join(ROOT, "include", "flux_attn.h")
    _edit(os.path.join(c, "flux_api.cpp"), '#include "../../include/flux_attn.h"', f'#include "{inc}"')
    _edit(os.path.join(c, "flux_internal.h"), "    int window_blocks;\n};",
          "    int window_blocks;\n    unsigned long long* trace;\n};")
    _edit(os.path.join(c, "flux_internal.h"), "hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);",
          "hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);\nextern unsigned long long* g_trace;")
    _edit(os.path.join(c, "flux_api.cpp"), "    a.num_cu = device_cu_count();\n    hipError_t e = in_dtype",
          "    a.num_cu = device_cu_count();\n    a.trace = flux::g_trace;\n    hipError_t e = in_dtype")
    _edit(os.path.join(c, "flux_api.cpp"), 'extern "C" {\n',
          'namespace flux { unsigned long long* g_trace = nullptr; }\nextern "C" {\n'
          'void flux_probe_set_trace(void* p) { flux::g_trace = (unsigned long long*)p; }\n')
    p = os.path.join(c, "prefill_bf16.hip")
    s = open(p).read()
    stamp = lambda n: f"                    const unsigned long long {n} = probe ? __builtin_amdgcn_s_memtime() : 0ull;\n"
    w0 = s.index("                auto step = [&](auto slot_tag) {\n")
    w1 = s.index("\n                };\n", w0) + 1
    body = s[w0:w1]
    sync = "                    __syncthreads();\n"
    i1 = body.index("\n" + sync) + 1
    body = body[:i1] + stamp("t1") + sync + stamp("t2") + body[i1 + len(sync):]
    i3 = body.index("                    __builtin_amdgcn_s_waitcnt(0x0f70);")
    i3e = body.index("\n", i3) + 1
    body = body[:i3] + stamp("t3") + body[i3:i3e] + stamp("t4") + body[i3e:]
    i5 = body.index("\n" + sync, body.index("t4 =")) + 1
    body = (body[:i5 + len(sync)] + stamp("t5") +
            "                    if (probe && pstep < 64 && lane == 0) {\n"
            "                        unsigned long long* dst = a.trace + ((size_t)(pslot * 8 + wave) * 64 + pstep) * 7;\n"
            "                        dst[0] = t0; dst[1] = t1; dst[2] = t2; dst[3] = t3; dst[4] = t4; dst[5] = r0;\n"
            "                        dst[6] = t5;\n"
            "                    }\n                    ++pstep;\n" + body[i5 + len(sync):])
    head = "                    constexpr int sl = decltype(slot_tag)::value;\n"
    body = body.replace(head, head + stamp("t0") +
                        "                    const unsigned long long r0 = probe ? __builtin_amdgcn_s_memrealtime() : 0ull;\n", 1)
    pre = ("                int pstep = 0;\n"
           "                const int pslot = (blockIdx.x == 0) ? 0 : (blockIdx.x == 97) ? 1 : (blockIdx.x == 203) ? 2 : -1;\n"
           "                const bool probe = a.trace && pslot >= 0 && k == 1;\n")
    open(p, "w").write(s[:w0] + pre + body + s[w1:])
    bp = os.path.join(PKG, "build.py")
    _edit(bp, 'OBJDIR = os.path.join(ROOT, "_build")', 'OBJDIR = os.path.join(HERE, "_build")')
    r = subprocess.run([sys.executable, bp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stdout[-4000:] + r.stderr[-4000:])
    shutil.rmtree(os.path.join(PKG, "_build"), ignore_errors=True)
    return os.path.join(PKG, "libflux_attn.so")


def _medians(tr):
    """tr [slots, waves, steps, 7] -> per-wave medians of the segments over the recorded steady steps (the first
    two of each traced unit left out; a unit with fewer than 64 steps leaves the rest of its rows at zero)."""
    import numpy as np
    seg = {"first_phase_work": (0, 1), "mid_barrier_wait": (1, 2), "second_phase_work": (2, 3),
           "load_wait": (3, 4)}
    parts, steps = [], []
    for sl in range(tr.shape[0]):
        n = int((tr[sl, :, :, 0] > 0).all(axis=0).sum())
        if n >= 4:
            parts.append(tr[sl, :, 2:n])
            steps.append((tr[sl, :, 3:n, 0] - tr[sl, :, 2:n - 1, 0]).ravel())
    t = np.concatenate(parts, axis=1)
    out = {"steps_recorded": int(t.shape[1])}
    for name, (a, b) in seg.items():
        out[name] = [int(np.median(t[w, :, b] - t[w, :, a])) for w in range(N_WAVES)]
    out["step"] = int(np.median(np.concatenate(steps)))
    busiest = max(out["first_phase_work"][w] + out["mid_barrier_wait"][w] + out["second_phase_work"][w] +
                  out["load_wait"][w] for w in range(N_WAVES))
    out["end_of_step_barrier_and_loop"] = out["step"] - busiest
    # per step, across the 8 waves: from the last wave's arrival at a barrier to the first wave's stamp right
    # after it (the barrier's release), how far apart the waves arrive at the end-of-step one, and per wave
    # from that barrier's release to the next step's first stamp (the loop's branch back to its head)
    mid_rel, end_rel, end_spread, top, top_on, top_back = [], [], [], [], [], []
    for sl in range(tr.shape[0]):
        n = int((tr[sl, :, :, 0] > 0).all(axis=0).sum())
        if n >= 4:
            x = tr[sl, :, 2:n]
            mid_rel.append(x[:, :, 2].min(axis=0) - x[:, :, 1].max(axis=0))
            end_rel.append(x[:, :, 6].min(axis=0) - x[:, :, 4].max(axis=0))
            gap = x[:, 1:, 0] - x[:, :-1, 6]
            top.append(gap.ravel())
            # the loop runs two steps per pass: an even step is followed by the second copy (straight on),
            # an odd one by the branch back to the loop head
            top_on.append(gap[:, 0::2].ravel())
            top_back.append(gap[:, 1::2].ravel())
            end_spread.append(x[:, :, 4].max(axis=0) - x[:, :, 4].min(axis=0))
    out["mid_barrier_release"] = int(np.median(np.concatenate(mid_rel)))
    out["end_barrier_release"] = int(np.median(np.concatenate(end_rel)))
    out["end_barrier_to_next_step"] = int(np.median(np.concatenate(top)))
    out["end_barrier_to_next_step_straight_on"] = int(np.median(np.concatenate(top_on)))
    out["end_barrier_to_next_step_via_loop_branch"] = int(np.median(np.concatenate(top_back)))
    out["end_barrier_arrival_spread"] = int(np.median(np.concatenate(end_spread)))
    # s_memtime ticks per s_memrealtime tick (the latter counts a constant 100 MHz) over each traced unit
    ratios = []
    for sl in range(tr.shape[0]):
        n = int((tr[sl, :, :, 0] > 0).all(axis=0).sum())
        if n >= 4:
            dm = tr[sl, :, n - 1, 0] - tr[sl, :, 1, 0]
            dr = tr[sl, :, n - 1, 5] - tr[sl, :, 1, 5]
            ratios += list(dm[dr > 0] / dr[dr > 0])
    out["memtime_MHz"] = round(100.0 * float(np.median(ratios)), 1) if ratios else None
    return out


def run(dump_dir: str = "") -> dict:
    """Time and trace the three workloads; with dump_dir, also save each raw stamp array there (.npy)."""
    sys.path.insert(0, ROOT)
    sys.path.insert(0, PKG_PARENT)
    import numpy as np
    import torch
    import long_context_attention_tiled_amd as fa
    assert os.path.dirname(fa.LIB_PATH) == PKG, fa.LIB_PATH
    traced = fa._lib
    plain = ctypes.CDLL(os.path.join(ROOT, "long_context_attention_tiled_amd", "libflux_attn.so"))
    plain.flux_attn_prefill.argtypes = traced.flux_attn_prefill.argtypes
    plain.flux_attn_prefill.restype = traced.flux_attn_prefill.restype
    res = {}
    for name, S, mode in (("dense_s8192", 8192, 0), ("dense_s131072", 131072, 0), ("sparse_s131072", 131072, 1)):
        print(f"[phase_trace] {name}", file=sys.stderr, flush=True)
        B, Hq, Hkv, d = 1, 32, 8, 128
        g = torch.Generator(device="cuda").manual_seed(11)
        q = torch.randn((B, S, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
        k = torch.randn((B, S, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((B, S, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        o = torch.empty((B, S, Hq, d), dtype=torch.bfloat16, device="cuda")
        trace = torch.zeros(N_SLOTS * N_WAVES * N_STEPS * N_STAMPS, dtype=torch.int64, device="cuda")
        call = lambda: fa.flux_attn_prefill(q, k, v, o, None, causal=1, mode=mode)
        reps = 20 if S <= 8192 else 2

        def timed():
            call()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                call()
            e.record()
            torch.cuda.synchronize()
            return s.elapsed_time(e) / reps
        ms_plain = timed()
        fa.lib().flux_probe_set_trace(ctypes.c_void_p(trace.data_ptr()))
        ms_traced = timed()
        fa.lib().flux_probe_set_trace(None)
        tr = trace.view(N_SLOTS, N_WAVES, N_STEPS, N_STAMPS).cpu().numpy().astype(np.int64)
        r = {"ms_untraced": round(ms_plain, 4), "ms_traced": round(ms_traced, 4), **_medians(tr)}
        if dump_dir:
            np.save(os.path.join(dump_dir, f"phase_trace_{name}.npy"), tr)
        if S == 8192:   # the traced copy computes the same attention as the library itself
            traced_out = o.clone()
            fa._lib = plain
            try:
                call()
            finally:
                fa._lib = traced
            torch.cuda.synchronize()
            r["max_abs_diff_vs_library"] = float((traced_out.float() - o.float()).abs().max())
            assert r["max_abs_diff_vs_library"] <= 1e-2
        res[name] = r
        del q, k, v, o
        torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "build":
        print(build())
    elif len(sys.argv) > 1 and sys.argv[1] == "run":
        print(json.dumps(run(sys.argv[2] if len(sys.argv) > 2 else "")), flush=True)
    else:
        print(__doc__)
        sys.exit(2)
