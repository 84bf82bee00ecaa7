"""The host layer and the oracle under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/host_checks.cpp drives the pointer-writing host paths -- the block-mask builder
(every shape class, capacity errors), argument validation of every entry point, workspace sizing,
status strings -- and the fp64 oracle's functions.  This test builds it with the library's host
source (csrc/flux_api.cpp) and the oracle (oracle/flux_oracle.c) instrumented on the host side
(the device objects are the library's ordinary ones; GPU code is never instrumented), runs it,
and requires exit status 0 with no sanitizer report.
"""
import importlib.util
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm/bin"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr
    return r


def _device_objects():
    """The library's ordinary (uninstrumented) kernel objects, compiled if the build has not left them."""
    spec = importlib.util.spec_from_file_location("_flux_build_san",
                                                  os.path.join(ROOT, "long_context_attention_tiled_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    os.makedirs(b.OBJDIR, exist_ok=True)
    objs = []
    for src in b.SOURCES:
        if src == "flux_api.cpp":
            continue
        obj = os.path.join(b.OBJDIR, src + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(b.CSRC, src)):
            obj = b._compile(src, False)
        objs.append(obj)
    return objs


@pytest.mark.slow
def test_host_layer_and_oracle_clean_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    api_o = os.path.join(OUT, "flux_api.o")
    # host side instrumented, device side (none in this file) untouched
    _run([HIPCC, "-x", "hip", "-c", os.path.join(ROOT, "long_context_attention_tiled_amd", "csrc", "flux_api.cpp"),
          "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-g", "-O1",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"] + inc +
         ["-o", api_o])
    oracle_o = os.path.join(OUT, "flux_oracle.o")
    _run([os.path.join(LLVM, "clang"), "-c", "-std=c11", "-fopenmp", "-fPIC"] + SAN +
         [os.path.join(ROOT, "oracle", "flux_oracle.c"), "-o", oracle_o])
    drv_o = os.path.join(OUT, "host_checks.o")
    _run([os.path.join(LLVM, "clang++"), "-c", "-std=c++17"] + SAN + inc +
         [os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", drv_o])
    exe = os.path.join(OUT, "host_checks")
    _run([os.path.join(LLVM, "clang++"), "-fopenmp"] + SAN + [drv_o, api_o, oracle_o] + _device_objects() +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib:/opt/rocm/llvm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "host checks ok" in r.stdout, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
