"""ctypes binding of libceilings.so: device micro-benchmarks (pure MFMA loop, streaming read, the decode's
read pattern, the issue cost of direct HBM -> LDS loads, CU count and clock) that bench.py reports beside the attention kernels' roofline fractions.
Measurement context only; the attention path never calls it."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libceilings.so")

_i32, _i64, _p, _f32p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)

SIGNATURES = {
    "ceil_device_info": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]),
    "ceil_mfma_loop_flops": (ctypes.c_double, [_i32, _i32]),
    "ceil_mfma_loop": (ctypes.c_int, [_p, _i64, _p, _i64, _i32, _i32, _i32, _p]),
    "ceil_read_stream": (ctypes.c_int, [_p, _i64, _p, _i64, _i32, _p]),
    "ceil_read_decode": (ctypes.c_int, [_p, _p, _i64, _i64, _i32, _i32, _p, _i64, _p]),
    "ceil_lds_dma_issue": (ctypes.c_int, [_p, _i64, _p, _i64, _i32, _i32, _i32, _p]),
    "ceil_lds_dma_issue4": (ctypes.c_int, [_p, _i64, _p, _i64, _i32, _i32, _i32, _p, _i64, _p]),
    "ceil_lds_read": (ctypes.c_int, [_p, _i64, _p, _i64, _i32, _i32, _i32, _p]),
}


def load():
    """The library with typed entry points; raises if it has not been built."""
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run `python ceilings/build.py`")
    import torch  # noqa: F401  -- bind to the HIP runtime torch loaded (tensors and streams come from it)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


def check(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what} failed with hipError {status}")
