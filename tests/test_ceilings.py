"""The device micro-benchmarks bench.py reports beside the roofline fractions (ceilings/ceilings.hip).

CPU: the library loads, exports its entry points and rejects arguments that do not fit its kernels
(validation runs before any device call).  GPU: each kernel runs at a small size; the MFMA loops on
all-ones operands must leave exactly iters * 8 MFMAs * the contraction depth (16 or 32) in each of their
accumulator elements, which pins the number of MFMAs they issue (and so the FLOPs bench.py divides).
"""
import ctypes
import os

import pytest

import ceilings

HIP_INVALID_VALUE = 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ceilings.LIB_PATH):
        pytest.skip("libceilings.so not built")
    return ceilings.load()


def test_exports_and_flop_count(lib):
    for name in ceilings.SIGNATURES:
        assert hasattr(lib, name)
    assert lib.ceil_mfma_loop_flops(1024, 2000) == 1024 * 4 * 2000 * 32 * 2 * 32 * 32 * 16


def test_validation_before_launch(lib):
    assert lib.ceil_device_info(None, None) == HIP_INVALID_VALUE
    assert lib.ceil_mfma_loop(None, 1, None, 0, 1, 1, 0, None) == HIP_INVALID_VALUE
    assert lib.ceil_mfma_loop(16, 1, 16, 256, 1, 1, 2, None) == HIP_INVALID_VALUE        # unknown shape
    assert lib.ceil_mfma_loop(16, 1, 16, 255, 1, 1, 0, None) == HIP_INVALID_VALUE     # sink too small
    assert lib.ceil_read_stream(16, 24, 16, 256, 1, None) == HIP_INVALID_VALUE        # not a multiple of 16
    assert lib.ceil_read_decode(16, 16, 1, 192, 1, 2, 16, 256, None) == HIP_INVALID_VALUE   # L % (64 splits)
    assert lib.ceil_lds_dma_issue(16, 65536, 16, 16, 1, 9, 1, None) == HIP_INVALID_VALUE      # more than 8 loads
    assert lib.ceil_lds_dma_issue(16, 65536, 16, 16, 1, 4, 0, None) == HIP_INVALID_VALUE      # no active wave
    assert lib.ceil_lds_dma_issue(16, 65535, 16, 16, 1, 4, 8, None) == HIP_INVALID_VALUE      # source too small
    assert lib.ceil_lds_dma_issue(16, 65536, 16, 15, 1, 4, 8, None) == HIP_INVALID_VALUE      # out too small
    assert lib.ceil_lds_dma_issue4(16, 65536, 16, 16, 1, 3, 8, None, 0, None) == HIP_INVALID_VALUE   # unknown form
    assert lib.ceil_lds_dma_issue4(16, 65536, 16, 16, 1, 1, 9, None, 0, None) == HIP_INVALID_VALUE   # 9 waves
    assert lib.ceil_lds_dma_issue4(16, 65536, 16, 16, 1, 1, 8, 16, 32767, None) == HIP_INVALID_VALUE  # check short
    assert lib.ceil_lds_read(16, 16, 16, 512, 1, 2, 10, None) == HIP_INVALID_VALUE      # unknown form
    assert lib.ceil_lds_read(16, 15, 16, 512, 1, 0, 10, None) == HIP_INVALID_VALUE      # out too small
    assert lib.ceil_lds_read(16, 16, 16, 511, 1, 0, 10, None) == HIP_INVALID_VALUE      # sink too small


@pytest.mark.gpu
def test_kernels_run(lib):
    import torch
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    wgs, iters = 8, 10
    ops = torch.ones(8 * 64, dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(wgs * 256, dtype=torch.float32, device=dev)
    assert lib.ceil_mfma_loop(ops.data_ptr(), ops.numel() // 8, sink.data_ptr(), sink.numel(), wgs, iters, 0,
                              stream) == 0
    torch.cuda.synchronize()
    assert torch.all(sink == 4 * 16 * iters * 8 * 16).item()
    # 16x16x32: 8 accumulators of 4, each updated 8 times per iteration, 32 products per element
    sink.zero_()
    assert lib.ceil_mfma_loop(ops.data_ptr(), ops.numel() // 8, sink.data_ptr(), sink.numel(), wgs, iters, 1,
                              stream) == 0
    torch.cuda.synchronize()
    assert torch.all(sink == 8 * 4 * iters * 8 * 32).item()

    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    small = torch.zeros(256, dtype=torch.float32, device=dev)
    assert lib.ceil_read_stream(buf.data_ptr(), buf.numel() - 48, small.data_ptr(), 256, 7, stream) == 0
    B, L, H = 1, 256, 2
    kv = torch.zeros(2 * B * L * H * 128, dtype=torch.bfloat16, device=dev)
    half = B * L * H * 128
    assert lib.ceil_read_decode(kv.data_ptr(), kv[half:].data_ptr(), B, L, H, 2, small.data_ptr(), 256,
                                stream) == 0
    torch.cuda.synchronize()
    assert torch.all(small == 0).item()
    cu, clk = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.ceil_device_info(ctypes.byref(cu), ctypes.byref(clk)) == 0
    assert cu.value > 0 and clk.value > 0

    # direct-load issue timing: the active waves report positive cycle counts, issue <= issue + wait
    src = torch.zeros(4 * 65536, dtype=torch.uint8, device=dev)
    out = torch.zeros(4 * 16, dtype=torch.int64, device=dev)
    assert lib.ceil_lds_dma_issue(src.data_ptr(), src.numel(), out.data_ptr(), out.numel(), 4, 4, 3, stream) == 0
    torch.cuda.synchronize()
    t = out.view(4, 8, 2).cpu()
    assert bool((t[:, :3, 0] > 0).all()) and bool((t[:, :, 0] <= t[:, :, 1]).all())

    # the four-load runs (M0 set once, immediate offsets 0..3072; or M0 set per load): every active wave's
    # 4 KB of LDS holds bytes [8192*wave, +4096) of its workgroup's 64 KB, i.e. the immediate offset moved
    # the LDS destination and the global source alike
    src.copy_(torch.arange(src.numel(), device=dev, dtype=torch.int64).remainder(251).to(torch.uint8))
    chk = torch.zeros(4 * 8 * 4096, dtype=torch.uint8, device=dev)
    want = src.view(4, 8, 8192)[:, :, :4096].cpu()
    for form in (1, 2):
        chk.zero_()
        assert lib.ceil_lds_dma_issue4(src.data_ptr(), src.numel(), out.data_ptr(), out.numel(), 4, form, 5,
                                       chk.data_ptr(), chk.numel(), stream) == 0
        torch.cuda.synchronize()
        got = chk.view(4, 8, 4096).cpu()
        assert torch.equal(got[:, :5], want[:, :5]), form
        assert bool((got[:, 5:] == 0).all()) and bool((out.view(4, 8, 2)[:, :5, 0] > 0).all().cpu())

    # LDS read loop: every wave reports a positive cycle count and the bytes its 10 x 8 reads cover
    sink = torch.zeros(512, dtype=torch.int32, device=dev)
    for form, per_read in ((0, 1024), (1, 512)):
        out.zero_()
        assert lib.ceil_lds_read(out.data_ptr(), out.numel(), sink.data_ptr(), sink.numel(), 4, form, 10,
                                 stream) == 0
        torch.cuda.synchronize()
        t = out.view(4, 8, 2).cpu()
        assert bool((t[:, :, 0] > 0).all()) and bool((t[:, :, 1] == 10 * 8 * per_read).all()), form
