"""GPU check of the MFMA ceiling probe (libtdg_probe.so): it runs the number
of MFMAs it claims, which is what its FLOP count and the bench's ceiling
figure rest on.  bf16 stream: with every operand 1.0 each 16x16x32 MFMA adds
32 to each of its outputs; a lane holds 128 outputs (8 x 4 tiles of 4), each
updated twice per K tile, so its sum is 128 * 64 * iters exactly.  8-bit
stream: each 32x32x64 MFMA adds 64; a lane holds 128 outputs (4 x 2 tiles of
16), each updated twice per K tile: 128 * 128 * iters."""
import ctypes
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(ROOT, "tiled_dense_gemm_03_amd", "libtdg_probe.so"))
    lib.tdgp_operand_elems.restype = ctypes.c_size_t
    lib.tdgp_mfma_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.tdgp_operand_bytes_f8.restype = ctypes.c_size_t
    lib.tdgp_mfma_stream_f8.argtypes = lib.tdgp_mfma_stream.argtypes
    return lib


@pytest.mark.parametrize("value,iters,blocks", [(1.0, 10, 8), (1.0, 2047, 3), (0.0, 100, 256)])
def test_mfma_stream_counts(probe, value, iters, blocks):
    print("CASE probe value", value, "iters", iters, "blocks", blocks, flush=True)
    sys.stdout.flush()
    n = probe.tdgp_operand_elems()
    ops = torch.full((n,), value, dtype=torch.bfloat16, device="cuda")
    sink = torch.full((blocks * 512,), -1.0, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(blocks * 2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    assert probe.tdgp_mfma_stream(ops.data_ptr(), iters, blocks, sink.data_ptr(), clocks.data_ptr(),
                                  ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    expect = 128.0 * 64.0 * iters * value
    assert torch.equal(sink.cpu(), torch.full((blocks * 512,), expect, dtype=torch.float32))
    ck = clocks.view(blocks, 2).cpu()
    assert bool((ck > 0).all())


@pytest.mark.parametrize("byte,value,iters,blocks", [(0x38, 1.0, 10, 8), (0x38, 1.0, 1023, 3), (0x00, 0.0, 100, 256)])
def test_mfma_stream_f8_counts(probe, byte, value, iters, blocks):
    print("CASE probe f8 byte", byte, "iters", iters, "blocks", blocks, flush=True)
    sys.stdout.flush()
    ops = torch.full((probe.tdgp_operand_bytes_f8(),), byte, dtype=torch.uint8, device="cuda")
    sink = torch.full((blocks * 512,), -1.0, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(blocks * 2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    assert probe.tdgp_mfma_stream_f8(ops.data_ptr(), iters, blocks, sink.data_ptr(), clocks.data_ptr(),
                                     ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    expect = 128.0 * 128.0 * iters * value
    assert torch.equal(sink.cpu(), torch.full((blocks * 512,), expect, dtype=torch.float32))
    assert bool((clocks.view(blocks, 2).cpu() > 0).all())
