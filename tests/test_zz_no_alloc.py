"""The allocation-free entry point ``tdg_gemm_noalloc`` against ``tdg_gemm``
with a caller workspace (the same schedule with the split-K partials in the
library's scratch array instead): the outputs must be equal bit for bit, on
two calls in a row whose second is smaller, on problems that split K and on
one that does not, and on integer inputs also equal to the oracle's exact
sums.  Both calls go through the C ABI (ctypes, raw device pointers)."""
import ctypes
import sys

import pytest
import torch

from parity import check_exact, ref_gemm
from workloads import make_inputs

pytestmark = pytest.mark.gpu

CODE = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}


@pytest.fixture(scope="module")
def tdg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_03_amd as t
    return t


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def run_pair(tdg, layout, M, N, K, dt, odt, dist, seed):
    """(C from tdg_gemm_noalloc, C from tdg_gemm with a fresh workspace, A, B)."""
    transb = 1 if layout == "tn" else 0
    a, b = make_inputs(M, N, K, layout, "f16" if dt == torch.float16 else "bf16", dist, seed=seed)
    ad, bd = a.cuda(), b.cuda()
    lda, ldb = K, (K if transb else N)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    c_na = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    st = tdg._binding.lib.tdg_gemm_noalloc(0, transb, 0, M, N, K, ad.data_ptr(), lda, 0, bd.data_ptr(), ldb, 0,
                                           c_na.data_ptr(), N, 0, 1, CODE[dt], CODE[odt], stream)
    assert st == 0, tdg.tdg_last_error()
    need = tdg.tdg_gemm_workspace_size(transb, M, N, K, 1, 0)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    c_ws = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    st = tdg._binding.lib.tdg_gemm(0, transb, 0, M, N, K, ad.data_ptr(), lda, 0, bd.data_ptr(), ldb, 0,
                                   c_ws.data_ptr(), N, 0, 1, CODE[dt], CODE[odt], ws.data_ptr(), ws.numel(), stream)
    assert st == 0, tdg.tdg_last_error()
    torch.cuda.synchronize()
    return c_na.cpu(), c_ws.cpu(), a, b, need


# (layout, M, N, K, input, output): the first two of each pair split K (fewer
# 128 x 128 tiles than CUs, long K), the second smaller than the first; the
# last does not split.
CASES = [
    ("nn", 300, 520, 16384, torch.float16, torch.float32),
    ("nn", 260, 384, 16384, torch.float16, torch.float32),
    ("tn", 640, 520, 16384, torch.bfloat16, torch.bfloat16),
    ("tn", 512, 256, 16384, torch.bfloat16, torch.bfloat16),
    ("nn", 1024, 1024, 512, torch.float16, torch.float16),
]


@pytest.mark.parametrize("dist", ["uniform", "ints"])
def test_noalloc_equals_workspace_call(tdg, dist):
    for i, (layout, M, N, K, dt, odt) in enumerate(CASES):
        announce("noalloc", dist, layout, M, N, K, dt, odt)
        c_na, c_ws, a, b, need = run_pair(tdg, layout, M, N, K, dt, odt, dist, seed=40 + i)
        if i < 4:
            assert need > 0, "case %d should take the split-K schedule" % i
        assert torch.equal(c_na, c_ws), "%s %dx%dx%d: no-alloc result differs from the workspace call" % (
            layout, M, N, K)
        if dist == "ints":
            check_exact(c_na, ref_gemm(a, b, "f16" if dt == torch.float16 else "bf16", layout),
                        {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}[odt],
                        "noalloc %s %dx%dx%d" % (layout, M, N, K))
