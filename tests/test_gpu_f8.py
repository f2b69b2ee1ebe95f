"""GPU parity of the 8-bit path (E4M3 / E5M2 operands with E8M0 block scales
and fp32 row scales): the HIP library through its C ABI against the CPU
oracle's scaled product.

Exact cases use small-integer operands, block scales within a few binades
and power-of-two row scales, sized so that every partial sum is an integer
multiple of the smallest term below 2^24 of them: fp32 accumulation is then
exact, and so is the output rounding of the oracle's value.  Random cases use
the tolerances of the 16-bit path.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from parity import OUT_TORCH, check_exact, check_tol, to_f64
from workloads import make_f8_inputs, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_03_amd as t
    return t


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def pad_cols(x, mult):
    """Copy of a (rows, cols) uint8 array whose row stride is a multiple of
    `mult`, the padding filled with 0xFF (NaN as E8M0 and as E4M3 bytes);
    returns the padded array and the view of its first cols columns."""
    rows, cols = x.shape
    ld = -(-max(cols, 1) // mult) * mult
    p = np.full((rows, ld), 0xFF, dtype=np.uint8)
    p[:, :cols] = x
    return p, cols


def gpu_f8(tdg, a, b, afmt, bfmt, xa=None, xb=None, sa=None, sb=None, out="f32", transc=False, config=-1):
    """Run the library on host arrays (block-scale rows padded to a stride
    that is a multiple of 16 with NaN bytes) and return the CPU result."""
    ad, bd = dev(a), dev(b)
    xad = xbd = None
    if xa is not None:
        xp, cols = pad_cols(xa, 16)
        xad = dev(xp)[:, :cols]
    if xb is not None:
        xp, cols = pad_cols(xb, 16)
        xbd = dev(xp)[:, :cols]
    c = tdg.gemm_f8(ad, bd, a_fmt=afmt, b_fmt=bfmt, block_scale_a=xad, block_scale_b=xbd,
                    scale_a=dev(sa), scale_b=dev(sb), out_dtype=OUT_TORCH[out], transc=transc, config=config)
    torch.cuda.synchronize()
    return c.cpu()


FMTS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]
P2 = np.float32([0.5, 1.0, 2.0])


def pow2_scales(n, seed):
    return P2[np.random.default_rng(seed).integers(0, 3, size=n)]


# (M, N, K, spread of the block-scale exponents) -- the spread keeps sums exact
EXACT_SHAPES = [(64, 64, 128, 1), (300, 520, 1040, 1), (257, 264, 4096, 0), (1, 1, 16, 1), (129, 255, 2064, 1),
                (512, 256, 1024, 1)]


@pytest.mark.parametrize("config", [0, 1])
@pytest.mark.parametrize("shape", EXACT_SHAPES)
def test_f8_integer_exact(tdg, shape, config):
    M, N, K, spread = shape
    for idx, (afmt, bfmt) in enumerate(FMTS):
        out = ["f32", "bf16", "f16", "f32"][idx]
        seed = 1000 + 10 * idx + K
        announce("f8 exact", M, N, K, afmt, bfmt, out, "config", config)
        a, b, xa, xb, _, _ = make_f8_inputs(M, N, K, afmt, bfmt, "ints", seed, block_scales=True, spread=spread)
        sa, sb = pow2_scales(M, seed), pow2_scales(N, seed + 1)
        c = gpu_f8(tdg, a, b, afmt, bfmt, xa, xb, sa, sb, out=out, config=config)
        ref = oracle.gemm_f8(a, b, afmt, bfmt, xa=xa, xb=xb, sa=sa, sb=sb)
        check_exact(c, ref, out, "f8 %dx%dx%d %s.%s" % (M, N, K, afmt, bfmt))


@pytest.mark.parametrize("config", [0, 1])
@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (256, 512, 4096), (520, 130, 2048)])
def test_f8_random_tolerance(tdg, M, N, K, config):
    for idx, (afmt, bfmt) in enumerate(FMTS):
        out = ["bf16", "f32", "f16", "bf16"][idx]
        seed = 2000 + 10 * idx + K
        announce("f8 random", M, N, K, afmt, bfmt, out, "config", config)
        a, b, xa, xb, sa, sb = make_f8_inputs(M, N, K, afmt, bfmt, "normal", seed, block_scales=True, spread=4,
                                              row_scales=True)
        c = gpu_f8(tdg, a, b, afmt, bfmt, xa, xb, sa, sb, out=out, config=config)
        ref = oracle.gemm_f8(a, b, afmt, bfmt, xa=xa, xb=xb, sa=sa, sb=sb)
        check_tol(c, ref, out, K, "f8 %dx%dx%d %s.%s" % (M, N, K, afmt, bfmt))


@pytest.mark.parametrize("which", ["none", "a_only", "b_only", "tensor_scales"])
def test_f8_scale_variants_exact(tdg, which):
    M, N, K = 200, 300, 1040
    announce("f8 scales", which)
    a, b, xa, xb, _, _ = make_f8_inputs(M, N, K, "e4m3", "e4m3", "ints", 77, block_scales=True, spread=1)
    sa = sb = None
    if which == "none":
        xa = xb = None
    elif which == "a_only":
        xb = None
    elif which == "b_only":
        xa = None
    else:
        xa = xb = None
        sa, sb = np.float32([0.5]), np.float32([4.0])
    c = gpu_f8(tdg, a, b, "e4m3", "e4m3", xa, xb, sa, sb, out="f32")
    ref = oracle.gemm_f8(a, b, "e4m3", "e4m3", xa=xa, xb=xb, sa=sa, sb=sb)
    check_exact(c, ref, "f32", "f8 scales " + which)


@pytest.mark.parametrize("config", [0, 1])
def test_f8_transposed_store_exact(tdg, config):
    M, N, K = 300, 260, 1040
    announce("f8 transc", config)
    a, b, xa, xb, _, _ = make_f8_inputs(M, N, K, "e5m2", "e4m3", "ints", 78, block_scales=True, spread=1)
    sa, sb = pow2_scales(M, 5), pow2_scales(N, 6)
    c = gpu_f8(tdg, a, b, "e5m2", "e4m3", xa, xb, sa, sb, out="bf16", transc=True, config=config)
    assert tuple(c.shape) == (N, M)
    ref = oracle.gemm_f8(a, b, "e5m2", "e4m3", xa=xa, xb=xb, sa=sa, sb=sb)
    check_exact(c, ref.T.copy(), "bf16", "f8 transc")


def test_f8_k_edges_and_degenerate(tdg):
    # K = 16: one partial K tile and a single block; K tails within a
    # 32-element block and within a K tile; K = 0: zeros
    for K in (16, 48, 144, 272, 400, 1040):
        announce("f8 K edge", K)
        a, b, xa, xb, _, _ = make_f8_inputs(70, 290, K, "e4m3", "e5m2", "ints", 79 + K, block_scales=True, spread=1)
        c = gpu_f8(tdg, a, b, "e4m3", "e5m2", xa, xb, out="f32")
        check_exact(c, oracle.gemm_f8(a, b, "e4m3", "e5m2", xa=xa, xb=xb), "f32", "K=%d" % K)
    announce("f8 K=0")
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((7, 0), dtype=torch.uint8, device="cuda")
    c = tdg.gemm_f8(a, b, a_fmt="e4m3", b_fmt="e4m3", out=torch.full((5, 7), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(c == 0)


def test_f8_output_ownership_and_strides(tdg):
    """Operands with padded rows (NaN bytes in the padding), C inside a
    NaN-filled buffer with a guard band: only C's elements change."""
    M, N, K = 260, 300, 1040
    announce("f8 ownership")
    a, b, xa, xb, _, _ = make_f8_inputs(M, N, K, "e4m3", "e4m3", "ints", 80, block_scales=True, spread=1)
    ap, _ = pad_cols(a, 64)
    bp, _ = pad_cols(b, 48)
    ad, bd = dev(ap)[:, :K], dev(bp)[:, :K]
    xap, _ = pad_cols(xa, 32)
    xad = dev(xap)[:, :xa.shape[1]]
    ldc = N + 24
    buf = torch.full((M + 3, ldc), float("nan"), device="cuda")
    out = buf[1:M + 1, :N]
    tdg.gemm_f8(ad, bd, a_fmt="e4m3", b_fmt="e4m3", block_scale_a=xad, block_scale_b=dev(pad_cols(xb, 16)[0]),
                out=out)
    torch.cuda.synchronize()
    host = buf.cpu()
    inside = torch.zeros_like(host, dtype=torch.bool)
    inside[1:M + 1, :N] = True
    assert torch.all(torch.isnan(host[~inside])), "an element outside C was written"
    check_exact(host[1:M + 1, :N].contiguous(), oracle.gemm_f8(a, b, "e4m3", "e4m3", xa=xa, xb=xb), "f32",
                "f8 strided")


def test_f8_full_size_sampled_rows(tdg):
    """The 8192^3 E4M3 product with block and row scales, bf16 output, in the
    launch configuration the library picks for it; sampled rows against the
    oracle."""
    M = N = K = 8192
    announce("f8 8192^3 sampled")
    a, b, xa, xb, sa, sb = make_f8_inputs(M, N, K, "e4m3", "e4m3", "normal", 81, block_scales=True, spread=2,
                                          row_scales=True)
    c = gpu_f8(tdg, a, b, "e4m3", "e4m3", xa, xb, sa, sb, out="bf16")
    rows = sample_rows(M)
    ref = oracle.gemm_f8(a[rows], b, "e4m3", "e4m3", xa=xa[rows], xb=xb, sa=sa[rows], sb=sb)
    check_tol(c[torch.from_numpy(rows)], ref, "bf16", K, "f8 8192 sampled")


def test_f8_determinism(tdg):
    M, N, K = 1000, 1000, 2048
    announce("f8 determinism")
    a, b, xa, xb, sa, sb = make_f8_inputs(M, N, K, "e4m3", "e5m2", "normal", 82, block_scales=True, spread=3,
                                          row_scales=True)
    c1 = gpu_f8(tdg, a, b, "e4m3", "e5m2", xa, xb, sa, sb, out="f32")
    c2 = gpu_f8(tdg, a, b, "e4m3", "e5m2", xa, xb, sa, sb, out="f32")
    assert torch.equal(c1, c2)
    assert np.isfinite(to_f64(c1)).all()


@pytest.mark.parametrize("config", [0, 1])
@pytest.mark.parametrize("scaled", [False, True])
def test_f8_ieee_special_values(tdg, config, scaled):
    """NaN and infinities in 8-bit operands reach C as the oracle says: an
    E4M3 NaN (S.1111.111) in A makes its row NaN; E5M2 infinities in B make
    their column of C signed infinities (NaN where the A entry is 0); with
    and without block and row scales."""
    M, N, K = 96, 80, 256
    for afmt, bfmt in (("e4m3", "e5m2"), ("e5m2", "e5m2")):
        announce("f8 ieee", afmt, bfmt, "scaled" if scaled else "unscaled", "config", config)
        a, b, xa, xb, _, _ = make_f8_inputs(M, N, K, afmt, bfmt, "ints", 77, block_scales=scaled, spread=1)
        sa, sb = (pow2_scales(M, 5), pow2_scales(N, 6)) if scaled else (None, None)
        a = a.copy()
        b = b.copy()
        a[3, 10] = 0x7F                      # NaN in either format
        b[5, 20] = 0x7C                      # E5M2 +inf: column 5
        b[9, 200] = 0xFC                     # E5M2 -inf: column 9
        if afmt == "e5m2":
            a[40, 100] = 0xFC                # E5M2 -inf in A: row 40
        c = gpu_f8(tdg, a, b, afmt, bfmt, xa, xb, sa, sb, out="f32", config=config)
        ref = oracle.gemm_f8(a, b, afmt, bfmt, xa=xa, xb=xb, sa=sa, sb=sb)
        assert np.isnan(ref[3]).all() and np.isinf(ref[:, 5]).any() and np.isinf(ref[:, 9]).any()
        check_exact(c, ref, "f32", "f8 ieee %s.%s" % (afmt, bfmt))
