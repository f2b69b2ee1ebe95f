"""Pins of the CPU oracle's 8-bit path (decoders and the scaled product).

Everything here runs on the CPU.  The oracle's decoders are pinned to torch's
float8_e4m3fn / float8_e5m2 conversions (an independent implementation of the
same OCP formats) and to points fixed by the format definitions; the scaled
product is pinned to torch matrix products of independently decoded operands,
to closed forms of special scale patterns, and to symmetry.

Exactness: an E4M3 / E5M2 product has at most 8 significant bits and the
products of two such values span at most 2^-32 .. 2^31, so every partial sum of
a few thousand of them is exact in binary64 whatever the order; the unscaled
comparisons below are therefore equalities.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle
from workloads import F8_TORCH, make_f8_inputs


def torch_decode(bits: np.ndarray, fmt: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(F8_TORCH[fmt]).to(torch.float64)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_all_patterns_match_torch(fmt):
    allb = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_f8(allb, fmt)
    theirs = torch_decode(allb, fmt).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(theirs))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], theirs[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(theirs[ok]))


def test_decode_definition_points():
    e4 = lambda b: float(oracle.decode_f8(np.array([b], np.uint8), "e4m3")[0])  # noqa: E731
    e5 = lambda b: float(oracle.decode_f8(np.array([b], np.uint8), "e5m2")[0])  # noqa: E731
    # E4M3: bias 7, 3 fraction bits, only S.1111.111 is NaN
    assert e4(0x38) == 1.0 and e4(0x40) == 2.0 and e4(0xB8) == -1.0
    assert e4(0x7E) == 448.0 and e4(0xFE) == -448.0          # largest finite
    assert e4(0x78) == 256.0                                   # all-ones exponent is a normal binade
    assert math.isnan(e4(0x7F)) and math.isnan(e4(0xFF))
    assert e4(0x01) == 2.0 ** -9 and e4(0x07) == 7 * 2.0 ** -9  # subnormals
    assert e4(0x08) == 2.0 ** -6                               # smallest normal
    assert e4(0x80) == 0.0 and math.copysign(1.0, e4(0x80)) == -1.0
    # E5M2: bias 15, 2 fraction bits, binary16-like specials
    assert e5(0x3C) == 1.0 and e5(0x7B) == 57344.0
    assert e5(0x7C) == math.inf and e5(0xFC) == -math.inf
    assert all(math.isnan(e5(b)) for b in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert e5(0x01) == 2.0 ** -16 and e5(0x03) == 3 * 2.0 ** -16 and e5(0x04) == 2.0 ** -14
    # positive patterns are strictly increasing up to the largest finite value
    for fmt, top in (("e4m3", 0x7E), ("e5m2", 0x7B)):
        v = oracle.decode_f8(np.arange(top + 1, dtype=np.uint8), fmt)
        assert np.all(np.diff(v) > 0)


def test_decode_e8m0():
    allb = np.arange(256, dtype=np.uint8)
    v = oracle.decode_e8m0(allb)
    assert math.isnan(v[255])
    assert np.array_equal(v[:255], np.ldexp(1.0, np.arange(255) - 127))


@pytest.mark.parametrize("afmt,bfmt", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_unscaled_product_equals_torch_matmul(afmt, bfmt):
    a, b, *_ = make_f8_inputs(37, 29, 200, afmt, bfmt, "normal", seed=11)
    ref = (torch_decode(a, afmt) @ torch_decode(b, bfmt).T).numpy()
    got = oracle.gemm_f8(a, b, afmt, bfmt)
    assert np.array_equal(got, ref)


def test_uniform_block_scales_are_powers_of_two():
    a, b, *_ = make_f8_inputs(16, 24, 96, seed=12)
    base = oracle.gemm_f8(a, b, "e4m3", "e4m3")
    xa = np.full((16, 3), 127 + 3, np.uint8)
    xb = np.full((24, 3), 127 - 5, np.uint8)
    assert np.array_equal(oracle.gemm_f8(a, b, "e4m3", "e4m3", xa=xa, xb=xb), base * 2.0 ** -2)


@pytest.mark.parametrize("K,block", [(100, 32), (96, 32), (64, 16), (40, 64)])
def test_one_scaled_block(K, block):
    """Raising one block's scale adds (2^e - 1) times that block's own product:
    a wrong block index, block length or ragged last block fails this."""
    M, N = 9, 7
    a, b, *_ = make_f8_inputs(M, N, K, "e4m3", "e5m2", "normal", seed=13)
    nb = -(-K // block)
    ta, tb = torch_decode(a, "e4m3"), torch_decode(b, "e5m2")
    base = (ta @ tb.T).numpy()
    for t in range(nb):
        for side in ("a", "b"):
            xa = np.full((M, nb), 127, np.uint8)
            xb = np.full((N, nb), 127, np.uint8)
            (xa if side == "a" else xb)[:, t] = 127 + 4
            got = oracle.gemm_f8(a, b, "e4m3", "e5m2", xa=xa, xb=xb, block=block)
            k0, k1 = t * block, min((t + 1) * block, K)
            part = (ta[:, k0:k1] @ tb[:, k0:k1].T).numpy()
            assert np.array_equal(got, base + 15.0 * part), (t, side)


def test_block_scales_equal_per_element_scaling():
    """The block-scaled sum equals the plain product of operands whose every
    element is multiplied by its block's scale (the scale distributes over
    the block's sum)."""
    M, N, K = 20, 12, 160
    a, b, xa, xb, *_ = make_f8_inputs(M, N, K, "e4m3", "e4m3", "normal", seed=14, block_scales=True)
    fa = torch.from_numpy(oracle.decode_e8m0(xa)).repeat_interleave(32, dim=1)[:, :K]
    fb = torch.from_numpy(oracle.decode_e8m0(xb)).repeat_interleave(32, dim=1)[:, :K]
    ref = ((torch_decode(a, "e4m3") * fa) @ (torch_decode(b, "e4m3") * fb).T).numpy()
    got = oracle.gemm_f8(a, b, "e4m3", "e4m3", xa=xa, xb=xb)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # and the scales matter: without them the result differs
    assert not np.allclose(oracle.gemm_f8(a, b, "e4m3", "e4m3"), ref)


def test_row_scales_and_tensor_scale():
    M, N, K = 11, 13, 64
    a, b, _, _, sa, sb = make_f8_inputs(M, N, K, seed=15, row_scales=True)
    base = oracle.gemm_f8(a, b, "e4m3", "e4m3")
    got = oracle.gemm_f8(a, b, "e4m3", "e4m3", sa=sa, sb=sb)
    ref = sa.astype(np.float64)[:, None] * base * sb.astype(np.float64)[None, :]
    assert np.allclose(got, ref, rtol=1e-15, atol=0)
    one = oracle.gemm_f8(a, b, "e4m3", "e4m3", sa=np.float32([0.75]), sb=np.float32([2.0]))
    assert np.array_equal(one, base * 1.5)


def test_transpose_symmetry():
    M, N, K = 14, 10, 130
    a, b, xa, xb, sa, sb = make_f8_inputs(M, N, K, "e5m2", "e4m3", seed=16, block_scales=True,
                                          row_scales=True)
    c1 = oracle.gemm_f8(a, b, "e5m2", "e4m3", xa=xa, xb=xb, sa=sa, sb=sb)
    c2 = oracle.gemm_f8(b, a, "e4m3", "e5m2", xa=xb, xb=xa, sa=sb, sb=sa)
    # equal up to the order of the two row-scale multiplications (one rounding)
    assert np.allclose(c1, c2.T, rtol=4e-16, atol=0)
    c3 = oracle.gemm_f8(a, b, "e5m2", "e4m3", xa=xa, xb=xb)
    c4 = oracle.gemm_f8(b, a, "e4m3", "e5m2", xa=xb, xb=xa)
    assert np.array_equal(c3, c4.T)


def test_brute_force_tiny():
    """A few entries written out term by term with math.ldexp."""
    M, N, K = 3, 2, 70
    a, b, xa, xb, sa, sb = make_f8_inputs(M, N, K, "e4m3", "e5m2", "normal", seed=17,
                                          block_scales=True, row_scales=True)
    av, bv = torch_decode(a, "e4m3").tolist(), torch_decode(b, "e5m2").tolist()
    got = oracle.gemm_f8(a, b, "e4m3", "e5m2", xa=xa, xb=xb, sa=sa, sb=sb)
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += math.ldexp(av[i][k] * bv[j][k], int(xa[i, k // 32]) + int(xb[j, k // 32]) - 254)
            s *= float(sa[i]) * float(sb[j])
            assert math.isclose(got[i, j], s, rel_tol=1e-13, abs_tol=1e-300)


def test_nan_input_and_degenerate_sizes():
    a, b, *_ = make_f8_inputs(4, 5, 32, seed=18)
    a = a.copy()
    a[2, 7] = 0x7F                                  # E4M3 NaN
    c = oracle.gemm_f8(a, b, "e4m3", "e4m3")
    assert np.all(np.isnan(c[2])) and not np.any(np.isnan(np.delete(c, 2, axis=0)))
    z = oracle.gemm_f8(np.zeros((3, 0), np.uint8), np.zeros((4, 0), np.uint8), "e4m3", "e4m3")
    assert z.shape == (3, 4) and np.all(z == 0)
    assert oracle.gemm_f8(np.zeros((0, 8), np.uint8), np.zeros((4, 8), np.uint8), "e4m3", "e4m3").shape == (0, 4)
    with pytest.raises(ValueError):
        oracle.gemm_f8(a, b[:, :16], "e4m3", "e4m3")
    with pytest.raises(KeyError):
        oracle.gemm_f8(a, b, "e3m4", "e4m3")
