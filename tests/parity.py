"""Helpers for GPU-vs-oracle parity tests (not a test module itself).

The GPU side is called only through the C ABI (via the ``tiled_dense_gemm_03_amd``
binding); the reference side only through ``oracle``.  Both receive the same
host-generated fp16/bf16 bit patterns.

Comparison rules:
  exact   integer inputs: every product and partial sum is an integer far
          below 2^24, so the fp32 accumulator holds the exact sum and the one
          output rounding (RNE) must equal the oracle's exact sum encoded by
          the oracle's own RNE encoder -- bit for bit (+0 and -0 compare equal).
  fp16/bf16 output, random inputs:
          max|C_gpu - C_ref| <= 1e-2 * sqrt(K/1024) * max|C_ref| + 1e-3
  fp32 output, random inputs:
          max|C_gpu - C_ref| / max|C_ref| <= 1e-5 * sqrt(K)
  with C_ref the unrounded binary64 oracle value.
"""
import math

import numpy as np
import torch

from oracle import oracle
from workloads import bits

OUT_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def to_f64(c: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a CPU fp16/bf16/fp32 tensor."""
    c = c.detach().cpu().contiguous()
    if c.dtype == torch.float32:
        return c.numpy().astype(np.float64)
    if c.dtype == torch.float16:
        return c.view(torch.int16).numpy().view(np.uint16).view(np.float16).astype(np.float64)
    if c.dtype == torch.bfloat16:
        u = c.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise TypeError(c.dtype)


def ref_gemm(a, b, in_dtype, layout, rows=None):
    return oracle.gemm(bits(a), bits(b), in_dtype, layout, rows=rows)


def check_exact(c_gpu: torch.Tensor, ref: np.ndarray, out_dtype: str, what=""):
    got = to_f64(c_gpu)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if out_dtype == "f32":
        expect = ref.astype(np.float32).astype(np.float64)
        assert np.array_equal(expect, ref, equal_nan=True), "reference not exactly representable in fp32"
    else:
        expect = oracle.decode(oracle.encode(ref, out_dtype), out_dtype)
    bad = ~((got == expect) | (np.isnan(got) & np.isnan(expect)))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements differ; first %s: gpu %s vs expected %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(), got[tuple(idx.T)], expect[tuple(idx.T)]))


def tolerance(out_dtype: str, K: int, ref_absmax: float) -> float:
    if out_dtype == "f32":
        return 1e-5 * math.sqrt(K) * ref_absmax
    return 1e-2 * math.sqrt(K / 1024.0) * ref_absmax + 1e-3


def check_tol(c_gpu: torch.Tensor, ref: np.ndarray, out_dtype: str, K: int, what=""):
    got = to_f64(c_gpu)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    amax = float(np.max(np.abs(ref))) if ref.size else 0.0
    tol = tolerance(out_dtype, K, amax)
    assert err <= tol, "%s: max abs error %.3e > tolerance %.3e (max|ref| %.3e)" % (what, err, tol, amax)
    return err, tol
