"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.

This module holds only input generation: shapes, seeds and value
distributions.  It performs none of the product's arithmetic, and both the
GPU library and the CPU oracle receive exactly the bit patterns made here
(generated once on the host, rounded once to fp16/bf16 by torch's
round-to-nearest-even conversion).

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; draw A, then B, in
float32 from the stated distribution; convert to the input dtype.
  uniform  U[-1, 1)  (``2*rand - 1``)
  ints     integers uniform in {-2, ..., 2}
  normal   N(0, 1)
  normal_k N(0, 1) / sqrt(K)
Batched operands are drawn as one (batch, rows, cols) tensor.

8-bit operands (``make_f8_inputs``): A (M x K) then B (N x K) drawn as above
and converted by torch to float8_e4m3fn / float8_e5m2 (round to nearest even);
then, when asked for, the E8M0 block-scale bytes of A and of B, uniform
integers in [127 - spread, 127 + spread], and the float32 row scales of A and
of B, uniform in [0.5, 2).
"""
from dataclasses import dataclass
import math

import numpy as np
import torch

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
F8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@dataclass(frozen=True)
class Workload:
    name: str
    layout: str          # "nn": B is K x N; "tn": B is N x K and C = A B^T
    in_dtype: str        # "f16" | "bf16"
    out_dtype: str       # "f16" | "bf16" | "f32"
    M: int
    N: int
    K: int
    batch: int           # 0 = not batched
    dist: str
    seed: int
    exact: bool = False  # integer inputs: results must match bit for bit

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * max(1, self.batch)

    def describe(self) -> str:
        b = "%dx " % self.batch if self.batch else ""
        return "%s%s %s %dx%dx%d %s->%s" % (b, self.layout.upper(), self.in_dtype, self.M, self.N,
                                             self.K, self.dist, self.out_dtype)


# The five workloads of the method's test plan (the last split in two).
WORKLOADS = {
    # The worked 128x192 . 192x256 example with 64^3 tiles (2 x 4 tiles, 3 K steps).
    "worked_128x256x192": Workload("worked_128x256x192", "nn", "f16", "f16", 128, 256, 192, 0, "uniform", 1),
    # TN exactness: small integers, fp32 output, bit-exact.
    "tn_exact_1024": Workload("tn_exact_1024", "tn", "f16", "f32", 1024, 1024, 1024, 0, "ints", 2, exact=True),
    "nn_f16_4096": Workload("nn_f16_4096", "nn", "f16", "f16", 4096, 4096, 4096, 0, "normal_k", 3),
    # Headline peak-fraction workload.
    "nn_bf16_8192": Workload("nn_bf16_8192", "nn", "bf16", "bf16", 8192, 8192, 8192, 0, "normal", 4),
    # Ragged edge tiles in every dimension.
    "nn_f16_ragged_4095x5000x3000": Workload("nn_f16_ragged_4095x5000x3000", "nn", "f16", "f16",
                                             4095, 5000, 3000, 0, "uniform", 51),
    # Batched QK^T-shaped TN product, fp32 output (HBM-bound on the output).
    "tn_f16_batched_32x2048x2048x128": Workload("tn_f16_batched_32x2048x2048x128", "tn", "f16", "f32",
                                                2048, 2048, 128, 32, "normal", 52),
}


def _draw(gen: torch.Generator, shape, dist: str, K: int) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    if dist == "ints":
        return torch.randint(-2, 3, shape, generator=gen, dtype=torch.int64).to(torch.float32)
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    if dist == "normal_k":
        return torch.randn(shape, generator=gen, dtype=torch.float32) / math.sqrt(K)
    if dist == "ones":
        return torch.ones(shape, dtype=torch.float32)
    raise ValueError("unknown distribution %r" % dist)


def make_inputs(M: int, N: int, K: int, layout: str = "nn", in_dtype: str = "f16",
                dist: str = "uniform", seed: int = 0, batch: int = 0):
    """Return (A, B) as CPU tensors of ``in_dtype``: A is (batch?, M, K); B is
    (batch?, K, N) for NN or (batch?, N, K) for TN."""
    gen = torch.Generator("cpu")
    gen.manual_seed(seed)
    lead = (batch,) if batch else ()
    a_shape = lead + (M, K)
    b_shape = lead + ((K, N) if layout == "nn" else (N, K))
    a = _draw(gen, a_shape, dist, K).to(TORCH_DTYPE[in_dtype])
    b = _draw(gen, b_shape, dist, K).to(TORCH_DTYPE[in_dtype])
    return a, b


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.N, w.K, w.layout, w.in_dtype, w.dist, w.seed, w.batch)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of an fp16/bf16 CPU tensor as numpy uint16."""
    t = t.detach().cpu().contiguous()
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("expected fp16/bf16, got %s" % t.dtype)
    return t.view(torch.int16).numpy().view(np.uint16)


def sample_rows(M: int, band: int = 256, extra: int = 64, seed: int = 12345) -> np.ndarray:
    """Deterministic row sample for products too large to check whole: the
    first and last row of every ``band``-row band plus ``extra`` seeded rows."""
    rows = set()
    for start in range(0, M, band):
        rows.add(start)
        rows.add(min(start + band, M) - 1)
    rng = np.random.default_rng(seed)
    rows.update(int(r) for r in rng.integers(0, M, size=extra))
    return np.array(sorted(rows), dtype=np.int64)


def make_f8_inputs(M: int, N: int, K: int, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                   dist: str = "normal", seed: int = 0, block_scales: bool = False, spread: int = 4,
                   row_scales: bool = False, block: int = 32):
    """8-bit TN operands as numpy uint8 bit patterns: A (M, K), B (N, K); block
    scales xa (M, cdiv(K, block)), xb (N, cdiv(K, block)) or None; row scales
    sa (M,), sb (N,) float32 or None."""
    gen = torch.Generator("cpu")
    gen.manual_seed(seed)
    a = _draw(gen, (M, K), dist, K).to(F8_TORCH[a_fmt]).view(torch.uint8).numpy().copy()
    b = _draw(gen, (N, K), dist, K).to(F8_TORCH[b_fmt]).view(torch.uint8).numpy().copy()
    xa = xb = sa = sb = None
    nb = (K + block - 1) // block
    if block_scales:
        xa = torch.randint(127 - spread, 128 + spread, (M, nb), generator=gen).to(torch.uint8).numpy()
        xb = torch.randint(127 - spread, 128 + spread, (N, nb), generator=gen).to(torch.uint8).numpy()
    if row_scales:
        sa = (torch.rand((M,), generator=gen) * 1.5 + 0.5).numpy()
        sb = (torch.rand((N,), generator=gen) * 1.5 + 0.5).numpy()
    return a, b, xa, xb, sa, sb


@dataclass(frozen=True)
class F8Workload:
    name: str
    M: int
    N: int
    K: int
    a_fmt: str           # "e4m3" | "e5m2"
    b_fmt: str
    out_dtype: str       # "f16" | "bf16" | "f32"
    block_scales: bool   # E8M0 scales per row and 32-element K block
    row_scales: bool     # fp32 scales per row of A and of B
    dist: str
    seed: int
    spread: int = 4

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# 8-bit TN products (C = A B^T with scales), measured beside the 16-bit ones.
F8_WORKLOADS = {
    "tn_e4m3_8192_blockscaled": F8Workload("tn_e4m3_8192_blockscaled", 8192, 8192, 8192, "e4m3", "e4m3", "bf16",
                                           True, True, "normal", 83),
    "tn_e4m3_8192": F8Workload("tn_e4m3_8192", 8192, 8192, 8192, "e4m3", "e4m3", "bf16", False, False,
                               "normal", 84),
}


def f8_workload_inputs(w: F8Workload):
    return make_f8_inputs(w.M, w.N, w.K, w.a_fmt, w.b_fmt, w.dist, w.seed, block_scales=w.block_scales,
                          spread=w.spread, row_scales=w.row_scales)
