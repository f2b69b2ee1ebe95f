"""Pins of the oracle's GEMM against what the pages and mathematics fix.

Each pin is chosen so that a plausible slip in the oracle fails it:
  * the worked 128x192 . 192x256 example with 64^3 tiles, the traced read of
    program (1, 2) at K step 1, the BK = 32 variant and the 65 x 97 x 130 tail
    case (NineToothed GEMM primer, s1, s3, s4, s5, s8) -- wrong grid, wrong
    K-step count, wrong slice or wrong mask;
  * all-ones over the tail case gives K everywhere, and dropping the last K
    tile (a mistake planted in the oracle's tiled path) gives 128 -- a
    dropped term;
  * the 2048 + 1 + 1 example (s6) -- accumulator precision;
  * identities and permutations (one nonzero product per output) -- a
    transposed or mis-indexed operand;
  * an asymmetric closed form sum_p (i + 2p)(3p + j + 1) -- a wrong sign,
    index or operand order;
  * brute force over every shape in {1..4}^3 against numpy's float64 einsum,
    and random products against numpy's float64 matmul -- anything else.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import oracle
from workloads import bits, make_inputs


def f16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def dec(b, fmt="f16"):
    if fmt == "f16":
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Worked example, traced read, BK = 32, tails (NineToothed GEMM primer)
# --------------------------------------------------------------------------

def test_worked_example_grid_and_ksteps(golden):
    w = golden["worked_example"]
    g = oracle.tile_geometry(w["M"], w["N"], w["K"], w["BM"], w["BN"], w["BK"])
    assert list(g["grid"]) == w["grid"]
    assert g["ksteps"] == w["ksteps"] == w["A_layers"][1][0] == w["B_layers"][1][0]
    assert g["grid"][0] * g["grid"][1] == w["programs"]
    assert list(w["C_layers"][0]) == list(g["grid"])
    (r0, r1), (c0, c1) = g["a_nominal"]
    assert [r1 - r0, c1 - c0] == w["A_layers"][2]
    (r0, r1), (c0, c1) = g["b_nominal"]
    assert [r1 - r0, c1 - c0] == w["B_layers"][2]
    (r0, r1), (c0, c1) = g["c_nominal"]
    assert [r1 - r0, c1 - c0] == w["C_layers"][1]
    # Before the squeeze, program (i, j) holds one block row of A across all K
    # tiles and all K tiles of one block column of B.
    assert w["A_unsqueezed_group"] == [1, g["ksteps"]]
    assert w["B_unsqueezed_group"] == [g["ksteps"], 1]


def test_traced_read(golden):
    t = golden["traced_read"]
    w = golden["worked_example"]
    g = oracle.tile_geometry(w["M"], w["N"], w["K"], w["BM"], w["BN"], w["BK"], t["i"], t["j"], t["p"])
    assert [list(x) for x in g["c_valid"]] == [t["C_rows"], t["C_cols"]]
    assert [list(x) for x in g["a_valid"]] == [t["A_rows"], t["A_cols"]]
    assert [list(x) for x in g["b_valid"]] == [t["B_rows"], t["B_cols"]]


def test_traced_read_partial_sum_is_the_slice_product(golden):
    """The oracle's full product restricted to the traced output tile equals
    the sum over K tiles of the slice products the page names; the p = 1 term
    is exactly A[64:128, 64:128] @ B[64:128, 128:192]."""
    w = golden["worked_example"]
    a, b = make_inputs(w["M"], w["N"], w["K"], "nn", "f16", "ints", seed=101)
    A, B = dec(bits(a)), dec(bits(b))
    C = oracle.gemm(bits(a), bits(b), "f16", "nn")
    parts = [A[64:128, p * 64:(p + 1) * 64] @ B[p * 64:(p + 1) * 64, 128:192] for p in range(3)]
    assert np.array_equal(C[64:128, 128:192], parts[0] + parts[1] + parts[2])
    # a tiled run over only the first two K tiles misses exactly the p = 2 part
    t = oracle.tiled_gemm(bits(a), bits(b), "f16", "nn", 64, 64, 64, drop_last_k=True)
    assert np.array_equal(t[64:128, 128:192], parts[0] + parts[1])


def test_bk32_variant(golden):
    v = golden["bk32"]
    g = oracle.tile_geometry(v["M"], v["N"], v["K"], v["BM"], v["BN"], v["BK"])
    assert list(g["grid"]) == v["grid"] and g["ksteps"] == v["ksteps"]
    (r0, r1), (c0, c1) = g["a_nominal"]
    assert [r1 - r0, c1 - c0] == v["A_tile"]
    (r0, r1), (c0, c1) = g["b_nominal"]
    assert [r1 - r0, c1 - c0] == v["B_tile"]
    (r0, r1), (c0, c1) = g["c_nominal"]
    assert [r1 - r0, c1 - c0] == v["C_tile"]


def test_tail_geometry(golden):
    t = golden["tails"]
    g = oracle.tile_geometry(t["M"], t["N"], t["K"], t["BM"], t["BN"], t["BK"], 1, 1, t["ksteps"] - 1)
    assert list(g["grid"]) == t["grid"] and g["ksteps"] == t["ksteps"]
    assert list(g["a_nominal"][1]) == t["last_k_tile_nominal"]
    assert list(g["a_valid"][1]) == t["last_k_tile_valid"]
    assert list(g["b_valid"][0]) == t["last_k_tile_valid"]
    (r0, r1), (c0, c1) = g["c_valid"]
    assert [r1 - r0, c1 - c0] == t["corner_tile_valid_shape"]


def test_tail_store_mask_leaves_outside_untouched(golden):
    """Under the store mask only real elements are written; a sentinel frame
    around the matrix (C held in a larger buffer) is never touched."""
    t = golden["tails"]
    M, N, K = t["M"], t["N"], t["K"]
    a = f16_bits(np.ones((M, K)))
    b = f16_bits(np.ones((K, N)))
    c = oracle.tiled_gemm(a, b, "f16", "nn", 64, 64, 64, c_init=np.full((M, N), -7.0))
    assert np.all(c == K)


def test_all_ones_tail_case_and_dropped_last_tile(golden):
    o = golden["all_ones"]
    M, N, K = o["M"], o["N"], o["K"]
    a = f16_bits(np.ones((M, K)))
    b = f16_bits(np.ones((K, N)))
    plain = oracle.gemm(a, b, "f16", "nn")
    assert plain.shape == (M, N) and np.all(plain == o["value"])
    tiled = oracle.tiled_gemm(a, b, "f16", "nn", 64, 64, 64, acc="f32", out="f16")
    assert np.all(tiled == o["value"])
    # Negative control: the planted mistake must be visible.
    broken = oracle.tiled_gemm(a, b, "f16", "nn", 64, 64, 64, acc="f32", out="f16", drop_last_k=True)
    assert np.all(broken == o["value_if_last_k_tile_dropped"])
    # TN with B stored N x K gives the same.
    tn = oracle.gemm(a, f16_bits(np.ones((N, K))), "f16", "tn")
    assert np.all(tn == o["value"])


def test_fp32_accumulation_example(golden):
    e = golden["fp32_accumulation"]
    a = f16_bits(np.array([e["terms"]], dtype=np.float64))     # 1 x 3
    b = f16_bits(np.ones((3, 1)))                              # 3 x 1
    c16 = oracle.tiled_gemm(a, b, "f16", "nn", 64, 64, 64, acc="f16")
    c32 = oracle.tiled_gemm(a, b, "f16", "nn", 64, 64, 64, acc="f32", out="f16")
    assert c16[0, 0] == e["fp16_accumulator_steps"][-1]
    assert c32[0, 0] == e["fp32_accumulator_steps"][-1] == e["final_fp16_output_from_fp32_accumulator"]
    # every prefix of the sum, to see each intermediate step of the example
    for n in (1, 2, 3):
        p16 = oracle.tiled_gemm(a[:, :n], b[:n], "f16", "nn", 64, 64, 64, acc="f16")
        p32 = oracle.tiled_gemm(a[:, :n], b[:n], "f16", "nn", 64, 64, 64, acc="f32")
        assert p16[0, 0] == e["fp16_accumulator_steps"][n - 1]
        assert p32[0, 0] == e["fp32_accumulator_steps"][n - 1]
    assert oracle.gemm(a, b, "f16", "nn")[0, 0] == 2050.0


# --------------------------------------------------------------------------
# Tiled program == plain definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("shape,tile", [((128, 256, 192), (64, 64, 64)),
                                        ((128, 256, 192), (64, 64, 32)),
                                        ((65, 97, 130), (64, 64, 64)),
                                        ((33, 17, 70), (16, 32, 8))])
def test_tiled_equals_plain(layout, shape, tile):
    M, N, K = shape
    ai, bi = make_inputs(M, N, K, layout, "f16", "ints", seed=5)
    exact_p = oracle.gemm(bits(ai), bits(bi), "f16", layout)
    exact_t = oracle.tiled_gemm(bits(ai), bits(bi), "f16", layout, *tile)
    assert np.array_equal(exact_p, exact_t)
    af, bf = make_inputs(M, N, K, layout, "bf16", "uniform", seed=6)
    p = oracle.gemm(bits(af), bits(bf), "bf16", layout)
    t = oracle.tiled_gemm(bits(af), bits(bf), "bf16", layout, *tile)
    assert np.max(np.abs(p - t)) <= 1e-12 * max(1.0, np.max(np.abs(p)))


# --------------------------------------------------------------------------
# Identities, permutations, closed form
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,enc", [("f16", f16_bits), ("bf16", bf16_bits)])
def test_identity_and_permutation(fmt, enc):
    rng = np.random.default_rng(3)
    M, K = 37, 53
    Avals = rng.uniform(-1, 1, (M, K))
    A = enc(Avals)
    I = enc(np.eye(K))
    # NN: A . I == A (exact: one nonzero product per output)
    assert np.array_equal(oracle.gemm(A, I, fmt, "nn"), dec(A, fmt))
    # TN: A . I^T == A
    assert np.array_equal(oracle.gemm(A, I, fmt, "tn"), dec(A, fmt))
    # P . B permutes rows of B; A . P permutes columns of A
    perm = rng.permutation(K)
    P = np.zeros((K, K)); P[np.arange(K), perm] = 1.0
    B = enc(rng.uniform(-1, 1, (K, 29)))
    assert np.array_equal(oracle.gemm(enc(P), B, fmt, "nn"), dec(B, fmt)[perm])
    assert np.array_equal(oracle.gemm(A, enc(P), fmt, "nn"), dec(A, fmt)[:, np.argsort(perm)])
    # TN with B = P (stored N x K): C[i, j] = A[i, perm[j]]
    assert np.array_equal(oracle.gemm(A, enc(P), fmt, "tn"), dec(A, fmt)[:, perm])


def closed_form(M, N, K):
    """sum_{p<K} (i + 2p)(3p + j + 1) = 3i S1 + K i (j+1) + 6 S2 + 2 (j+1) S1,
    S1 = K(K-1)/2, S2 = (K-1)K(2K-1)/6."""
    i = np.arange(M)[:, None].astype(np.float64)
    j = np.arange(N)[None, :].astype(np.float64)
    S1 = K * (K - 1) / 2
    S2 = (K - 1) * K * (2 * K - 1) / 6
    return 3 * i * S1 + K * i * (j + 1) + 6 * S2 + 2 * (j + 1) * S1


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_closed_form(layout):
    M, N, K = 23, 31, 40
    i = np.arange(M)[:, None]; p = np.arange(K)[None, :]
    A = f16_bits(i + 2 * p)                      # M x K, values <= 100: exact in fp16
    Bkn = (3 * np.arange(K)[:, None] + np.arange(N)[None, :] + 1).astype(np.float64)   # K x N
    B = f16_bits(Bkn if layout == "nn" else Bkn.T)
    C = oracle.gemm(A, B, "f16", layout)
    assert np.array_equal(C, closed_form(M, N, K))
    # the symmetric form of the method's test plan: A = i + p, B = p + j
    A2 = f16_bits(i + p)
    B2kn = (np.arange(K)[:, None] + np.arange(N)[None, :]).astype(np.float64)
    C2 = oracle.gemm(A2, f16_bits(B2kn if layout == "nn" else B2kn.T), "f16", layout)
    ii, jj = np.arange(M)[:, None], np.arange(N)[None, :]
    ref2 = K * ii * jj + (ii + jj) * K * (K - 1) / 2 + (K - 1) * K * (2 * K - 1) / 6
    assert np.array_equal(C2, ref2)


# --------------------------------------------------------------------------
# Brute force and library routine
# --------------------------------------------------------------------------

def test_brute_force_all_tiny_shapes():
    rng = np.random.default_rng(11)
    for M, N, K in itertools.product(range(1, 5), repeat=3):
        for layout in ("nn", "tn"):
            Av = rng.integers(-2, 3, (M, K)).astype(np.float64)
            Bv = rng.integers(-2, 3, (K, N)).astype(np.float64)
            Bstore = Bv if layout == "nn" else Bv.T
            C = oracle.gemm(f16_bits(Av), f16_bits(Bstore), "f16", layout)
            assert np.array_equal(C, np.einsum("ik,kj->ij", Av, Bv)), (M, N, K, layout)


@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_random_vs_numpy_matmul(layout, fmt):
    M, N, K = 70, 90, 300
    a, b = make_inputs(M, N, K, layout, fmt, "normal", seed=9)
    A, B = dec(bits(a), fmt), dec(bits(b), fmt)
    ref = A @ (B if layout == "nn" else B.T)
    C = oracle.gemm(bits(a), bits(b), fmt, layout)
    assert np.max(np.abs(C - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_batched_and_row_subset():
    batch, M, N, K = 3, 20, 24, 16
    a, b = make_inputs(M, N, K, "tn", "f16", "ints", seed=4, batch=batch)
    C = oracle.gemm(bits(a), bits(b), "f16", "tn")
    for z in range(batch):
        A, B = dec(bits(a)[z]), dec(bits(b)[z])
        assert np.array_equal(C[z], A @ B.T)
    rows = np.array([0, 7, 19])
    Cr = oracle.gemm(bits(a), bits(b), "f16", "tn", rows=rows)
    assert np.array_equal(Cr, C[:, rows])
    # thread count does not change any bit
    C1 = oracle.gemm(bits(a), bits(b), "f16", "tn", nthreads=1)
    C7 = oracle.gemm(bits(a), bits(b), "f16", "tn", nthreads=7)
    assert np.array_equal(C1, C7) and np.array_equal(C1, C)


def test_degenerate_sizes():
    a = np.zeros((5, 0), dtype=np.uint16)
    b = np.zeros((0, 4), dtype=np.uint16)
    C = oracle.gemm(a, b, "f16", "nn")
    assert C.shape == (5, 4) and np.all(C == 0)        # K = 0: empty sum
    C = oracle.gemm(np.zeros((0, 3), np.uint16), np.zeros((3, 4), np.uint16), "f16", "nn")
    assert C.shape == (0, 4)


def test_bad_arguments_rejected():
    import ctypes
    buf = np.zeros(64, dtype=np.uint16)
    out = np.zeros(64)
    p = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    # negative size, lda < K, unknown format
    assert oracle.gemm_raw(0, 0, -1, 2, 2, p(buf), 2, 0, p(buf), 2, 0, p(out), 2, 0, 1) != 0
    assert oracle.gemm_raw(0, 0, 2, 2, 4, p(buf), 3, 0, p(buf), 2, 0, p(out), 2, 0, 1) != 0
    assert oracle.gemm_raw(0, 7, 2, 2, 2, p(buf), 2, 0, p(buf), 2, 0, p(out), 2, 0, 1) != 0
    # explicit lda larger than K is honoured
    A = np.zeros((2, 5), np.uint16); A[:, :3] = f16_bits(np.array([[1, 2, 3], [4, 5, 6]]))
    A[:, 3:] = f16_bits(np.full((2, 2), 99.0))     # padding must not be read
    B = f16_bits(np.eye(3))
    C = np.zeros((2, 3))
    assert oracle.gemm_raw(0, 0, 2, 3, 3, p(A), 5, 0, p(B), 3, 0, p(C), 3, 0, 1) == 0
    assert np.array_equal(C, [[1, 2, 3], [4, 5, 6]])


@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_ieee_special_values_term_by_term(layout, fmt):
    """NaN and infinities in the operands: each output compared with its own
    sum of products written out term by term in Python floats (IEEE binary64:
    a NaN term or +inf plus -inf gives NaN, inf times 0 gives NaN, inf times
    a nonzero value gives a signed infinity).  A NaN dropped by a masked path,
    or an infinity cancelled by a reordered sum, fails here."""
    M, N, K = 9, 7, 12
    rng = np.random.default_rng(5)
    Av = rng.integers(-2, 3, (M, K)).astype(np.float64)
    Bv = rng.integers(-2, 3, (K, N)).astype(np.float64)
    Av[1, 3] = np.nan
    Av[4, 2] = np.inf
    Bv[2, 0] = 0.0                      # inf * 0 at (4, 0)
    Bv[2, 1:4] = [1.0, -2.0, 2.0]       # signed infinities at (4, 1..3)
    Av[6, 5], Av[6, 8] = np.inf, -np.inf
    Bv[5, :], Bv[8, :] = 1.0, 1.0       # +inf - inf across row 6
    Bv[10, 4] = np.nan                  # column 4 all NaN
    Bv[9, 6] = -np.inf
    enc = f16_bits if fmt == "f16" else bf16_bits
    Bstore = Bv if layout == "nn" else Bv.T
    C = oracle.gemm(enc(Av), enc(np.ascontiguousarray(Bstore)), fmt, layout)
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(Av[i, k]) * float(Bv[k, j])
            assert (np.isnan(s) and np.isnan(C[i, j])) or s == C[i, j], (i, j, s, C[i, j])
    assert np.isnan(C[1]).all() and np.isnan(C[:, 4]).all() and np.isnan(C[6]).all() and np.isnan(C[4, 0])
    assert np.isinf(C[4, 1:4]).all()
