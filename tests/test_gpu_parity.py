"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Covers the six workloads of the method's test plan at full size (row-sampled
where the oracle cannot do the whole product in seconds), their integer
variants bit for bit, every tile configuration on ragged shapes, strided
operands, guard bands and NaN poison in padding, degenerate sizes and
run-to-run determinism.
"""
import sys

import pytest
import torch

from parity import OUT_TORCH, check_exact, check_tol, ref_gemm
from workloads import WORKLOADS, make_inputs, sample_rows, workload_inputs

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


def gpu_gemm(tdg, a, b, layout, out_dtype, config=-1):
    ad, bd = a.cuda(), b.cuda()
    c = tdg.gemm(ad, bd, layout=layout, out_dtype=OUT_TORCH[out_dtype], config=config)
    torch.cuda.synchronize()
    return c.cpu()


# ---------------------------------------------------------------------------
# The six workloads at full size
# ---------------------------------------------------------------------------

SMALL = ["worked_128x256x192", "tn_exact_1024"]
LARGE = ["nn_f16_4096", "nn_bf16_8192", "nn_f16_ragged_4095x5000x3000", "tn_f16_batched_32x2048x2048x128"]


@pytest.mark.parametrize("name", SMALL)
def test_small_workloads_whole(tdg, name):
    w = WORKLOADS[name]
    announce(name)
    a, b = workload_inputs(w)
    c = gpu_gemm(tdg, a, b, w.layout, w.out_dtype)
    ref = ref_gemm(a, b, w.in_dtype, w.layout)
    if w.exact:
        check_exact(c, ref, w.out_dtype, name)
    else:
        check_tol(c, ref, w.out_dtype, w.K, name)


@pytest.mark.parametrize("name", LARGE)
def test_large_workloads_sampled_rows(tdg, name):
    """Full-size product in the launch configuration the benchmark times;
    the oracle computes the first and last row of every 256-row band plus 64
    seeded rows (every tile row and tile column is touched)."""
    w = WORKLOADS[name]
    announce(name)
    a, b = workload_inputs(w)
    c = gpu_gemm(tdg, a, b, w.layout, w.out_dtype)
    rows = sample_rows(w.M)
    if w.batch:
        # every problem of the batch, sampled rows of each
        ref = ref_gemm(a, b, w.in_dtype, w.layout, rows=rows)
        check_tol(c[:, rows], ref, w.out_dtype, w.K, name)
    else:
        ref = ref_gemm(a, b, w.in_dtype, w.layout, rows=rows)
        check_tol(c[rows], ref, w.out_dtype, w.K, name)


@pytest.mark.parametrize("name", ["worked_128x256x192", "nn_f16_4096", "nn_bf16_8192",
                                  "nn_f16_ragged_4095x5000x3000", "tn_f16_batched_32x2048x2048x128"])
def test_integer_variants_bit_exact(tdg, name):
    """The same shapes, layouts and dtypes with integer inputs in {-2..2}:
    the GPU result must equal the oracle's exact sum, rounded once."""
    w = WORKLOADS[name]
    announce(name, "ints")
    a, b = make_inputs(w.M, w.N, w.K, w.layout, w.in_dtype, "ints", seed=w.seed + 1000, batch=w.batch)
    c = gpu_gemm(tdg, a, b, w.layout, w.out_dtype)
    if w.M * w.N * w.K * max(1, w.batch) <= 2 ** 28:
        check_exact(c, ref_gemm(a, b, w.in_dtype, w.layout), w.out_dtype, name)
        return
    rows = sample_rows(w.M)
    ref = ref_gemm(a, b, w.in_dtype, w.layout, rows=rows)
    check_exact(c[:, rows] if w.batch else c[rows], ref, w.out_dtype, name)


# ---------------------------------------------------------------------------
# Every tile configuration on ragged shapes
# ---------------------------------------------------------------------------

# (M, N, K): tails in M, N and K; "several full K tiles then a tail"; one tile;
# fewer rows or columns than one MFMA tile.  K and N are multiples of 8 so the
# vectorised configurations apply; the predicated ones also get odd sizes.
VEC_SHAPES = [(1, 8, 8), (17, 24, 16), (33, 40, 72), (64, 64, 64), (65, 72, 200), (127, 136, 256),
              (129, 264, 136), (255, 248, 520), (257, 520, 64), (300, 8, 1032)]
PRED_SHAPES = [(1, 1, 1), (2, 3, 5), (15, 17, 31), (33, 31, 63), (65, 97, 130), (63, 129, 197),
               (130, 65, 257), (257, 255, 129)]


def _config_ids(tdg, vec):
    """Vectorised configurations (aligned operands only) or the predicated ones."""
    return [i for i in range(tdg.tdg_num_configs()) if tdg.tdg_config_name(i).endswith("_pred") != vec]


@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("in_dtype,out_dtype", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32")])
def test_every_config_integer_exact(tdg, layout, in_dtype, out_dtype):
    for vec, shapes in ((True, VEC_SHAPES), (False, VEC_SHAPES + PRED_SHAPES)):
        for cfg in _config_ids(tdg, vec):
            for (M, N, K) in shapes:
                announce(layout, in_dtype, out_dtype, tdg.tdg_config_name(cfg), M, N, K)
                a, b = make_inputs(M, N, K, layout, in_dtype, "ints", seed=M * 7 + N * 3 + K)
                c = gpu_gemm(tdg, a, b, layout, out_dtype, config=cfg)
                check_exact(c, ref_gemm(a, b, in_dtype, layout), out_dtype,
                            "%s %s %dx%dx%d" % (layout, tdg.tdg_config_name(cfg), M, N, K))


# The primer's tail-test plan (NineToothed GEMM primer, section 5, last
# paragraph): M, N and K tails each tested on their own and together,
# including several full K tiles followed by a tail.  Edge values around the
# tile and MFMA sizes; a seeded sample of (M, N, K) per configuration, plus
# the three one-dimension-ragged cases at the largest edge.
TAIL_VALUES = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _tail_shapes(cfg, layout, vec, count=10):
    import random
    rng = random.Random(1000 * cfg + (layout == "tn"))
    ok = (lambda v: v % 8 == 0) if vec else (lambda v: True)
    ks = [v for v in TAIL_VALUES if ok(v)]
    ns = [v for v in TAIL_VALUES if ok(v)] if (vec and layout == "nn") else TAIL_VALUES
    shapes = [(257, max(ns), max(ks)), (max(TAIL_VALUES), 17 if 17 in ns else 16, max(ks)),
              (255, max(ns), 129 if 129 in ks else 136)]
    shapes += [(rng.choice(TAIL_VALUES), rng.choice(ns), rng.choice(ks)) for _ in range(count)]
    return shapes


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_tail_sweep_every_config_exact(tdg, layout):
    for cfg in range(tdg.tdg_num_configs()):
        name = tdg.tdg_config_name(cfg)
        vec = not name.endswith("_pred")
        for (M, N, K) in _tail_shapes(cfg, layout, vec):
            announce("tail sweep", layout, name, M, N, K)
            a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=M * 131 + N * 7 + K + cfg)
            c = gpu_gemm(tdg, a, b, layout, "f32", config=cfg)
            check_exact(c, ref_gemm(a, b, "bf16", layout), "f32", "%s %s %dx%dx%d" % (layout, name, M, N, K))


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_every_config_random_tolerance(tdg, layout):
    for cfg in range(tdg.tdg_num_configs()):
        vec = not tdg.tdg_config_name(cfg).endswith("_pred")
        for (M, N, K) in ([(65, 72, 200), (257, 264, 520)] + ([] if vec else [(63, 129, 197)])):
            for in_dtype, out_dtype in (("f16", "f16"), ("bf16", "bf16"), ("f16", "f32")):
                announce(layout, tdg.tdg_config_name(cfg), M, N, K, in_dtype, out_dtype)
                a, b = make_inputs(M, N, K, layout, in_dtype, "uniform", seed=cfg + 17)
                c = gpu_gemm(tdg, a, b, layout, out_dtype, config=cfg)
                check_tol(c, ref_gemm(a, b, in_dtype, layout), out_dtype, K, "cfg %d" % cfg)


# ---------------------------------------------------------------------------
# Strides, guard bands, NaN poison
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("pad", [8, 3])
def test_strided_operands_guard_band_and_nan_padding(tdg, layout, pad):
    """Operands are views into larger buffers whose padding columns hold NaN;
    C is a view into a buffer pre-filled with a sentinel.  The NaN must not
    reach C and nothing outside C's view may change.  pad=3 breaks 16-byte
    alignment of the rows (predicated path), pad=8 keeps it (vector path)."""
    M, N, K = 131, 136, 200
    announce("strided", layout, pad)
    a, b = make_inputs(M, N, K, layout, "f16", "ints", seed=77)
    A = torch.full((M, K + pad), float("nan"), dtype=torch.float16)
    A[:, :K] = a
    rb, cb = b.shape
    B = torch.full((rb, cb + pad), float("nan"), dtype=torch.float16)
    B[:, :cb] = b
    Cbuf = torch.full((M + 2, N + 2 * pad), -12345.0, dtype=torch.float32).cuda()
    Cview = Cbuf[1:M + 1, pad:pad + N]
    tdg.gemm(A.cuda()[:, :K], B.cuda()[:, :cb], layout=layout, out_dtype=torch.float32, out=Cview)
    torch.cuda.synchronize()
    host = Cbuf.cpu()
    check_exact(host[1:M + 1, pad:pad + N], ref_gemm(a, b, "f16", layout), "f32", "strided")
    mask = torch.ones_like(host, dtype=torch.bool)
    mask[1:M + 1, pad:pad + N] = False
    assert torch.all(host[mask] == -12345.0), "write outside C"


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_batched_strided(tdg, layout):
    batch, M, N, K = 5, 70, 88, 136
    announce("batched", layout)
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=5, batch=batch)
    c = gpu_gemm(tdg, a, b, layout, "f32")
    ref = ref_gemm(a, b, "bf16", layout)
    check_exact(c, ref, "f32", "batched")
    # broadcast B (2-D b with batched a)
    c2 = tdg.gemm(a.cuda(), b[0].cuda(), layout=layout, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref2 = ref_gemm(a, b[0:1].expand(batch, *b.shape[1:]).contiguous(), "bf16", layout)
    check_exact(c2.cpu(), ref2, "f32", "broadcast B")


# ---------------------------------------------------------------------------
# Degenerate sizes, pinned page examples, determinism, subnormals
# ---------------------------------------------------------------------------

def test_k_zero_writes_zeros_and_empty_is_noop(tdg):
    announce("degenerate")
    a = torch.empty((33, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, 40), dtype=torch.float16, device="cuda")
    out = torch.full((33, 40), 7.0, dtype=torch.float32, device="cuda")
    tdg.gemm(a, b, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    a = torch.empty((0, 16), dtype=torch.float16, device="cuda")
    b = torch.ones((16, 8), dtype=torch.float16, device="cuda")
    assert tdg.gemm(a, b).shape == (0, 8)


def test_page_examples_on_gpu(tdg, golden):
    """All-ones over the 65 x 97 x 130 tail case gives 130 everywhere, and
    2048 + 1 + 1 gives 2050 with the fp32 accumulator and fp16 output
    (NineToothed GEMM primer, s6 and s8 exercise 3)."""
    announce("page examples")
    o = golden["all_ones"]
    a = torch.ones((o["M"], o["K"]), dtype=torch.float16)
    b = torch.ones((o["K"], o["N"]), dtype=torch.float16)
    for cfg in range(tdg.tdg_num_configs()):
        if not tdg.tdg_config_name(cfg).endswith("_pred"):
            continue   # K = 130 is not a whole number of 8-element granules
        c = gpu_gemm(tdg, a, b, "nn", "f16", config=cfg)
        assert torch.all(c == o["value"])
    c = gpu_gemm(tdg, a, b, "nn", "f16")
    assert c.shape == (o["M"], o["N"]) and torch.all(c == o["value"])
    e = golden["fp32_accumulation"]
    a = torch.tensor([e["terms"]], dtype=torch.float16)
    b = torch.ones((3, 1), dtype=torch.float16)
    c = gpu_gemm(tdg, a, b, "nn", "f16")
    assert float(c[0, 0]) == e["final_fp16_output_from_fp32_accumulator"]


@pytest.mark.parametrize("name", ["nn_f16_4096", "tn_f16_batched_32x2048x2048x128"])
def test_determinism(tdg, name):
    w = WORKLOADS[name]
    announce("determinism", name)
    a, b = workload_inputs(w)
    ad, bd = a.cuda(), b.cuda()
    c1 = tdg.gemm(ad, bd, layout=w.layout, out_dtype=OUT_TORCH[w.out_dtype])
    c2 = tdg.gemm(ad, bd, layout=w.layout, out_dtype=OUT_TORCH[w.out_dtype])
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.uint8) if c1.dtype != torch.float32 else c1.view(torch.int32),
                       c2.view(torch.uint8) if c2.dtype != torch.float32 else c2.view(torch.int32))


def test_fp16_subnormal_inputs(tdg):
    """Subnormal fp16 inputs are used as their exact values (no flush): with
    A = 2^-24 * small integers and B = small integers the exact products are
    multiples of 2^-24, and the fp32 output holds them exactly."""
    announce("subnormals")
    M, N, K = 64, 72, 136
    gen = torch.Generator().manual_seed(3)
    ai = torch.randint(-3, 4, (M, K), generator=gen).to(torch.float64)
    bi = torch.randint(-3, 4, (K, N), generator=gen).to(torch.float64)
    a = (ai * 2.0 ** -24).to(torch.float16)          # subnormal fp16 values
    b = bi.to(torch.float16)
    assert torch.equal(a.to(torch.float64), ai * 2.0 ** -24)
    c = gpu_gemm(tdg, a, b, "nn", "f32")
    ref = ref_gemm(a, b, "f16", "nn")
    check_exact(c, ref, "f32", "subnormal")


# ---------------------------------------------------------------------------
# Split-K schedule (tdg_gemm_ws)
# ---------------------------------------------------------------------------

# Problems with few 128 x 128 tiles and a long K: the library cuts every tile
# into K slices of 16 K tiles (15 tiles x 16 slices, 9 x 16, 8 x 16 on 256
# CUs); the slices of one tile land on different XCDs.
SPLIT_SHAPES = [("nn", 300, 520, 16384, "f16", "f32"),
                ("tn", 257, 264, 16384, "bf16", "bf16"),
                ("nn", 512, 256, 16384, "bf16", "f16")]


def _ws_size(tdg, layout, M, N, K, batch=1):
    return tdg.tdg_gemm_workspace_size(1 if layout == "tn" else 0, M, N, K, batch, 0)


@pytest.mark.parametrize("layout,M,N,K,in_dtype,out_dtype", SPLIT_SHAPES)
def test_split_k_integer_exact_and_matches_unsplit(tdg, layout, M, N, K, in_dtype, out_dtype):
    announce("split-k ints", layout, M, N, K, in_dtype, out_dtype)
    assert _ws_size(tdg, layout, M, N, K) > 0, "shape should take the split-K schedule"
    a, b = make_inputs(M, N, K, layout, in_dtype, "ints", seed=M + N + K)
    c = gpu_gemm(tdg, a, b, layout, out_dtype)
    check_exact(c, ref_gemm(a, b, in_dtype, layout), out_dtype, "split-k %dx%dx%d" % (M, N, K))
    c0 = tdg.gemm(a.cuda(), b.cuda(), layout=layout, out_dtype=OUT_TORCH[out_dtype], split_k=False)
    torch.cuda.synchronize()
    assert torch.equal(c, c0.cpu())


@pytest.mark.parametrize("layout,M,N,K,in_dtype,out_dtype", SPLIT_SHAPES)
def test_split_k_random_tolerance_and_determinism(tdg, layout, M, N, K, in_dtype, out_dtype):
    announce("split-k random", layout, M, N, K, in_dtype, out_dtype)
    a, b = make_inputs(M, N, K, layout, in_dtype, "normal", seed=M * 3 + K)
    ad, bd = a.cuda(), b.cuda()
    c1 = tdg.gemm(ad, bd, layout=layout, out_dtype=OUT_TORCH[out_dtype])
    c2 = tdg.gemm(ad, bd, layout=layout, out_dtype=OUT_TORCH[out_dtype])
    torch.cuda.synchronize()
    check_tol(c1.cpu(), ref_gemm(a, b, in_dtype, layout), out_dtype, K, "split-k random")
    assert torch.equal(c1.view(torch.int16) if c1.element_size() == 2 else c1.view(torch.int32),
                       c2.view(torch.int16) if c2.element_size() == 2 else c2.view(torch.int32))


def test_split_k_workspace_reuse_and_errors(tdg):
    """One caller-owned workspace serves consecutive calls of different
    sizes (its counters are back at zero after each call); a workspace that
    is too small or misaligned is rejected before anything runs."""
    announce("split-k workspace")
    shapes = [("nn", 300, 520, 16384), ("nn", 1024, 1024, 16384), ("nn", 512, 256, 16384)]
    need = max(_ws_size(tdg, *s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for (layout, M, N, K) in shapes + shapes[:1]:
        a, b = make_inputs(M, N, K, layout, "f16", "ints", seed=K)
        ad, bd = a.cuda(), b.cuda()
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        st = tdg.tdg_gemm_ws(0, M, N, K, ad.data_ptr(), K, 0, bd.data_ptr(), N, 0, c.data_ptr(), N, 0, 1,
                             tdg.TDG_F16, tdg.TDG_F32, ws.data_ptr(), need, stream)
        assert st == tdg.TDG_SUCCESS, tdg.tdg_last_error()
        torch.cuda.synchronize()
        rows = sample_rows(M)
        check_exact(c.cpu()[rows], ref_gemm(a, b, "f16", layout, rows=rows), "f32", "reuse %dx%dx%d" % (M, N, K))
    M, N, K = 300, 520, 16384
    a = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    b = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    small = _ws_size(tdg, "nn", M, N, K) - 1024
    st = tdg.tdg_gemm_ws(0, M, N, K, a.data_ptr(), K, 0, b.data_ptr(), N, 0, c.data_ptr(), N, 0, 1,
                         tdg.TDG_F16, tdg.TDG_F32, ws.data_ptr(), small, stream)
    assert st == tdg.TDG_INVALID_VALUE and "workspace" in tdg.tdg_last_error()
    st = tdg.tdg_gemm_ws(0, M, N, K, a.data_ptr(), K, 0, b.data_ptr(), N, 0, c.data_ptr(), N, 0, 1,
                         tdg.TDG_F16, tdg.TDG_F32, ws.data_ptr() + 16, need - 16, stream)
    assert st == tdg.TDG_INVALID_VALUE and "aligned" in tdg.tdg_last_error()


@pytest.mark.parametrize("layout,M,N,K", [("nn", 4096, 5020, 264),    # 16 x 20 tiles: columns 0..4095 whole rounds
                                          ("tn", 5000, 4096, 256),    # 20 x 16 tiles: rows 0..4095 whole rounds
                                          ("tn", 4095, 5000, 3000)])
def test_partial_round_cut_exact(tdg, layout, M, N, K):
    """A single problem with a partial last round of 256 x 256 tiles is cut
    into whole rounds of 256 x 256 tiles and a 128 x 128 remainder (two
    launches): integer inputs must come out exact on both sides of the cut."""
    announce("cut", layout, M, N, K)
    a, b = make_inputs(M, N, K, layout, "f16", "ints", seed=M + 2 * N + K)
    c = gpu_gemm(tdg, a, b, layout, "f16")
    rows = sample_rows(M)
    check_exact(c[rows], ref_gemm(a, b, "f16", layout, rows=rows), "f16", "cut %dx%dx%d" % (M, N, K))
    cf = gpu_gemm(tdg, a, b, layout, "f32")
    check_exact(cf[rows], ref_gemm(a, b, "f16", layout, rows=rows), "f32", "cut fp32 %dx%dx%d" % (M, N, K))


# A partial last round of 256 x 256 tiles served in one launch: whole tiles,
# then the left-over tiles cut into K slices merged by the last slice to
# finish (the library picks it when no band of whole rounds exists, or when
# the 128 x 128 rest of the two-launch cut would fill fewer than half of the
# CUs).  (M, N, K): 17 x 17 tiles with no band; a band of 16 tile columns
# with a rest of 64 small tiles; the same cut in rows.
ROUND_SPLIT_SHAPES = [(4352, 4352, 1024), (4096, 4352, 2048), (4352, 4096, 2048)]


@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("M,N,K", ROUND_SPLIT_SHAPES)
def test_round_split_exact_and_deterministic(tdg, layout, M, N, K):
    announce("round split", layout, M, N, K)
    assert tdg.tdg_gemm_workspace_size(1 if layout == "tn" else 0, M, N, K, 1, 0) > 0, "should plan a K split"
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=M + N + K + 7)
    ad, bd = a.cuda(), b.cuda()
    c1 = tdg.gemm(ad, bd, layout=layout, out_dtype=torch.float32)
    c2 = tdg.gemm(ad, bd, layout=layout, out_dtype=torch.float32)
    c3 = tdg.gemm(ad, bd, layout=layout, out_dtype=torch.float32, split_k=False)   # no workspace: the cut
    torch.cuda.synchronize()
    assert torch.equal(c1, c2), "the one-launch schedule is not deterministic"
    rows = sample_rows(M)
    ref = ref_gemm(a, b, "bf16", layout, rows=rows)
    check_exact(c1.cpu()[rows], ref, "f32", "round split %s %dx%dx%d" % (layout, M, N, K))
    check_exact(c3.cpu()[rows], ref, "f32", "without workspace %s %dx%dx%d" % (layout, M, N, K))


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_round_split_random_tolerance(tdg, layout):
    M, N, K = 4352, 4352, 2048
    announce("round split random", layout, M, N, K)
    a, b = make_inputs(M, N, K, layout, "f16", "normal_k", seed=88)
    c = gpu_gemm(tdg, a, b, layout, "f16")
    rows = sample_rows(M)
    check_tol(c[rows], ref_gemm(a, b, "f16", layout, rows=rows), "f16", K, "round split random")


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_output_ownership_map(tdg, layout):
    """Every output element is written exactly once, by the lane that owns
    it: with A = identity (M = K) the product is B itself, and B's entries
    encode their own (row, column) (exact integers in fp16), so a misplaced,
    missing or doubled element shows up as a wrong code.  Run on every
    vectorised configuration, over a shape that spans several tiles and
    ragged edges."""
    M = K = 520
    N = 392
    announce("ownership", layout)
    code = (torch.arange(M).view(M, 1) % 64) * 32 + (torch.arange(N).view(1, N) % 32) - 1024   # |code| <= 1024
    a = torch.eye(M, K, dtype=torch.float16)
    b = code.to(torch.float16)                    # B[k][j] = code(k, j)
    if layout == "tn":
        b = b.t().contiguous()                    # stored N x K
    expect = code.to(torch.float32)
    for cfg in _config_ids(tdg, True):
        c = gpu_gemm(tdg, a, b, layout, "f32", config=cfg)
        bad = (c != expect).nonzero()
        assert bad.numel() == 0, "%s: %d misplaced elements, first at %s" % (
            tdg.tdg_config_name(cfg), bad.shape[0], bad[:4].tolist())


# ---------------------------------------------------------------------------
# Storage orders: A stored M x K or K x M, B stored K x N or N x K, C stored
# M x N or N x M (tdg_gemm; the Python front passes transposed views)
# ---------------------------------------------------------------------------

def _stored(t, transposed):
    """`t` on the device, as itself or as the transposed view of its
    transposed copy (same logical matrix, the other major order)."""
    return t.t().contiguous().cuda().t() if transposed else t.contiguous().cuda()


@pytest.mark.parametrize("ta", [0, 1])
@pytest.mark.parametrize("tb", [0, 1])
@pytest.mark.parametrize("tc", [0, 1])
def test_storage_orders_integer_exact(tdg, ta, tb, tc):
    for (M, N, K) in [(264, 392, 520), (520, 136, 264), (64, 128, 72)]:
        announce("storage", ta, tb, tc, M, N, K)
        a, b = make_inputs(M, N, K, "nn", "f16", "ints", seed=M + N + K + 4 * ta + 2 * tb + tc)
        A, B = _stored(a, ta), _stored(b, tb)
        out = torch.full((N, M), 77.0, device="cuda").t() if tc else torch.full((M, N), 77.0, device="cuda")
        tdg.gemm(A, B, layout="nn", out=out)
        torch.cuda.synchronize()
        check_exact(out.cpu(), ref_gemm(a, b, "f16", "nn"), "f32", "storage %d%d%d %dx%dx%d" % (ta, tb, tc, M, N, K))


@pytest.mark.parametrize("ta,tb,tc", [(1, 0, 0), (1, 1, 1), (0, 0, 1)])
def test_storage_orders_random_batched(tdg, ta, tb, tc):
    batch, M, N, K = 3, 136, 264, 392
    announce("storage random", ta, tb, tc)
    a, b = make_inputs(M, N, K, "nn", "bf16", "normal", seed=11, batch=batch)
    A = a.transpose(1, 2).contiguous().cuda().transpose(1, 2) if ta else a.cuda()
    B = b.transpose(1, 2).contiguous().cuda().transpose(1, 2) if tb else b.cuda()
    out = (torch.empty((batch, N, M), dtype=torch.bfloat16, device="cuda").transpose(1, 2) if tc
           else torch.empty((batch, M, N), dtype=torch.bfloat16, device="cuda"))
    tdg.gemm(A, B, layout="nn", out=out)
    torch.cuda.synchronize()
    check_tol(out.cpu(), ref_gemm(a, b, "bf16", "nn"), "bf16", K, "storage random")


@pytest.mark.parametrize("M,N,K", [(4096, 5016, 264), (5000, 4096, 256)])
def test_storage_a_transposed_partial_round_cut(tdg, M, N, K):
    """An A stored K x M through the 256 x 256 / 128 x 128 cut (columns, then
    rows: the row cut moves A's base along its contiguous dimension)."""
    announce("cut transa", M, N, K)
    a, b = make_inputs(M, N, K, "nn", "f16", "ints", seed=M + K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    tdg.gemm(_stored(a, True), b.cuda(), layout="nn", out=out)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    check_exact(out.cpu()[rows], ref_gemm(a, b, "f16", "nn", rows=rows), "f32", "cut transa")


def test_storage_order_support_rules(tdg):
    """A stored K x M needs the vectorised kernel: a ragged M is refused with
    TDG_NOT_SUPPORTED; a transposed store with B stored N x K is the plain
    TN product on exchanged operands and takes any shape."""
    announce("storage rules")
    M, N, K = 63, 40, 72
    a, b = make_inputs(M, N, K, "nn", "f16", "ints", seed=5)
    with pytest.raises(tdg.TdgError) as err:
        tdg.gemm(_stored(a, True), b.cuda(), layout="nn", out_dtype=torch.float32)
    assert err.value.status == tdg.TDG_NOT_SUPPORTED
    out = torch.empty((N, M), dtype=torch.float32, device="cuda").t()
    tdg.gemm(a.cuda(), _stored(b, True), layout="nn", out=out)        # ta 0, tb 1, tc 1
    torch.cuda.synchronize()
    check_exact(out.cpu(), ref_gemm(a, b, "f16", "nn"), "f32", "transc any shape")


# ---------------------------------------------------------------------------
# Autotuning (tdg_autotune)
# ---------------------------------------------------------------------------

def test_autotune_records_and_serves_the_winner(tdg):
    """The tuned configuration serves later automatic calls of the same
    problem (seen through tdg_select_config) and computes the same exact
    product; clearing the cache restores the library's own choice."""
    M, N, K = 1024, 1024, 1024
    announce("autotune", M, N, K)
    tdg.tdg_autotune_clear()
    a, b = make_inputs(M, N, K, "nn", "f16", "ints", seed=21)
    ad, bd = a.cuda(), b.cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    default = tdg.select_config(ad, bd, out_dtype=torch.float32)
    name = tdg.autotune(ad, bd, out=out, reps=3)
    assert name == "auto" or name in tdg.config_names()
    chosen = tdg.tdg_config_name(tdg.select_config(ad, bd, out_dtype=torch.float32))
    if name != "auto":
        assert chosen == name
    c = tdg.gemm(ad, bd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_exact(c.cpu(), ref_gemm(a, b, "f16", "nn"), "f32", "after autotune")
    tdg.tdg_autotune_clear()
    assert tdg.select_config(ad, bd, out_dtype=torch.float32) == default


def test_autotune_transposed_operands(tdg):
    M, N, K = 520, 264, 392
    announce("autotune storage")
    a, b = make_inputs(M, N, K, "nn", "bf16", "ints", seed=22)
    A, B = _stored(a, True), _stored(b, True)
    out = torch.empty((N, M), dtype=torch.float32, device="cuda").t()
    name = tdg.autotune(A, B, out=out, reps=2)
    assert name == "auto" or name in tdg.config_names()
    out.zero_()
    tdg.gemm(A, B, out=out)
    torch.cuda.synchronize()
    check_exact(out.cpu(), ref_gemm(a, b, "bf16", "nn"), "f32", "autotuned storage")
    tdg.tdg_autotune_clear()


# ---------------------------------------------------------------------------
# Persistent form of the 16x16x32 kernel: workgroups walking several tiles
# ---------------------------------------------------------------------------

# The library's own choice of the persistent kernel: two or more rounds of
# 256 x 256 tiles with K <= 512 (fp32 output: batches only), in both layouts
# (the automatic path, not a forced configuration).
@pytest.mark.parametrize("layout,M,N,K,batch,in_dtype,out_dtype", [("nn", 4096, 4096, 320, 2, "bf16", "bf16"),
                                                                   ("tn", 6100, 5400, 192, 0, "f16", "f16"),
                                                                   ("tn", 3000, 2700, 192, 4, "f16", "f32"),
                                                                   ("nn", 2048, 2048, 512, 8, "f16", "f32"),
                                                                   # 32 x 17 tiles: cut into 32 x 16 on the
                                                                   # persistent kernel and a 128 x 128 rest
                                                                   ("nn", 8192, 4352, 256, 0, "bf16", "bf16")])
def test_automatic_persistent_choice_exact(tdg, layout, M, N, K, batch, in_dtype, out_dtype):
    announce("auto persistent", layout, M, N, K, batch, in_dtype, out_dtype)
    a, b = make_inputs(M, N, K, layout, in_dtype, "ints", seed=M + K + batch, batch=batch)
    ad, bd = a.cuda(), b.cuda()
    assert tdg.config_names()[tdg.select_config(ad, bd, layout, OUT_TORCH[out_dtype])].endswith("_m16p")
    c = gpu_gemm(tdg, a, b, layout, out_dtype)
    rows = sample_rows(M)
    ref = ref_gemm(a, b, in_dtype, layout, rows=rows)
    check_exact(c[:, rows] if batch else c[rows], ref, out_dtype, "auto persistent %s %dx%dx%d b%d" % (layout, M, N, K, batch))


# (layout, M, N, K, batch): more 256 x 256 tiles than CUs, so workgroups take
# two or more tiles; ragged M, N and K tails; K = 64 (one K tile: the loads
# run ahead across several tiles); a batch whose tiles switch problems.
PERSISTENT_SHAPES = [("tn", 4347, 4349, 200, 0), ("nn", 4352, 4344, 64, 0), ("tn", 2048, 2048, 72, 5),
                     ("nn", 4360, 4096, 136, 0)]


@pytest.mark.parametrize("layout,M,N,K,batch", PERSISTENT_SHAPES)
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_persistent_kernel_integer_exact(tdg, layout, M, N, K, batch, out_dtype):
    cfg = [i for i in range(tdg.tdg_num_configs()) if tdg.tdg_config_name(i).endswith("_m16p")][0]
    announce("persistent", layout, M, N, K, batch, out_dtype)
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=M + N + K + batch, batch=batch)
    c = gpu_gemm(tdg, a, b, layout, out_dtype, config=cfg)
    check_exact(c, ref_gemm(a, b, "bf16", layout), out_dtype, "persistent %s %dx%dx%d b%d" % (layout, M, N, K, batch))


def test_persistent_kernel_random_and_repeatable(tdg):
    cfg = [i for i in range(tdg.tdg_num_configs()) if tdg.tdg_config_name(i).endswith("_m16p")][0]
    M, N, K = 4352, 4608, 1000
    announce("persistent random", M, N, K)
    a, b = make_inputs(M, N, K, "tn", "f16", "normal_k", seed=91)
    c1 = gpu_gemm(tdg, a, b, "tn", "f16", config=cfg)
    c2 = gpu_gemm(tdg, a, b, "tn", "f16", config=cfg)
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    rows = sample_rows(M)
    check_tol(c1[torch.from_numpy(rows)], ref_gemm(a, b, "f16", "tn", rows=rows), "f16", K, "persistent random")


# The 4-wave configuration (128 x 128 wave tiles, accumulators in AccVGPRs
# through the tied inline-assembly MFMA): several tiles, ragged edges, long K,
# both layouts and a batch whose tiles change problems.
FOUR_WAVE_SHAPES = [("nn", 1000, 1304, 2056, 0), ("tn", 777, 1024, 1544, 0), ("tn", 512, 520, 4104, 3),
                    ("nn", 256, 256, 64, 0)]


def _four_wave_config(tdg):
    return [i for i in range(tdg.tdg_num_configs()) if tdg.tdg_config_name(i) == "256x256x64_s2_w2x2_m16"][0]


@pytest.mark.parametrize("layout,M,N,K,batch", FOUR_WAVE_SHAPES)
@pytest.mark.parametrize("in_dtype,out_dtype", [("f16", "f16"), ("bf16", "f32")])
def test_four_wave_config_integer_exact(tdg, layout, M, N, K, batch, in_dtype, out_dtype):
    cfg = _four_wave_config(tdg)
    announce("4-wave", layout, M, N, K, batch, in_dtype, out_dtype)
    a, b = make_inputs(M, N, K, layout, in_dtype, "ints", seed=M + 3 * N + K + batch, batch=batch)
    c = gpu_gemm(tdg, a, b, layout, out_dtype, config=cfg)
    check_exact(c, ref_gemm(a, b, in_dtype, layout), out_dtype, "4-wave %s %dx%dx%d b%d" % (layout, M, N, K, batch))


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_four_wave_config_random_matches_default(tdg, layout):
    """Random data: within tolerance of the oracle on sampled rows, and
    repeatable launch to launch."""
    cfg = _four_wave_config(tdg)
    M, N, K = 1536, 1792, 3000
    announce("4-wave random", layout, M, N, K)
    a, b = make_inputs(M, N, K, layout, "bf16", "normal", seed=97)
    c1 = gpu_gemm(tdg, a, b, layout, "bf16", config=cfg)
    c2 = gpu_gemm(tdg, a, b, layout, "bf16", config=cfg)
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    rows = sample_rows(M)
    check_tol(c1[torch.from_numpy(rows)], ref_gemm(a, b, "bf16", layout, rows=rows), "bf16", K, "4-wave random")


# Leading dimensions so large that a 256-row (or 128-row) tile spans 2 GiB or
# more: the direct-to-LDS kernels address a tile with 32-bit offsets, so the
# library must pick a kernel that does not (checked on the host) and still
# produce the exact result.  About 5 GB of device memory per operand.
@pytest.mark.parametrize("which", ["lda", "ldc"])
def test_leading_dimension_past_32_bit_offsets(tdg, which):
    M, N, K = 300, 264, 136
    big = (1 << 23) + 64                      # elements: 256 rows x big x 2 bytes > 2 GiB
    announce("huge", which, big)
    a, b = make_inputs(M, N, K, "nn", "f16", "ints", seed=123)
    ref = ref_gemm(a, b, "f16", "nn")
    if which == "lda":
        buf = torch.zeros((M - 1) * big + K, dtype=torch.float16, device="cuda")
        ad = torch.as_strided(buf, (M, K), (big, 1))
        ad.copy_(a.cuda())
        c = tdg.gemm(ad, b.cuda(), layout="nn", out_dtype=torch.float16)
        torch.cuda.synchronize()
        check_exact(c.cpu(), ref, "f16", "huge lda")
    else:
        buf = torch.full(((M - 1) * big + N,), float("nan"), dtype=torch.float16, device="cuda")
        cd = torch.as_strided(buf, (M, N), (big, 1))
        tdg.gemm(a.cuda(), b.cuda(), layout="nn", out=cd)
        torch.cuda.synchronize()
        check_exact(cd.cpu(), ref, "f16", "huge ldc")
        # nothing outside C was written: the first gap between rows 0 and 1
        assert torch.isnan(buf[N:big].cpu()).all()
    del buf
    torch.cuda.empty_cache()


def test_batch_stride_past_32_bit(tdg):
    """Three TN problems whose A and C lie more than 2 GiB apart (batch
    strides of 2^30 + 64 elements): exact results for every problem."""
    batch, M, N, K = 3, 200, 264, 72
    stride = (1 << 30) + 64
    announce("huge batch stride", stride)
    a, b = make_inputs(M, N, K, "tn", "bf16", "ints", seed=321, batch=batch)
    ref = ref_gemm(a, b, "bf16", "tn")
    abuf = torch.zeros((batch - 1) * stride + M * K, dtype=torch.bfloat16, device="cuda")
    ad = torch.as_strided(abuf, (batch, M, K), (stride, K, 1))
    ad.copy_(a.cuda())
    cbuf = torch.full(((batch - 1) * stride + M * N,), float("nan"), dtype=torch.float32, device="cuda")
    cd = torch.as_strided(cbuf, (batch, M, N), (stride, N, 1))
    tdg.gemm(ad, b.cuda(), layout="tn", out=cd)
    torch.cuda.synchronize()
    check_exact(cd.cpu(), ref, "f32", "huge batch stride")
    del abuf, cbuf
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# IEEE special values inside the operands
# ---------------------------------------------------------------------------

def _plant_specials(a, b, layout):
    """Integer operands with NaN and infinities planted where the result does
    not depend on the summation order: a NaN in A (its row of C is NaN), a
    NaN in B (its column of C is NaN), one +inf in A (its row of C is +-inf,
    or NaN where the matching B entry is 0), and +inf and -inf in one row of
    A against equal B rows (NaN)."""
    nan, inf = float("nan"), float("inf")
    a = a.clone()
    b = b.clone()
    a[5, 7] = nan
    a[100, 30] = inf
    a[200, 40] = inf
    a[200, 41] = -inf

    def setb(k, n, v):
        if layout == "nn":
            b[k, n] = v
        else:
            b[n, k] = v
    N = b.shape[1] if layout == "nn" else b.shape[0]
    for n in range(N):
        setb(40, n, 1.0)
        setb(41, n, 1.0)
    setb(50, 60, nan)
    return a, b


# (M, N, K, configuration or None for the automatic choice, with split-K)
SPECIAL_CASES = [(384, 320, 256, "256x256x64_s2_w2x4_m16"), (384, 320, 256, "128x128x64_s4_w2x4_m16"),
                 (384, 320, 256, "256x256x64_s2_w2x4_m16p"), (384, 320, 256, "256x256x64_s2_w2x4_lds"),
                 (384, 320, 256, "64x64x64_w2x2_pred"), (1024, 1024, 4096, None)]


@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("M,N,K,cfg", SPECIAL_CASES)
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_ieee_special_values_propagate(tdg, layout, M, N, K, cfg, out_dtype):
    """NaN and infinities in A and B reach C as IEEE arithmetic says (the
    oracle sums the same bit patterns in binary64), through the one-tile,
    persistent, 32 x 32 x 16, predicated and split-K paths."""
    announce("ieee specials", layout, M, N, K, cfg, out_dtype)
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=M + N + K + (layout == "tn"))
    a, b = _plant_specials(a, b, layout)
    config = -1 if cfg is None else tdg.config_names().index(cfg)
    if cfg is None:
        assert tdg.tdg_gemm_workspace_size(1 if layout == "tn" else 0, M, N, K, 1, 0) > 0, "should plan a K split"
    c = gpu_gemm(tdg, a, b, layout, out_dtype, config=config)
    ref = ref_gemm(a, b, "bf16", layout)
    import numpy as np
    assert np.isnan(ref[5]).all() and np.isnan(ref[:, 60]).all() and np.isnan(ref[200]).all()
    assert np.isinf(ref[100]).any()
    check_exact(c, ref, out_dtype, "ieee specials %s %s" % (layout, cfg))


# ---------------------------------------------------------------------------
# A rows that do not start on 128-byte lines: the A-window form
# ---------------------------------------------------------------------------

# (layout, M, N, K, lda, byte offset of A past a 128-byte line)
AWIN_CASES = [("nn", 520, 264, 3000, 3000, 0), ("tn", 300, 512, 1000, 1016, 16), ("nn", 257, 304, 136, 200, 48),
              ("tn", 512, 520, 64, 72, 112), ("nn", 256, 256, 8, 8, 0), ("tn", 511, 257, 520, 600, 80)]


@pytest.mark.parametrize("layout,M,N,K,lda,a_off", AWIN_CASES)
@pytest.mark.parametrize("auto", [False, True])
def test_a_window_exact(tdg, layout, M, N, K, lda, a_off, auto):
    """A stored with row stride lda (rows off the 128-byte lines) starting
    a_off bytes past a line, NaN in every byte between the rows and before
    the first: the A-window configuration (forced, or the library's choice)
    reads exactly the rows' K elements -- any other byte would make a sum
    NaN -- and the result is bit-exact."""
    announce("a window", layout, M, N, K, lda, a_off, "auto" if auto else "forced")
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=M + N + K + lda)
    pre = 64 + a_off // 2                               # elements before A (a_off bytes past a line)
    store = torch.full((pre + M * lda + 64,), float("nan"), dtype=torch.bfloat16)
    view = store.as_strided((M, K), (lda, 1), pre)
    view.copy_(a)
    sd = store.cuda()
    assert sd.data_ptr() % 128 == 0
    ad = sd.as_strided((M, K), (lda, 1), pre)
    bd = b.cuda()
    if auto:
        c = tdg.gemm(ad, bd, layout=layout, out_dtype=torch.float32)
        if M * N >= 256 * 256 * 256 and (lda * 2) % 128:
            assert tdg.config_names()[tdg.select_config(ad, bd, layout, torch.float32)].endswith("_m16aw")
    else:
        cfg = tdg.config_names().index("256x256x64_s2_w2x4_m16aw")
        c = tdg.gemm(ad, bd, layout=layout, out_dtype=torch.float32, config=cfg)
    torch.cuda.synchronize()
    check_exact(c.cpu(), ref_gemm(a, b, "bf16", layout), "f32", "a window %s %dx%dx%d lda %d" % (layout, M, N, K, lda))


def test_a_window_choice(tdg):
    """The library picks the 256 x 256 A-window form for products of at
    least one round of 256 x 256 tiles whose A rows are off the 128-byte
    lines, in both layouts, the 128 x 128 one for smaller TN products only,
    and the plain forms for aligned rows."""
    names = tdg.config_names()
    def pick(layout, M, N, K, lda):
        ad = torch.empty(M, lda, dtype=torch.float16, device="cuda")[:, :K]
        bd = torch.empty((N, K) if layout == "tn" else (K, N), dtype=torch.float16, device="cuda")
        return names[tdg.select_config(ad, bd, layout, torch.float16)]
    assert pick("tn", 4096, 4096, 3000, 3000).endswith("_m16aw")
    assert pick("tn", 4096, 4096, 3000, 3008) == "256x256x64_s2_w2x4_m16"
    assert pick("nn", 4095, 5000, 3000, 3000) == "256x256x64_s2_w2x4_m16aw"
    assert pick("nn", 4095, 5000, 3000, 3008) == "256x256x64_s2_w2x4_m16"
    assert pick("tn", 1024, 1024, 3000, 3000) == "128x128x64_s4_w2x4_m16aw"
    assert pick("nn", 1024, 1024, 3000, 3000) == "128x128x64_s4_w2x4_m16"


# (layout, batch, M, N, K, lda, batch stride of A in elements): the batch
# stride moves each problem's rows to another offset within the 128-byte
# lines, so every problem of a call has its own row shifts.
AWIN_BATCH_CASES = [("tn", 3, 300, 264, 1000, 1016, 1016 * 300 + 24),
                    ("nn", 2, 257, 304, 520, 600, 600 * 257 + 8),
                    ("tn", 2, 130, 97, 136, 200, 200 * 130 + 56)]


@pytest.mark.parametrize("cfg", ["256x256x64_s2_w2x4_m16aw", "128x128x64_s4_w2x4_m16aw"])
@pytest.mark.parametrize("layout,batch,M,N,K,lda,sa", AWIN_BATCH_CASES)
def test_a_window_batched_exact(tdg, cfg, layout, batch, M, N, K, lda, sa):
    """Both A-window configurations, forced, on batched products whose A
    rows sit off the 128-byte lines by a shift that changes from problem to
    problem, NaN in every byte around the rows: bit-exact against the
    oracle problem by problem."""
    announce("a window batched", cfg, layout, batch, M, N, K, lda, sa)
    assert sa >= M * lda and (sa * 2) % 128 != 0
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=batch + M + N + K, batch=batch)
    pre = 64 + 8
    store = torch.full((pre + (batch - 1) * sa + M * lda + 64,), float("nan"), dtype=torch.bfloat16)
    store.as_strided((batch, M, K), (sa, lda, 1), pre).copy_(a)
    sd = store.cuda()
    assert sd.data_ptr() % 128 == 0
    ad = sd.as_strided((batch, M, K), (sa, lda, 1), pre)
    c = tdg.gemm(ad, b.cuda(), layout=layout, out_dtype=torch.float32, config=tdg.config_names().index(cfg))
    torch.cuda.synchronize()
    check_exact(c.cpu(), ref_gemm(a, b, "bf16", layout), "f32", "a window batched %s %s" % (cfg, layout))


@pytest.mark.parametrize("M,N,K", [(512, 512, 16008), (4352, 4352, 1000), (4095, 5000, 3000)])
def test_a_window_split_schedules_exact(tdg, M, N, K):
    """TN products with A rows off the 128-byte lines through the library's
    own schedules: split-K on the 128 x 128 A-window form (few tiles, long
    K), the one-launch partial round or the cut on the 256 x 256 one;
    bit-exact and the same bits on a second call."""
    announce("a window schedules", M, N, K)
    assert (K * 2) % 128 != 0
    a, b = make_inputs(M, N, K, "tn", "bf16", "ints", seed=M + N + K + 5)
    ad, bd = a.cuda(), b.cuda()
    assert "_m16aw" in tdg.config_names()[tdg.select_config(ad, bd, "tn", torch.float32)]
    c1 = tdg.gemm(ad, bd, layout="tn", out_dtype=torch.float32)
    c2 = tdg.gemm(ad, bd, layout="tn", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    rows = sample_rows(M) if M * N * K > 2 ** 31 else None
    ref = ref_gemm(a, b, "bf16", "tn", rows=rows)
    check_exact(c1.cpu()[rows] if rows is not None else c1.cpu(), ref, "f32", "a window schedules %dx%dx%d" % (M, N, K))
