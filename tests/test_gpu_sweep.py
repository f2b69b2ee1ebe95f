"""A seeded sweep of the library's automatic schedule against the oracle.

Each case draws a layout, input and output types, a shape (mostly small and
ragged, some of several rounds of 256 x 256 tiles with a short K), an A
leading dimension with or without padding (padding that is not a multiple of
8 elements sends the call to the predicated kernels; a multiple of 8 that is
not a multiple of 64 puts A's rows off the 128-byte lines) and sometimes a
batch.  Inputs are small integers, so every product and sum is exact in
fp32 and the result must equal the oracle bit for bit (after the output
rounding the oracle applies).  A second set forces the two A-window
configurations on small shapes with rows off the lines.
"""
import random
import sys

import pytest
import torch

from parity import OUT_TORCH, check_exact, ref_gemm
from workloads import make_inputs, sample_rows

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


def draw_case(i):
    rng = random.Random(7000 + i)
    layout = rng.choice(["nn", "tn"])
    in_dt = rng.choice(["f16", "bf16"])
    out_dt = rng.choice(["f16", "bf16", "f32"])
    if rng.random() < 0.25:        # several rounds of 256 x 256 tiles, short K
        M, N, K = rng.randint(3000, 4700), rng.randint(3000, 4700), rng.choice([8, 64, 136, 200, 264])
        batch = 0
    else:
        M, N, K = rng.randint(1, 640), rng.randint(1, 640), rng.randint(1, 720)
        batch = rng.choice([0, 0, 0, 2, 3])
    if layout == "nn" and rng.random() < 0.7:
        N = max(8, N - N % 8)                      # mostly vectorisable NN B rows
    pad = rng.choice([0, 0, 8, 8 * rng.randint(1, 15), rng.randint(1, 7)])
    return layout, in_dt, out_dt, M, N, K, K + pad, batch


CASES = [draw_case(i) for i in range(40)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sweep_automatic_schedule_exact(tdg, case):
    layout, in_dt, out_dt, M, N, K, lda, batch = CASES[case]
    announce("sweep", case, layout, in_dt, out_dt, M, N, K, lda, batch)
    a, b = make_inputs(M, N, K, layout, in_dt, "ints", seed=case, batch=batch)
    lead = (batch,) if batch else ()
    nb = batch or 1
    sa = M * lda
    store = torch.zeros(nb * sa + 8, dtype=a.dtype)
    view = store.as_strided(lead + (M, K), ((sa,) if batch else ()) + (lda, 1))
    view.copy_(a)
    sd = store.cuda()
    ad = sd.as_strided(lead + (M, K), ((sa,) if batch else ()) + (lda, 1))
    c = tdg.gemm(ad, b.cuda(), layout=layout, out_dtype=OUT_TORCH[out_dt])
    torch.cuda.synchronize()
    c = c.cpu()
    rows = sample_rows(M) if M * N * K * nb > 2 ** 31 else None
    ref = ref_gemm(a, b, in_dt, layout, rows=rows)
    got = c[..., rows, :] if rows is not None else c
    check_exact(got, ref, out_dt, "sweep case %d %s" % (case, (layout, in_dt, out_dt, M, N, K, lda, batch)))


def draw_window_case(i):
    rng = random.Random(9000 + i)
    layout = rng.choice(["nn", "tn"])
    M, N, K = rng.randint(1, 600), rng.randint(1, 600), rng.randint(8, 700)
    K -= K % 8                                     # the vectorised forms take whole 8-element granules
    if layout == "nn":
        N = max(8, N - N % 8)
    lda = K + 8 * rng.choice([1, 2, 3, 5, 7, 9])
    if (lda * 2) % 128 == 0:
        lda += 8
    cfg = rng.choice(["256x256x64_s2_w2x4_m16aw", "128x128x64_s4_w2x4_m16aw"])
    return layout, M, N, K, lda, cfg


WINDOW_CASES = [draw_window_case(i) for i in range(12)]


@pytest.mark.parametrize("case", range(len(WINDOW_CASES)))
def test_sweep_a_window_forced_exact(tdg, case):
    layout, M, N, K, lda, cfg = WINDOW_CASES[case]
    announce("sweep window", case, layout, M, N, K, lda, cfg)
    assert (lda * 2) % 128 != 0 and lda % 8 == 0
    a, b = make_inputs(M, N, K, layout, "bf16", "ints", seed=100 + case)
    store = torch.zeros(M * lda + 8, dtype=a.dtype)
    store.as_strided((M, K), (lda, 1)).copy_(a)
    ad = store.cuda().as_strided((M, K), (lda, 1))
    c = tdg.gemm(ad, b.cuda(), layout=layout, out_dtype=torch.float32, config=tdg.config_names().index(cfg))
    torch.cuda.synchronize()
    check_exact(c.cpu(), ref_gemm(a, b, "bf16", layout), "f32", "window case %d" % case)
