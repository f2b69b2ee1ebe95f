"""One MFMA of each kind the kernels use, run on the GPU on small exact
integers (libtdg_probe.so, tdgp_mfma_lanes), against the host model of its
lane maps (tests/lane_model.py): the operands are placed into lane slots by
the model's operand maps, and every lane's accumulator registers must hold
the product entries the model's result map names -- exactly, since every
product and sum here is a small integer (times a power of two for the scaled
8-bit MFMA).  This pins the maps the kernels' fragment loads, epilogues and
the CPU ownership test are built on (the printed thread map of cute (6)
tiled_mma, section 3, done for gfx950)."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from lane_model import MFMA, scale_slot_32x32x64

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KINDS = {0: ("16x16x32", torch.float16), 1: ("16x16x32", torch.bfloat16), 2: ("32x32x16", torch.float16),
         3: ("32x32x16", torch.bfloat16), 4: ("32x32x64f8", torch.float8_e4m3fn)}


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(ROOT, "tiled_dense_gemm_03_amd", "libtdg_probe.so"))
    lib.tdgp_mfma_lanes.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def lane_bytes(mat, slot, elems, dtype, operand_rows_first):
    """64 x 32 bytes: lane l's slot e holds mat[row][k] for (row, k) = slot(l, e)
    (mat is rows x K for X, and K x cols for Y, hence the flag)."""
    vals = torch.zeros((64, elems), dtype=torch.float32)
    for l in range(64):
        for e in range(elems):
            r, k = slot(l, e)
            vals[l, e] = mat[r, k] if operand_rows_first else mat[k, r]
    raw = vals.to(dtype).view(torch.uint8).reshape(64, -1)
    out = torch.zeros((64, 32), dtype=torch.uint8)
    out[:, :raw.shape[1]] = raw
    return out


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_one_mfma_matches_host_model(probe, kind):
    name, dtype = KINDS[kind]
    spec = MFMA[name]
    print("CASE mfma lanes", kind, name, dtype, flush=True)
    sys.stdout.flush()
    gen = torch.Generator().manual_seed(900 + kind)
    X = torch.randint(-3, 4, (spec["M"], spec["K"]), generator=gen).float()
    Y = torch.randint(-3, 4, (spec["K"], spec["N"]), generator=gen).float()
    xb = lane_bytes(X, spec["x"], spec["elems"], dtype, True).cuda()
    yb = lane_bytes(Y, spec["y"], spec["elems"], dtype, False).cuda()
    if kind == 4:
        # per (row, block) and (column, block) power-of-two scales 2^(-2..2)
        ex = torch.randint(-2, 3, (32, 2), generator=gen)
        ey = torch.randint(-2, 3, (32, 2), generator=gen)
        sx = torch.tensor([127 + int(ex[scale_slot_32x32x64(l)]) for l in range(64)], dtype=torch.uint8).cuda()
        sy = torch.tensor([127 + int(ey[scale_slot_32x32x64(l)]) for l in range(64)], dtype=torch.uint8).cuda()
        D = torch.zeros((32, 32), dtype=torch.float64)
        for b in range(2):
            part = X[:, 32 * b:32 * b + 32].double() @ Y[32 * b:32 * b + 32, :].double()
            D += part * (2.0 ** ex[:, b].double()).view(32, 1) * (2.0 ** ey[:, b].double()).view(1, 32)
        sxp, syp = sx.data_ptr(), sy.data_ptr()
    else:
        D = X.double() @ Y.double()
        sxp = syp = None
    d = torch.full((64 * 16,), float("nan"), dtype=torch.float32, device="cuda")
    rc = probe.tdgp_mfma_lanes(kind, xb.data_ptr(), yb.data_ptr(), sxp, syp, d.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = d.cpu().double().numpy().reshape(64, 16)
    expect = np.zeros((64, spec["regs"]))
    for l in range(64):
        for r in range(spec["regs"]):
            expect[l, r] = D[spec["d"](l, r)]
    bad = np.argwhere(got[:, :spec["regs"]] != expect)
    assert bad.size == 0, "kind %d: %d lane registers differ from the model, first (lane, reg) %s: %s vs %s" % (
        kind, len(bad), bad[:4].tolist(), got[tuple(bad[:4].T)], expect[tuple(bad[:4].T)])
