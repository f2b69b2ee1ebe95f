"""Host model of who computes what (helpers, not a test module).

The pages build the product from an MMA atom repeated over threads and then
over tiles, and check by printing, on the host, which thread owns each output
element (cute (6) tiled_mma, section 3, the EU Repeat (2, 2, 1) thread map)
and by checking every address and operand slot of a copy with a small host
program (qingsen, "from partition_S to copy_unpack", the section that checks
addresses and argument binding with a small program).  This module is that
host program for gfx950: plain Python maps, written from the MFMA operand
layouts the kernels state, that

  * place an operand element (row or column, k) in (lane, element slot) and
    an accumulator register (lane, register) at (row, column) of the MFMA
    result, for the three MFMAs the kernels use;
  * compose those maps with each tile configuration's wave grid and MFMA tile
    repeat into (wave, lane, i, j, register) -> C element of the workgroup
    tile.

``tests/test_lane_model_cpu.py`` checks that every map is a bijection (each
element owned exactly once); ``tests/test_gpu_mfma_lanes.py`` runs one MFMA
of each kind on the GPU with small exact integers and compares every lane's
registers with these maps.
"""

# ---- one MFMA: D (M x N) = X (M x K) . Y (K x N) -------------------------
#
# x_slot(l, e) -> (m, k): element slot e of lane l in the X operand;
# y_slot(l, e) -> (n, k): likewise for the Y operand (lane supplies column n);
# d_slot(l, r) -> (m, n): accumulator register r of lane l.


def _x16(l, e):
    return l % 16, 8 * (l // 16) + e


def _d16(l, r):
    return 4 * (l // 16) + r, l % 16


def _x32(l, e):
    return l % 32, 8 * (l // 32) + e


def _d32(l, r):
    return 8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32


def _x32f8(l, e):
    g = l // 32
    return l % 32, (16 * g + e) if e < 16 else (32 + 16 * g + e - 16)


MFMA = {
    # v_mfma_f32_16x16x32_{f16,bf16}: 8 sixteen-bit elements per lane and operand
    "16x16x32": dict(M=16, N=16, K=32, elems=8, regs=4, x=_x16, y=_x16, d=_d16),
    # v_mfma_f32_32x32x16_{f16,bf16}
    "32x32x16": dict(M=32, N=32, K=16, elems=8, regs=16, x=_x32, y=_x32, d=_d32),
    # v_mfma_scale_f32_32x32x64_f8f6f4 on 8-bit operands: 32 bytes per lane
    "32x32x64f8": dict(M=32, N=32, K=64, elems=32, regs=16, x=_x32f8, y=_x32f8, d=_d32),
}


def scale_slot_32x32x64(l):
    """(row, 32-element K block) whose scale is lane l's scale byte (the same
    for the X and Y operands of the scaled 32 x 32 x 64 MFMA)."""
    return l % 32, l // 32


# ---- tile configurations ---------------------------------------------------
#
# How each kernel places its MFMA result tiles.  A wave w of a WM x WN grid
# owns the (BM/WM) x (BN/WN) sub-tile at (w / WN, w % WN); accumulator tile
# (i, j) covers its rows atom_m*i .. and columns atom_n*j ...  The kernels
# that pass the B fragment as the X operand (MFMA computes a block of C^T)
# have D's row as the output column and D's column as the output row.
KERNELS = {
    # kind: (MFMA, operands exchanged)
    0: ("32x32x16", False),    # register-staged kernel: mfma(A, B)
    1: ("32x32x16", True),     # direct-to-LDS 32 x 32 x 16 kernel: mfma(B, A)
    2: ("16x16x32", True),     # 16 x 16 x 32 kernel: mfma(B, A)
    3: ("16x16x32", True),     # its persistent form
    4: ("16x16x32", True),     # its ping-pong form
    5: ("16x16x32", True),     # its A-window form
    "f8": ("32x32x64f8", True),
}


def parse_config(name):
    """(kind, BM, BN, WM, WN) of a configuration name such as
    ``256x256x64_s2_w2x4_m16`` or ``f8_256x256x128_s2_w2x4``."""
    parts = name.split("_")
    if parts[0] == "f8":
        kind, parts = "f8", parts[1:]
    else:
        kind = {"lds": 1, "vec": 0, "pred": 0, "m16": 2, "m16p": 3, "m16pp": 4, "m16aw": 5}[parts[-1]]
    bm, bn = (int(v) for v in parts[0].split("x")[:2])
    wave = [p for p in parts if p.startswith("w") and "x" in p][0]
    wm, wn = (int(v) for v in wave[1:].split("x"))
    return kind, bm, bn, wm, wn


def owner_map(kind, bm, bn, wm, wn):
    """{(wave, lane, i, j, r): (row, column) of the workgroup tile}."""
    mf, swapped = KERNELS[kind]
    spec = MFMA[mf]
    am, an = spec["M"], spec["N"]
    wtm, wtn = bm // wm, bn // wn
    rm, rn = wtm // am, wtn // an
    assert rm * am == wtm and rn * an == wtn, "wave tile must be a whole number of MFMA tiles"
    out = {}
    for w in range(wm * wn):
        wr, wc = w // wn, w % wn
        for lane in range(64):
            for i in range(rm):
                for j in range(rn):
                    for r in range(spec["regs"]):
                        p, q = spec["d"](lane, r)
                        m, n = (q, p) if swapped else (p, q)
                        out[(w, lane, i, j, r)] = (wr * wtm + am * i + m, wc * wtn + an * j + n)
    return out
