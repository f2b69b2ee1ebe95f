"""The host model of the kernels' work split (tests/lane_model.py), checked on
the CPU for every tile configuration the library offers: each MFMA's operand
slots and accumulator registers cover their matrices exactly once, and every
configuration's (wave, lane, accumulator tile, register) -> output element
map covers the workgroup tile exactly once -- no element owned twice, none
left out (cute (6) tiled_mma, section 3: the thread map of a repeated atom;
qingsen "from partition_S to copy_unpack": checking every slot with a small
host program).  The GPU side of the same maps is tests/test_gpu_mfma_lanes.py
(one MFMA per kind) and the ownership test of tests/test_gpu_parity.py (every
configuration, end to end)."""
import os

import pytest

from lane_model import KERNELS, MFMA, owner_map, parse_config, scale_slot_32x32x64

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tdg():
    if not os.path.exists(os.path.join(ROOT, "tiled_dense_gemm_03_amd", "libtdg.so")):
        pytest.skip("library not built")
    import tiled_dense_gemm_03_amd as t
    return t


@pytest.mark.parametrize("kind", sorted(MFMA))
def test_mfma_slots_are_bijections(kind):
    s = MFMA[kind]
    for name, fn, rows, cols in (("X", s["x"], s["M"], s["K"]), ("Y", s["y"], s["N"], s["K"])):
        seen = {fn(l, e) for l in range(64) for e in range(s["elems"])}
        assert len(seen) == 64 * s["elems"] == rows * cols, (kind, name)
        assert seen == {(r, k) for r in range(rows) for k in range(cols)}, (kind, name)
    d = {s["d"](l, r) for l in range(64) for r in range(s["regs"])}
    assert len(d) == 64 * s["regs"] == s["M"] * s["N"]
    assert d == {(m, n) for m in range(s["M"]) for n in range(s["N"])}


def test_scale_slots_cover_rows_and_blocks():
    got = {scale_slot_32x32x64(l) for l in range(64)}
    assert got == {(r, b) for r in range(32) for b in range(2)}


def test_operand_runs_are_contiguous_k():
    """Each lane's 16-bit operand slots are 8 consecutive k (one 16-byte LDS
    read of a K-contiguous row serves a whole operand register quad), and the
    8-bit operand's 32 bytes are two runs of 16 consecutive k."""
    for kind in ("16x16x32", "32x32x16"):
        f = MFMA[kind]["x"]
        for l in range(64):
            rows = {f(l, e)[0] for e in range(8)}
            ks = [f(l, e)[1] for e in range(8)]
            assert len(rows) == 1 and ks == list(range(ks[0], ks[0] + 8)) and ks[0] % 8 == 0
    f = MFMA["32x32x64f8"]["x"]
    for l in range(64):
        ks = [f(l, e)[1] for e in range(32)]
        assert ks[:16] == list(range(ks[0], ks[0] + 16)) and ks[16:] == list(range(ks[16], ks[16] + 16))


def test_accumulator_rows_for_row_stores():
    """The kernels that exchange the operands get four consecutive output
    columns of one row per lane (one 16-byte store or LDS write of C)."""
    for kind, (mf, swapped) in KERNELS.items():
        if not swapped:
            continue
        s = MFMA[mf]
        for l in range(64):
            for base in range(0, s["regs"], 4):
                cells = [s["d"](l, base + r) for r in range(4)]
                rows = {p for p, q in cells}      # D rows = output columns
                cols = {q for p, q in cells}      # D column = output row
                assert len(cols) == 1 and sorted(rows) == list(range(min(rows), min(rows) + 4)), (kind, l)


def _check_owner(kind, bm, bn, wm, wn, what):
    own = owner_map(kind, bm, bn, wm, wn)
    cells = list(own.values())
    assert len(set(cells)) == len(cells), "%s: an output element is owned twice" % what
    assert set(cells) == {(r, c) for r in range(bm) for c in range(bn)}, "%s: the tile is not covered" % what


def test_every_configuration_owns_its_tile_once(tdg):
    names = [tdg.tdg_config_name(i) for i in range(tdg.tdg_num_configs())]
    assert len(names) >= 10
    for name in names:
        kind, bm, bn, wm, wn = parse_config(name)
        _check_owner(kind, bm, bn, wm, wn, name)


def test_every_8bit_configuration_owns_its_tile_once(tdg):
    for i in range(tdg.tdg_f8_num_configs()):
        name = tdg.tdg_f8_config_name(i)
        kind, bm, bn, wm, wn = parse_config(name)
        assert kind == "f8"
        _check_owner(kind, bm, bn, wm, wn, name)


def test_model_catches_a_wrong_map():
    """Negative control: a wave grid that reuses a column of waves, or an MFMA
    result map with a dropped term, is caught by the same check."""
    own = owner_map(2, 128, 128, 2, 2)
    broken = {k: (v[0], v[1] % 64) for k, v in own.items()}     # waves of column 1 land on column 0
    assert len(set(broken.values())) < len(broken)
    d16 = MFMA["16x16x32"]["d"]
    wrong = {(4 * (l // 16), l % 16) for l in range(64) for r in range(4)}   # register term dropped
    assert len(wrong) < 64 * 4 and {d16(l, r) for l in range(64) for r in range(4)} != wrong
