"""CPU-side checks of the C ABI: the library loads, exports every entry point
declared in include/tdg.h, and rejects bad arguments synchronously, before
touching any device (no compute call is made here)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tdg.h")
LIB = os.path.join(ROOT, "tiled_dense_gemm_03_amd", "libtdg.so")


@pytest.fixture(scope="module")
def tdg():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "tdg_build", os.path.join(ROOT, "tiled_dense_gemm_03_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import tiled_dense_gemm_03_amd as t
    return t


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tdg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("tdg_gemm_nn", "tdg_gemm_tn", "tdg_gemm_nn_batched", "tdg_gemm_tn_batched",
                     "tdg_status_string", "tdg_last_error", "tdg_abi_version"):
        assert required in names


def test_every_declared_symbol_is_exported(tdg):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(tdg._binding.lib, name)
    assert set(tdg.EXPORTED) == set(declared_functions())


def test_version_configs_and_status_strings(tdg):
    assert tdg.tdg_abi_version() == 4
    n = tdg.tdg_num_configs()
    assert n >= 2
    names = [tdg.tdg_config_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert tdg.tdg_config_name(n) is None and tdg.tdg_config_name(-1) is None
    assert tdg.tdg_status_string(tdg.TDG_SUCCESS) == "TDG_SUCCESS"
    assert tdg.tdg_status_string(tdg.TDG_INVALID_VALUE) == "TDG_INVALID_VALUE"
    assert tdg.tdg_status_string(99) == "TDG_UNKNOWN_STATUS"


P = 1 << 20  # a fake, 16-byte aligned address: never dereferenced by these calls


@pytest.mark.parametrize("args,needle", [
    ((-1, 8, 8, P, 8, P, 8, P, 8, 0, 0), "negative"),
    ((8, -1, 8, P, 8, P, 8, P, 8, 0, 0), "negative"),
    ((8, 8, -1, P, 8, P, 8, P, 8, 0, 0), "negative"),
    ((8, 8, 16, P, 8, P, 8, P, 8, 0, 0), "lda"),
    ((8, 16, 8, P, 8, P, 8, P, 16, 0, 0), "ldb"),
    ((8, 16, 8, P, 8, P, 16, P, 8, 0, 0), "ldc"),
    ((8, 8, 8, P, 8, P, 8, P, 8, 2, 0), "ab_type"),
    ((8, 8, 8, P, 8, P, 8, P, 8, 0, 5), "c_type"),
    ((8, 8, 8, None, 8, P, 8, P, 8, 0, 0), "NULL"),
    ((8, 8, 8, P, 8, P, 8, None, 8, 0, 0), "NULL"),
    ((8, 8, 8, P + 1, 8, P, 8, P, 8, 0, 0), "aligned"),
    ((8, 8, 8, P, 8, P, 8, P + 2, 8, 0, 2), "aligned"),
    ((1 << 31, 8, 8, P, 8, P, 8, P, 8, 0, 0), "2^31"),
])
def test_invalid_arguments_rejected_before_launch(tdg, args, needle):
    st = tdg.tdg_gemm_nn(*args, None)
    assert st == tdg.TDG_INVALID_VALUE
    assert needle in tdg.tdg_last_error()


def test_tn_leading_dimension_rule(tdg):
    # TN: B is N x K, so ldb must be >= K (not N)
    assert tdg.tdg_gemm_tn(8, 32, 16, P, 16, P, 8, P, 32, 0, 0, None) == tdg.TDG_INVALID_VALUE
    assert "ldb" in tdg.tdg_last_error()


def test_batched_rules(tdg):
    # negative batch, negative stride, overlapping C
    assert tdg.tdg_gemm_nn_batched(8, 8, 8, P, 8, 64, P, 8, 64, P, 8, 64, -1, 0, 0, None) == tdg.TDG_INVALID_VALUE
    assert tdg.tdg_gemm_nn_batched(8, 8, 8, P, 8, -64, P, 8, 64, P, 8, 64, 2, 0, 0, None) == tdg.TDG_INVALID_VALUE
    assert tdg.tdg_gemm_tn_batched(8, 8, 8, P, 8, 64, P, 8, 64, P, 8, 32, 2, 0, 0, None) == tdg.TDG_INVALID_VALUE
    assert "overlap" in tdg.tdg_last_error()


def test_empty_problems_succeed_without_a_device(tdg):
    assert tdg.tdg_gemm_nn(0, 8, 8, None, 8, None, 8, None, 8, 0, 0, None) == tdg.TDG_SUCCESS
    assert tdg.tdg_gemm_tn(8, 0, 8, None, 8, None, 8, None, 1, 1, 2, None) == tdg.TDG_SUCCESS
    assert tdg.tdg_gemm_nn_batched(8, 8, 8, None, 8, 0, None, 8, 0, None, 8, 0, 0, 0, 0, None) == tdg.TDG_SUCCESS


def test_forced_config_checks(tdg):
    n = tdg.tdg_num_configs()
    assert tdg.tdg_gemm_ex(0, 8, 8, 8, P, 8, 0, P, 8, 0, P, 8, 0, 1, 0, 0, n, None) == tdg.TDG_INVALID_VALUE
    vec0 = [i for i in range(n) if not tdg.tdg_config_name(i).endswith("_pred")][0]
    # misaligned A (odd address) cannot take a vectorised configuration
    assert tdg.tdg_gemm_ex(0, 8, 8, 8, P + 2, 8, 0, P, 8, 0, P, 8, 0, 1, 0, 0, vec0, None) == tdg.TDG_INVALID_VALUE
    assert "aligned" in tdg.tdg_last_error()


def test_config_selection(tdg):
    def sel(transb, M, N, K, a=P, lda=None, b=P, ldb=None, batch=1, c_type=0):
        lda = lda or K
        ldb = ldb or (K if transb else N)
        return tdg.tdg_config_name(tdg.tdg_select_config(transb, M, N, K, a, lda, b, ldb, P, N, batch, 0, c_type))
    assert sel(0, 8192, 8192, 8192) == "256x256x64_s2_w2x4_m16"
    assert sel(1, 8192, 8192, 8192) == "256x256x64_s2_w2x4_m16"
    assert sel(1, 8192, 8192, 8192, c_type=2) == "256x256x64_s2_w2x4_m16"
    assert sel(1, 4096, 4096, 4096) == "256x256x64_s2_w2x4_m16"
    # A rows off the 128-byte lines: the A-window forms (256 x 256 for both
    # layouts, 128 x 128 for TN only)
    assert sel(0, 4095, 5000, 3000) == "256x256x64_s2_w2x4_m16aw"
    assert sel(0, 4095, 5000, 3000, lda=3008) == "256x256x64_s2_w2x4_m16"
    assert sel(1, 4096, 4096, 3000) == "256x256x64_s2_w2x4_m16aw"
    assert sel(1, 4096, 4096, 3000, lda=3008) == "256x256x64_s2_w2x4_m16"
    assert sel(0, 4096, 4096, 3000) == "256x256x64_s2_w2x4_m16aw"
    assert sel(1, 1024, 1024, 3000) == "128x128x64_s4_w2x4_m16aw"
    assert sel(0, 1024, 1024, 3000) == "128x128x64_s4_w2x4_m16"
    # the persistent kernel: several rounds of 256 x 256 tiles and K <= 512
    # (fp32 output: batches only)
    assert sel(1, 2048, 2048, 128, batch=32) == "256x256x64_s2_w2x4_m16p"
    assert sel(1, 2048, 2048, 128, batch=32, c_type=2) == "256x256x64_s2_w2x4_m16p"
    assert sel(0, 4096, 4096, 512, batch=4, c_type=2) == "256x256x64_s2_w2x4_m16p"
    assert sel(1, 8192, 8192, 128, c_type=2) == "256x256x64_s2_w2x4_m16"       # fp32, single problem
    assert sel(1, 8192, 8192, 128) == "256x256x64_s2_w2x4_m16p"
    assert sel(0, 4096, 4096, 512, batch=4) == "256x256x64_s2_w2x4_m16p"
    assert sel(0, 4096, 4096, 520, lda=576, batch=4) == "256x256x64_s2_w2x4_m16"
    assert sel(0, 4096, 4096, 520, batch=4) == "256x256x64_s2_w2x4_m16aw"   # lda 520: rows off the lines
    assert sel(1, 4096, 4096, 256) == "256x256x64_s2_w2x4_m16"          # a single round
    assert sel(0, 1024, 1024, 1024) == "128x128x64_s4_w2x4_m16"
    assert sel(0, 65, 97, 130).endswith("_pred")            # K not a multiple of 8
    assert not sel(1, 64, 97, 128).endswith("_pred")        # TN: N may be ragged
    assert sel(0, 64, 97, 128).endswith("_pred")            # NN: B rows need N % 8 == 0
    assert sel(0, 64, 64, 64, a=P + 2).endswith("_pred")    # misaligned base
    assert tdg.tdg_select_config(0, -1, 8, 8, P, 8, P, 8, P, 8, 1, 0, 0) == -1


def test_no_device_is_reported_not_run(tdg):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = tdg.tdg_gemm_nn(64, 64, 64, P, 64, P, 64, P, 64, 0, 0, None)
    assert st == tdg.TDG_NOT_SUPPORTED


def test_split_k_workspace_plan(tdg):
    """Workspace sizes of the split-K schedule on a 256-CU device.  Problems
    below one round of 256 x 256 tiles run on 128 x 128 tiles; when those are
    fewer than 256 they are split into at most 256 / tiles K slices of at
    least 16 K tiles, if that gives 128 work items or more.  4 bytes per fp32
    partial element, after a fixed block of one counter per CU (1 KiB)."""
    tile = 128 * 128 * 4
    ws = lambda transb, M, N, K, batch=1: tdg.tdg_gemm_workspace_size(transb, M, N, K, batch, 256)
    assert ws(0, 8192, 8192, 8192) == 0                        # 1024 tiles of 256 x 256
    assert ws(1, 2048, 2048, 128, 32) == 0                     # 2048 tiles
    # 320 tiles of 256 x 256: 256 whole tiles, the other 64 in 4 K slices of 11-12 K tiles
    assert ws(0, 4095, 5000, 3000) == 64 * 4 * 256 * 256 * 4 + 1024
    assert ws(1, 5000, 4095, 3000) == 64 * 4 * 256 * 256 * 4 + 1024
    assert ws(0, 4352, 4096, 1024) == 16 * 2 * 256 * 256 * 4 + 1024   # 272 tiles: 16 left over, 2 slices of 8
    assert ws(0, 4352, 4096, 256) == 0                         # 4 K tiles: too short to split (and persistent)
    assert ws(0, 4096, 4096, 4096, 2) == 0                     # batched: no partial-round split
    assert ws(0, 2048, 2048, 8192) == 0                        # 256 tiles of 128 x 128
    assert ws(0, 1024, 1024, 16384) == 64 * 4 * tile + 1024    # 64 tiles, 4 slices of 64 K tiles
    assert ws(0, 1024, 1024, 1024) == 0                        # 16 K tiles: too short to split
    assert ws(0, 300, 520, 16384) == 15 * 16 * tile + 1024     # 15 tiles, 16 slices of 16 K tiles
    assert ws(0, 300, 520, 8192) == 0                          # 15 x 8 slices: too few work items
    assert ws(1, 512, 256, 16384) == 8 * 16 * tile + 1024      # 8 tiles, 16 slices
    assert ws(0, 1024, 1024, 512) == 0
    assert ws(0, 0, 8, 8) == 0 and ws(0, 8, 8, 0) == 0 and ws(2, 64, 64, 64) == 0


def test_split_k_workspace_bound(tdg):
    """The bound serves every call: at most one 256 x 256 fp32 partial per CU
    after the counter block, and at least every size the plans ask for."""
    tile = 256 * 256 * 4
    for cus in (64, 80, 256, 304):
        bound = tdg.tdg_gemm_workspace_bound(cus)
        assert bound == cus * tile + (cus * 4 + 255) // 256 * 256
        for transb in (0, 1):
            for M, N, K in ((1024, 1024, 16384), (300, 520, 16384), (512, 256, 16384), (128, 128, 1 << 20),
                            (130, 1000, 65536), (4000, 100, 100000), (1, 1, 1 << 24), (4095, 5000, 3000),
                            (4352, 4096, 1 << 20), (8448, 8192, 4096)):
                for batch in (1, 2, 3):
                    assert tdg.tdg_gemm_workspace_size(transb, M, N, K, batch, cus) <= bound


def test_autotune_argument_checks(tdg):
    import ctypes
    best = ctypes.c_int(7)
    st = tdg.tdg_autotune(0, 0, 0, 64, 64, 64, P, 64, 0, P, 64, 0, P, 64, 0, 1, 0, 0, None, 0, 0, best, None)
    assert st == tdg.TDG_INVALID_VALUE and "reps" in tdg.tdg_last_error()
    st = tdg.tdg_autotune(0, 0, 0, 64, 64, 64, P, 32, 0, P, 64, 0, P, 64, 0, 1, 0, 0, None, 0, 5, best, None)
    assert st == tdg.TDG_INVALID_VALUE and "lda" in tdg.tdg_last_error()
    import torch
    if not torch.cuda.is_available():
        st = tdg.tdg_autotune(0, 0, 0, 64, 64, 64, P, 64, 0, P, 64, 0, P, 64, 0, 1, 0, 0, None, 0, 5, best, None)
        assert st == tdg.TDG_NOT_SUPPORTED
    tdg.tdg_autotune_clear()


def test_general_entry_point_checks(tdg):
    """tdg_gemm checks leading dimensions against each storage order."""
    g = lambda ta, tb, tc, lda, ldb, ldc: tdg.tdg_gemm(ta, tb, tc, 40, 24, 16, P, lda, 0, P, ldb, 0, P, ldc, 0, 1,
                                                         0, 0, None, 0, None)
    assert g(1, 0, 0, 32, 24, 24) == tdg.TDG_INVALID_VALUE and "lda" in tdg.tdg_last_error()   # A is K x M: lda >= 40
    assert g(0, 1, 0, 16, 8, 24) == tdg.TDG_INVALID_VALUE and "ldb" in tdg.tdg_last_error()    # B is N x K: ldb >= 16
    assert g(0, 0, 1, 16, 24, 24) == tdg.TDG_INVALID_VALUE and "ldc" in tdg.tdg_last_error()   # C is N x M: ldc >= 40
    assert g(2, 0, 0, 16, 24, 24) == tdg.TDG_INVALID_VALUE
    assert g(0, 0, 2, 16, 24, 24) == tdg.TDG_INVALID_VALUE


def test_f8_configs(tdg):
    n = tdg.tdg_f8_num_configs()
    names = [tdg.tdg_f8_config_name(i) for i in range(n)]
    assert n >= 2 and all(names) and len(set(names)) == n
    assert tdg.tdg_f8_config_name(n) is None and tdg.tdg_f8_config_name(-1) is None


def _f8_call(tdg, **kw):
    a = dict(transc=0, M=64, N=64, K=128, A=P, lda=128, a_type=tdg.TDG_E4M3, B=P, ldb=128, b_type=tdg.TDG_E4M3,
             block_scale_a=None, ld_bsa=0, block_scale_b=None, ld_bsb=0, scale_a=None, inc_a=0, scale_b=None,
             inc_b=0, C=P, ldc=64, c_type=tdg.TDG_F32, config=-1, stream=None)
    a.update(kw)
    return tdg.tdg_gemm_f8(*a.values())


@pytest.mark.parametrize("kw,status,needle", [
    (dict(transc=2), "INVALID", "transc"),
    (dict(M=-1), "INVALID", "negative"),
    (dict(K=-16), "INVALID", "negative"),
    (dict(a_type=0), "INVALID", "a_type"),
    (dict(b_type=2), "INVALID", "a_type"),
    (dict(c_type=3), "INVALID", "c_type"),
    (dict(lda=64), "INVALID", "lda"),
    (dict(ldb=112), "INVALID", "lda"),
    (dict(ldc=32), "INVALID", "ldc"),
    (dict(transc=1, M=128, ldc=64), "INVALID", "ldc"),
    (dict(block_scale_a=P, ld_bsa=2), "INVALID", "ceil(K/32)"),
    (dict(block_scale_b=P, ld_bsb=0), "INVALID", "ceil(K/32)"),
    (dict(inc_a=-1), "INVALID", "increments"),
    (dict(config=7), "INVALID", "config"),
    (dict(C=None), "INVALID", "NULL"),
    (dict(B=None), "INVALID", "NULL"),
    (dict(C=P + 2, c_type=2), "INVALID", "aligned"),
    (dict(scale_a=P + 2), "INVALID", "4-byte"),
    (dict(A=P + 8), "NOT_SUPPORTED", "16-byte"),
    (dict(lda=136), "NOT_SUPPORTED", "multiples of 16"),
    (dict(K=120, lda=128, ldb=128), "NOT_SUPPORTED", "multiples of 16"),
    (dict(block_scale_a=P + 4, ld_bsa=16), "NOT_SUPPORTED", "16-byte"),
    (dict(block_scale_b=P, ld_bsb=8), "NOT_SUPPORTED", "multiple of 16"),
    (dict(lda=1 << 24, ldb=1 << 24), "NOT_SUPPORTED", "32-bit"),
])
def test_f8_invalid_arguments_rejected_before_launch(tdg, kw, status, needle):
    st = _f8_call(tdg, **kw)
    expect = tdg.TDG_INVALID_VALUE if status == "INVALID" else tdg.TDG_NOT_SUPPORTED
    assert st == expect, (st, tdg.tdg_last_error())
    assert needle in tdg.tdg_last_error()


def test_f8_degenerate_sizes_succeed_without_a_device(tdg):
    assert _f8_call(tdg, M=0) == tdg.TDG_SUCCESS
    assert _f8_call(tdg, N=0, A=None, B=None, C=None) == tdg.TDG_SUCCESS


PROBE_HEADER = os.path.join(ROOT, "tiled_dense_gemm_03_amd", "probe", "tdg_probe.h")
PROBE_LIB = os.path.join(ROOT, "tiled_dense_gemm_03_amd", "libtdg_probe.so")


def test_probe_library_exports_its_header(tdg):
    """The MFMA ceiling probe beside the library: every function its header
    declares is exported, and bad arguments are refused before any launch."""
    import ctypes
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tdgp_[a-z0-9_]+)\s*\(", text)))
    assert names == ["tdgp_flops", "tdgp_flops_f8", "tdgp_mfma_lanes", "tdgp_mfma_stream", "tdgp_mfma_stream_f8",
                     "tdgp_operand_bytes_f8", "tdgp_operand_elems"]
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    assert set(names) <= exported
    lib = ctypes.CDLL(PROBE_LIB)
    lib.tdgp_operand_elems.restype = ctypes.c_size_t
    lib.tdgp_flops.restype = ctypes.c_double
    lib.tdgp_flops.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.tdgp_mfma_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tdgp_operand_elems() == 24 * 512 * 8
    # 64 MFMAs of 16x16x32 per wave per K tile, 8 waves per workgroup
    assert lib.tdgp_flops(3, 5) == 2.0 * 16 * 16 * 32 * 64 * 8 * 5 * 3
    fake = 1 << 20                           # never dereferenced: each call below fails its checks first
    assert lib.tdgp_mfma_stream(None, 1, 1, fake, None, None) == 1
    assert lib.tdgp_mfma_stream(fake, 1, 1, None, None, None) == 1
    assert lib.tdgp_mfma_stream(fake + 8, 1, 1, fake, None, None) == 1     # operands not 16-byte aligned
    assert lib.tdgp_mfma_stream(fake, 0, 1, fake, None, None) == 1
    assert lib.tdgp_mfma_stream(fake, 1, 0, fake, None, None) == 1
    assert lib.tdgp_mfma_stream(fake, 1, 65537, fake, None, None) == 1
    lib.tdgp_operand_bytes_f8.restype = ctypes.c_size_t
    lib.tdgp_flops_f8.restype = ctypes.c_double
    lib.tdgp_flops_f8.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.tdgp_mfma_stream_f8.argtypes = lib.tdgp_mfma_stream.argtypes
    assert lib.tdgp_operand_bytes_f8() == 12 * 512 * 32
    # 16 MFMAs of 32x32x64 per wave per K tile, 8 waves per workgroup
    assert lib.tdgp_flops_f8(3, 5) == 2.0 * 32 * 32 * 64 * 16 * 8 * 5 * 3
    assert lib.tdgp_mfma_stream_f8(None, 1, 1, fake, None, None) == 1
    assert lib.tdgp_mfma_stream_f8(fake + 16, 1, 1, fake, None, None) == 1  # operands not 32-byte aligned
    assert lib.tdgp_mfma_stream_f8(fake, 0, 1, fake, None, None) == 1
    lib.tdgp_mfma_lanes.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tdgp_mfma_lanes(5, fake, fake, None, None, fake, None) == 1          # no such kind
    assert lib.tdgp_mfma_lanes(-1, fake, fake, None, None, fake, None) == 1
    assert lib.tdgp_mfma_lanes(0, fake + 16, fake, None, None, fake, None) == 1     # X not 32-byte aligned
    assert lib.tdgp_mfma_lanes(0, fake, None, None, None, fake, None) == 1
    assert lib.tdgp_mfma_lanes(4, fake, fake, None, fake, fake, None) == 1          # scaled kind without scales
