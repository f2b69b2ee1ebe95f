"""ctypes binding of ``libtdg.so``: the C ABI of ``include/tdg.h``, one Python
function per C entry point with the same name and argument order.

This layer only marshals arguments: integers, raw device pointers and a
stream handle.  All work happens in the HIP library.  If the library has not
been built, importing this module raises, so no caller can silently run
anything else in its place.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtdg.so")

TDG_F16, TDG_BF16, TDG_F32, TDG_E4M3, TDG_E5M2 = 0, 1, 2, 3, 4
TDG_SUCCESS, TDG_INVALID_VALUE, TDG_NOT_SUPPORTED, TDG_LAUNCH_FAILED = 0, 1, 2, 3

if not os.path.exists(LIB_PATH):
    raise ImportError("tiled_dense_gemm_03_amd: %s is not built; run `python -c 'import __graft_entry__ as g; "
                      "g.build()'` (or tiled_dense_gemm_03_amd/build.py) first" % LIB_PATH)

lib = ctypes.CDLL(LIB_PATH)

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int
_sz = ctypes.c_size_t

_SIG = {
    "tdg_gemm_nn": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _vp]),
    "tdg_gemm_tn": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _vp]),
    "tdg_gemm_nn_batched": (_int, [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                                   _int, _int, _vp]),
    "tdg_gemm_tn_batched": (_int, [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                                   _int, _int, _vp]),
    "tdg_gemm_ex": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                           _int, _int, _int, _vp]),
    "tdg_gemm_ws": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                           _int, _int, _vp, _sz, _vp]),
    "tdg_gemm_workspace_size": (_sz, [_int, _i64, _i64, _i64, _i64, _int]),
    "tdg_gemm_workspace_bound": (_sz, [_int]),
    "tdg_gemm": (_int, [_int, _int, _int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                        _int, _int, _vp, _sz, _vp]),
    "tdg_gemm_noalloc": (_int, [_int, _int, _int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64,
                                _i64, _i64, _int, _int, _vp]),
    "tdg_autotune": (_int, [_int, _int, _int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                            _i64, _int, _int, _vp, _sz, _int, ctypes.POINTER(_int), _vp]),
    "tdg_autotune_clear": (None, []),
    "tdg_gemm_f8": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _int, _vp, _i64, _int, _vp, _i64, _vp, _i64,
                           _vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _vp]),
    "tdg_f8_num_configs": (_int, []),
    "tdg_f8_config_name": (ctypes.c_char_p, [_int]),
    "tdg_num_configs": (_int, []),
    "tdg_config_name": (ctypes.c_char_p, [_int]),
    "tdg_select_config": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _int, _int]),
    "tdg_status_string": (ctypes.c_char_p, [_int]),
    "tdg_last_error": (ctypes.c_char_p, []),
    "tdg_abi_version": (_int, []),
}

for _name, (_res, _args) in _SIG.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIG)


def tdg_gemm_nn(M, N, K, A, lda, B, ldb, C, ldc, ab_type, c_type, stream):
    return lib.tdg_gemm_nn(M, N, K, A, lda, B, ldb, C, ldc, ab_type, c_type, stream)


def tdg_gemm_tn(M, N, K, A, lda, B, ldb, C, ldc, ab_type, c_type, stream):
    return lib.tdg_gemm_tn(M, N, K, A, lda, B, ldb, C, ldc, ab_type, c_type, stream)


def tdg_gemm_nn_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                        stream):
    return lib.tdg_gemm_nn_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type,
                                   c_type, stream)


def tdg_gemm_tn_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                        stream):
    return lib.tdg_gemm_tn_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type,
                                   c_type, stream)


def tdg_gemm_ex(transb, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                config, stream):
    return lib.tdg_gemm_ex(transb, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type,
                           c_type, config, stream)


def tdg_gemm_ws(transb, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                workspace, workspace_bytes, stream):
    return lib.tdg_gemm_ws(transb, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type,
                           c_type, workspace, workspace_bytes, stream)


def tdg_gemm(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type,
             c_type, workspace, workspace_bytes, stream):
    return lib.tdg_gemm(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                        ab_type, c_type, workspace, workspace_bytes, stream)


def tdg_gemm_noalloc(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                     ab_type, c_type, stream):
    return lib.tdg_gemm_noalloc(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                                batch, ab_type, c_type, stream)


def tdg_gemm_workspace_size(transb, M, N, K, batch, num_cus):
    return lib.tdg_gemm_workspace_size(transb, M, N, K, batch, num_cus)


def tdg_gemm_workspace_bound(num_cus):
    return lib.tdg_gemm_workspace_bound(num_cus)


def tdg_autotune(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                 ab_type, c_type, workspace, workspace_bytes, reps, best_config, stream):
    """best_config: a ctypes.c_int (passed by reference)."""
    return lib.tdg_autotune(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                            batch, ab_type, c_type, workspace, workspace_bytes, reps, ctypes.byref(best_config),
                            stream)


def tdg_autotune_clear():
    lib.tdg_autotune_clear()


def tdg_gemm_f8(transc, M, N, K, A, lda, a_type, B, ldb, b_type, block_scale_a, ld_bsa, block_scale_b, ld_bsb,
                scale_a, inc_a, scale_b, inc_b, C, ldc, c_type, config, stream):
    return lib.tdg_gemm_f8(transc, M, N, K, A, lda, a_type, B, ldb, b_type, block_scale_a, ld_bsa, block_scale_b,
                           ld_bsb, scale_a, inc_a, scale_b, inc_b, C, ldc, c_type, config, stream)


def tdg_f8_num_configs():
    return lib.tdg_f8_num_configs()


def tdg_f8_config_name(config):
    r = lib.tdg_f8_config_name(config)
    return None if r is None else r.decode()


def tdg_num_configs():
    return lib.tdg_num_configs()


def tdg_config_name(config):
    r = lib.tdg_config_name(config)
    return None if r is None else r.decode()


def tdg_select_config(transb, M, N, K, A, lda, B, ldb, C, ldc, batch, ab_type, c_type):
    return lib.tdg_select_config(transb, M, N, K, A, lda, B, ldb, C, ldc, batch, ab_type, c_type)


def tdg_status_string(status):
    return lib.tdg_status_string(status).decode()


def tdg_last_error():
    return lib.tdg_last_error().decode()


def tdg_abi_version():
    return lib.tdg_abi_version()
