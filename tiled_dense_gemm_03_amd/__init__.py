"""Tiled dense GEMM for AMD Instinct MI355X (gfx950).

``gemm(a, b, layout="nn" | "tn", out_dtype=None, out=None)`` computes
A @ B (NN, b is K x N) or A @ B^T (TN, b is N x K) for fp16/bf16 device
tensors with fp32 accumulation, optionally batched over a leading dimension,
by one call into the HIP library ``libtdg.so`` on the current torch stream.
The raw C entry points are re-exported with their C names (``tdg_gemm_nn``
and friends); torch supplies device memory and the stream only.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    TDG_BF16,
    TDG_E4M3,
    TDG_E5M2,
    TDG_F16,
    TDG_F32,
    TDG_INVALID_VALUE,
    TDG_LAUNCH_FAILED,
    TDG_NOT_SUPPORTED,
    TDG_SUCCESS,
    tdg_abi_version,
    tdg_autotune,
    tdg_autotune_clear,
    tdg_config_name,
    tdg_f8_config_name,
    tdg_f8_num_configs,
    tdg_gemm,
    tdg_gemm_ex,
    tdg_gemm_f8,
    tdg_gemm_nn,
    tdg_gemm_nn_batched,
    tdg_gemm_noalloc,
    tdg_gemm_tn,
    tdg_gemm_tn_batched,
    tdg_gemm_workspace_bound,
    tdg_gemm_workspace_size,
    tdg_gemm_ws,
    tdg_last_error,
    tdg_num_configs,
    tdg_select_config,
    tdg_status_string,
)
from .api import TdgError, autotune, config_names, gemm, gemm_f8, select_config  # noqa: F401
