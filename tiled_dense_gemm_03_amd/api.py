"""Tensor-level front of the C ABI: shape/stride marshalling only.

Accepts torch tensors on a ROCm device whose matrices are row-major (unit
last stride) or column-major (unit second-to-last stride, e.g. a ``.t()``
view), reads their sizes, strides and data pointers, and makes exactly one
call into ``libtdg.so`` on ``torch.cuda.current_stream()``.  No arithmetic of
the product happens here.
"""
import ctypes

import torch

from . import _binding as _b

_AB = {torch.float16: _b.TDG_F16, torch.bfloat16: _b.TDG_BF16}
_CT = {torch.float16: _b.TDG_F16, torch.bfloat16: _b.TDG_BF16, torch.float32: _b.TDG_F32}


class TdgError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s: %s" % (_b.tdg_status_string(status), detail))
        self.status = status


def _check(status):
    if status != _b.TDG_SUCCESS:
        raise TdgError(status, _b.tdg_last_error())


def _storage(t, name):
    """(transposed, ld): how the (rows x cols) matrices of `t` are stored --
    row-major with row stride ld, or column-major (the stored matrix is
    cols x rows with row stride ld)."""
    if t.dim() not in (2, 3):
        raise ValueError("%s must be 2-D or 3-D (batched), got %d-D" % (name, t.dim()))
    rows, cols = t.size(-2), t.size(-1)
    if cols <= 1 or t.stride(-1) == 1:
        return False, max(t.stride(-2), cols, 1)
    if rows <= 1 or t.stride(-2) == 1:
        return True, max(t.stride(-1), rows, 1)
    raise ValueError("%s must have unit stride in one of its last two dimensions" % name)


def config_names():
    return [_b.tdg_config_name(i) for i in range(_b.tdg_num_configs())]


def _dims(a, b, layout):
    M, K = a.shape[-2], a.shape[-1]
    if layout == "nn":
        Kb, N = b.shape[-2], b.shape[-1]
    elif layout == "tn":
        N, Kb = b.shape[-2], b.shape[-1]
    else:
        raise ValueError("layout must be 'nn' or 'tn'")
    if Kb != K:
        raise ValueError("inner dimensions differ: A has K=%d, B has K=%d" % (K, Kb))
    return M, N, K


def _ld(t):
    # row stride in elements; a single-row matrix may report any stride
    return max(t.stride(-2), t.size(-1), 1)


def select_config(a, b, layout="nn", out_dtype=None):
    """Index of the tile configuration the library picks for these operands."""
    M, N, K = _dims(a, b, layout)
    batch = a.shape[0] if a.dim() == 3 else 1
    ct = _CT[out_dtype or a.dtype]
    return _b.tdg_select_config(1 if layout == "tn" else 0, M, N, K, a.data_ptr(), _ld(a), b.data_ptr(), _ld(b),
                                None, N, batch, _AB[a.dtype], ct)


# Split-K workspaces, one per (device, stream) so that calls that may run at
# the same time never share one; zero-filled once by torch, kept zero-filled by
# the library.  Each is allocated once, at the library's bound for the device
# (tdg_gemm_workspace_bound: enough for any call), and never replaced or
# freed: a HIP graph captured with one keeps using its address on every
# replay.  A replay and an eager call on the same stream's workspace must not
# overlap in time (torch replays a graph on the stream it is replayed from).
_workspaces = {}
# Workspace bytes the library asks for, per problem (the answer depends only
# on the sizes and the device's compute-unit count).
_ws_need = {}


def _workspace(device, stream, nbytes):
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, stream)
    ws = _workspaces.get(key)
    if ws is None:
        with torch.cuda.device(index):
            bound = _b.tdg_gemm_workspace_bound(0)
        ws = torch.zeros(max(bound, nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    if ws.numel() < nbytes:
        raise RuntimeError("split-K workspace of %d bytes is below the %d bytes a call asks for "
                           "(the library's bound)" % (ws.numel(), nbytes))
    return ws


def _marshal(a, b, layout, out_dtype, out):
    """Sizes, storage orders, strides and the output tensor of one call."""
    if a.dtype not in _AB or b.dtype != a.dtype:
        raise TypeError("a and b must both be float16 or both bfloat16 (got %s, %s)" % (a.dtype, b.dtype))
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("a and b must be device tensors")
    ta, lda = _storage(a, "a")
    b_col, ldb = _storage(b, "b")
    M, N, K = _dims(a, b, layout)
    # transb: B stored N x K.  "nn" gives b as (K, N): row-major -> K x N;
    # "tn" gives b as (N, K): row-major -> N x K.  A column-major view flips it.
    tb = (layout == "tn") != b_col
    batched = a.dim() == 3 or b.dim() == 3
    batch = a.shape[0] if a.dim() == 3 else (b.shape[0] if b.dim() == 3 else 1)
    if a.dim() == 3 and b.dim() == 3 and a.shape[0] != b.shape[0]:
        raise ValueError("batch sizes differ")
    odt = out_dtype or (out.dtype if out is not None else a.dtype)
    if odt not in _CT:
        raise TypeError("out_dtype must be float16, bfloat16 or float32")
    shape = (batch, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=odt, device=a.device)
    elif tuple(out.shape) != shape or out.dtype != odt:
        raise ValueError("out must be %s of %s, got %s of %s" % (shape, odt, tuple(out.shape), out.dtype))
    tc, ldc = _storage(out, "out")
    sA = a.stride(0) if a.dim() == 3 else 0
    sB = b.stride(0) if b.dim() == 3 else 0
    sC = out.stride(0) if out.dim() == 3 else 0
    return (int(ta), int(tb), int(tc), M, N, K, lda, sA, ldb, sB, ldc, sC, batch, odt, out)


def gemm(a, b, layout="nn", out_dtype=None, out=None, config=-1, split_k=True):
    """C = A @ B (layout "nn", b is (K, N)) or A @ B^T ("tn", b is (N, K)).

    a: (M, K) or (batch, M, K); b likewise batched or not (a 2-D b is shared
    by every problem of a batched a).  Each matrix may be row-major or
    column-major (a transposed view such as ``x.t()``), A, B and ``out``
    alike.  fp16/bf16 inputs of the same dtype, fp32 accumulation; out_dtype
    defaults to the input dtype and may be float32.  ``out`` is written in
    place; otherwise a new row-major tensor is returned.  ``config`` forces a
    tile configuration (tests and sweeps; row-major A and C only); -1 lets
    the library choose, and then ``split_k`` lets it use its split-K schedule
    (a workspace per device and stream, allocated by torch once).
    """
    ta, tb, tc, M, N, K, lda, sA, ldb, sB, ldc, sC, batch, odt, out = _marshal(a, b, layout, out_dtype, out)
    dev = a.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    if config == -1:
        ws = None
        if split_k:
            key = (tb, M, N, K, batch, dev.index)
            need = _ws_need.get(key)
            if need is None:
                with torch.cuda.device(dev):
                    need = _b.tdg_gemm_workspace_size(tb, M, N, K, batch, 0)
                if len(_ws_need) >= 4096:
                    _ws_need.clear()
                _ws_need[key] = need
            if need:
                ws = _workspace(dev, stream, need)
        args = (ta, tb, tc, M, N, K, a.data_ptr(), lda, sA, b.data_ptr(), ldb, sB, out.data_ptr(), ldc, sC, batch,
                _AB[a.dtype], _CT[odt], ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0, stream)
        call = _b.lib.tdg_gemm
    else:
        if ta or tc:
            raise ValueError("a forced configuration takes row-major a and out")
        args = (tb, M, N, K, a.data_ptr(), lda, sA, b.data_ptr(), ldb, sB, out.data_ptr(), ldc, sC, batch,
                _AB[a.dtype], _CT[odt], int(config), stream)
        call = _b.lib.tdg_gemm_ex
    # the library launches on the current device: make it a's (the common
    # case needs no switch)
    if dev.index is None or dev.index == torch.cuda.current_device():
        _check(call(*args))
    else:
        with torch.cuda.device(dev):
            _check(call(*args))
    return out


def autotune(a, b, layout="nn", out_dtype=None, out=None, reps=10):
    """Time every tile configuration (and the library's own schedule) on
    these operands and remember the fastest for later ``gemm`` calls of the
    same problem in this process.  Synchronises the current stream and
    writes ``out``.  Returns the winning configuration's name, or "auto"."""
    ta, tb, tc, M, N, K, lda, sA, ldb, sB, ldc, sC, batch, odt, out = _marshal(a, b, layout, out_dtype, out)
    stream = torch.cuda.current_stream(a.device).cuda_stream
    best = ctypes.c_int(-2)
    with torch.cuda.device(a.device):
        need = _b.tdg_gemm_workspace_size(tb, M, N, K, batch, 0)
        ws = _workspace(a.device, stream, need) if need else None
        _check(_b.tdg_autotune(ta, tb, tc, M, N, K,
                               a.data_ptr(), lda, sA, b.data_ptr(), ldb, sB,
                               out.data_ptr(), ldc, sC, batch,
                               _AB[a.dtype], _CT[odt],
                               ws.data_ptr() if ws is not None else None,
                               ws.numel() if ws is not None else 0, int(reps), best, stream))
    return "auto" if best.value < 0 else _b.tdg_config_name(best.value)


_F8 = {torch.float8_e4m3fn: _b.TDG_E4M3, torch.float8_e5m2: _b.TDG_E5M2}
_F8_NAME = {"e4m3": _b.TDG_E4M3, "e5m2": _b.TDG_E5M2}


def _f8_operand(t, fmt, name):
    """(dtype code, tensor) for an 8-bit operand: a float8 tensor, or a uint8
    tensor of bit patterns with its format named by `fmt`."""
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError("%s must be a 2-D row-major tensor" % name)
    if t.dtype in _F8:
        return _F8[t.dtype]
    if t.dtype == torch.uint8 and fmt in _F8_NAME:
        return _F8_NAME[fmt]
    raise ValueError("%s must be float8_e4m3fn / float8_e5m2, or uint8 with its format given" % name)


def _f8_marshal(a, b, a_fmt, b_fmt, block_scale_a, block_scale_b, scale_a, scale_b, out, out_dtype, transc):
    at = _f8_operand(a, a_fmt, "a")
    bt = _f8_operand(b, b_fmt, "b")
    M, K = a.shape
    N, Kb = b.shape
    if Kb != K:
        raise ValueError("inner dimensions differ: A has K=%d, B has K=%d" % (K, Kb))
    shape = (N, M) if transc else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype or torch.float32, device=a.device)
    if out.dtype not in _CT or tuple(out.shape) != shape or (out.size(1) > 1 and out.stride(1) != 1):
        raise ValueError("out must be a row-major %s tensor of fp16/bf16/fp32" % (shape,))

    def blk(x, rows, name):
        if x is None:
            return None, 0
        if x.dtype != torch.uint8 or x.dim() != 2 or x.size(0) != rows or (x.size(1) > 1 and x.stride(1) != 1):
            raise ValueError("%s must be a row-major uint8 (rows, ceil(K/32)) tensor of E8M0 bytes" % name)
        return x.data_ptr(), max(x.stride(0), x.size(1))

    def row(x, rows, name):
        if x is None:
            return None, 0
        if x.dtype != torch.float32 or x.dim() != 1 or x.numel() not in (1, rows):
            raise ValueError("%s must be a float32 tensor of 1 or %d entries" % (name, rows))
        return x.data_ptr(), (0 if x.numel() == 1 else x.stride(0))

    xa, ldxa = blk(block_scale_a, M, "block_scale_a")
    xb, ldxb = blk(block_scale_b, N, "block_scale_b")
    sa, inca = row(scale_a, M, "scale_a")
    sb, incb = row(scale_b, N, "scale_b")
    lda = max(a.stride(0), K, 1)
    ldb = max(b.stride(0), K, 1)
    ldc = max(out.stride(0), shape[1], 1)
    args = (int(bool(transc)), M, N, K, a.data_ptr(), lda, at, b.data_ptr(), ldb, bt, xa, ldxa, xb, ldxb,
            sa, inca, sb, incb, out.data_ptr(), ldc, _CT[out.dtype])
    return out, args


def gemm_f8(a, b, *, a_fmt=None, b_fmt=None, block_scale_a=None, block_scale_b=None, scale_a=None, scale_b=None,
            out_dtype=None, out=None, transc=False, config=-1):
    """8-bit TN product ``C = scale_a[:, None] * scale_b[None, :] * (A B^T)``
    with optional E8M0 block scales per 32 elements of K (see ``tdg.h``).

    ``a`` (M, K) and ``b`` (N, K): float8_e4m3fn / float8_e5m2 tensors, or
    uint8 bit patterns with ``a_fmt`` / ``b_fmt`` in {"e4m3", "e5m2"}.
    ``block_scale_a`` (M, ceil(K/32)) and ``block_scale_b`` (N, ceil(K/32)):
    uint8 E8M0 bytes (16-byte aligned, row stride a multiple of 16).  ``scale_a`` (M,) or (1,),
    ``scale_b`` (N,) or (1,): float32.  ``transc``: return / write C^T
    (N, M).  Returns ``out`` (a new fp32 tensor unless ``out_dtype`` or
    ``out`` say otherwise)."""
    out, args = _f8_marshal(a, b, a_fmt, b_fmt, block_scale_a, block_scale_b, scale_a, scale_b, out, out_dtype,
                            transc)
    stream = torch.cuda.current_stream(a.device).cuda_stream
    _check(_b.tdg_gemm_f8(*args, config, stream))
    return out
