"""Thin Python binding of libqmx (include/qmx.h).

Argument marshalling only: every function checks tensor placement, dtype,
shape and contiguity, allocates the output if none is given, and calls the
C ABI on torch's current HIP stream.  All arithmetic runs in the HIP
kernels; there is no CPU fallback.  A missing ``libqmx.so`` raises.

Dtypes: ``torch.float32``, ``torch.float16`` and ``torch.bfloat16`` map to
QMX_F32, QMX_F16 and QMX_BF16.  Packed weights are ``torch.int32`` or
``torch.uint32`` tensors holding the uint32 words bit for bit.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmx.so")

QMX_F32, QMX_F16, QMX_BF16 = 0, 1, 2
QMX_ROUTE_QMV, QMX_ROUTE_QMM_T, QMX_ROUTE_QMM_T_SPLITK = 0, 1, 2
QMX_MAX_SPLITS = 16
ROUTE_NAMES = {0: "qmv", 1: "qmm_t", 2: "qmm_t_splitk"}

_TORCH_TO_QMX = {torch.float32: QMX_F32, torch.float16: QMX_F16, torch.bfloat16: QMX_BF16}
_QMX_TO_TORCH = {v: k for k, v in _TORCH_TO_QMX.items()}
_WORD_DTYPES = (torch.int32, getattr(torch, "uint32", torch.int32))

_lib = None

_EXPORTS = {
    # name: (restype, argtypes)
    "qmx_qmv": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_void_p]),
    "qmx_qmm_t": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_void_p]),
    "qmx_qmm_t_splitk": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7
                         + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qmx_qmm_t_partials": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 7
                           + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qmx_splitk_accumulate": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 4 + [ctypes.c_void_p]),
    "qmx_splitk_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "qmx_qmm_t_splitk_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [ctypes.c_void_p]),
    "qmx_matvec_q8_0": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_void_p]),
    "qmx_matvec_q4_k": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_void_p]),
    "qmx_matvec_q8_i8": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 2 + [ctypes.c_void_p]),
    "qmx_plan": (ctypes.c_int, [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_int)] * 2),
    "qmx_qmm_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "qmx_qmm": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6
                + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qmx_qmm_batched": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_longlong] * 4
                        + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qmx_qmm_batched_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 7 + [ctypes.c_void_p]
                                        + [ctypes.c_longlong] * 2),
    "qmx_plan_batched": (ctypes.c_int, [ctypes.c_int] * 8 + [ctypes.POINTER(ctypes.c_int)] * 2),
    "qmx_qmm_gather": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 6 + [ctypes.c_longlong] * 4
                       + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qmx_qmm_gather_sorted": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 6 + [ctypes.c_longlong] * 4
                              + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qmx_qmm_gather_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 8 + [ctypes.c_void_p]
                                       + [ctypes.c_longlong] * 2),
    "qmx_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "qmx_api_version": (ctypes.c_int, []),
}


class QmxError(RuntimeError):
    """A negative qmx_status returned by the library."""

    def __init__(self, status: int, func: str):
        self.status = status
        super().__init__(f"{func}: {strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libqmx (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m matmul_affine_qmv_amd.build` "
                               "(or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(status: int) -> str:
    return lib().qmx_strerror(int(status)).decode()


def api_version() -> int:
    return lib().qmx_api_version()


def _check(status: int, func: str) -> None:
    if status != 0:
        raise QmxError(status, func)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _TORCH_TO_QMX[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _need_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")


def _affine_args(w_packed, scales, biases, x, bits, group_size, out, need_out=True):
    if x.dim() != 2 or w_packed.dim() != 2:
        raise ValueError("x must be [M, K] and w_packed [N, K*bits/32]")
    if w_packed.dtype not in _WORD_DTYPES:
        raise ValueError("w_packed must hold uint32 words (torch.int32 or torch.uint32)")
    M, K = x.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 32 != K * bits:
        raise ValueError(f"w_packed has {w_packed.shape[1]} words per row; K={K} at {bits} bits needs "
                         f"{K * bits / 32}")
    G = K // group_size if group_size else 0
    for name, t in (("scales", scales), ("biases", biases)):
        if tuple(t.shape) != (N, G):
            raise ValueError(f"{name} must be [N, K/group_size] = {(N, G)}, got {tuple(t.shape)}")
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype {x.dtype}")
    if not need_out:
        _need_cuda(w_packed, scales, biases, x)
        return M, N, K, None
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (M, N) or out.dtype != x.dtype:
        raise ValueError(f"out must be [M, N] = {(M, N)} of dtype {x.dtype}")
    _need_cuda(w_packed, scales, biases, x, out)
    return M, N, K, out


def qmv(w_packed, scales, biases, x, out=None, *, bits=4, group_size=64):
    """out[M, N] = x @ dequant(W).T via qmx_qmv."""
    M, N, K, out = _affine_args(w_packed, scales, biases, x, bits, group_size, out)
    _check(lib().qmx_qmv(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N, K, bits,
                         group_size, _dtype_code(x), _stream(x)), "qmx_qmv")
    return out


def qmm_t(w_packed, scales, biases, x, out=None, *, bits=4, group_size=64):
    """out[M, N] = x @ dequant(W).T via qmx_qmm_t (matrix cores, unsplit)."""
    M, N, K, out = _affine_args(w_packed, scales, biases, x, bits, group_size, out)
    _check(lib().qmx_qmm_t(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N, K, bits,
                           group_size, _dtype_code(x), _stream(x)), "qmx_qmm_t")
    return out


def splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    return lib().qmx_splitk_workspace_bytes(M, N, splits)


def _workspace(x, nbytes, workspace):
    if workspace is None:
        return torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=x.device)
    _need_cuda(workspace)
    return workspace


def qmm_t_splitk(w_packed, scales, biases, x, out=None, *, bits=4, group_size=64, splits=2, workspace=None):
    """out[M, N] via qmx_qmm_t_splitk (float32 partials + accumulate kernel)."""
    M, N, K, out = _affine_args(w_packed, scales, biases, x, bits, group_size, out)
    need = splitk_workspace_bytes(M, N, splits)
    workspace = _workspace(x, need, workspace)
    _check(lib().qmx_qmm_t_splitk(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N, K,
                                  bits, group_size, _dtype_code(x), splits, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(x)),
           "qmx_qmm_t_splitk")
    return out


def qmm_t_splitk_noalloc(w_packed, scales, biases, x, out=None, *, bits=4, group_size=64, splits=2):
    """out[M, N] via qmx_qmm_t_splitk_noalloc: qmm_t_splitk with the partials in
    the library's per-device scratch array (no workspace, nothing allocated
    beyond `out` when the caller passes none)."""
    M, N, K, out = _affine_args(w_packed, scales, biases, x, bits, group_size, out)
    _check(lib().qmx_qmm_t_splitk_noalloc(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N, K,
                                          bits, group_size, _dtype_code(x), splits, _stream(x)),
           "qmx_qmm_t_splitk_noalloc")
    return out


def qmm_t_partials(w_packed, scales, biases, x, *, bits=4, group_size=64, splits=2, workspace=None):
    """float32 split-K partials [splits, M, N] via qmx_qmm_t_partials (the first
    kernel of qmm_t_splitk alone)."""
    M, N, K, _ = _affine_args(w_packed, scales, biases, x, bits, group_size, None, need_out=False)
    need = splitk_workspace_bytes(M, N, splits)
    workspace = _workspace(x, need, workspace)
    _check(lib().qmx_qmm_t_partials(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), M, N, K, bits,
                                    group_size, _dtype_code(x), splits, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(x)),
           "qmx_qmm_t_partials")
    return workspace.view(-1)[: splits * M * N].view(splits, M, N)


def splitk_accumulate(workspace, out, splits):
    """out[M, N] = the float32 partials summed over the split axis in order and
    rounded once (qmx_splitk_accumulate)."""
    if not (workspace.is_cuda and out.is_cuda):
        raise ValueError("splitk_accumulate: tensors must be on the GPU")
    if workspace.dtype != torch.float32 or not workspace.is_contiguous() or not out.is_contiguous():
        raise ValueError("splitk_accumulate: contiguous float32 workspace and contiguous out required")
    M, N = out.shape
    if workspace.numel() < splits * M * N:
        raise ValueError("splitk_accumulate: workspace smaller than splits * M * N")
    _check(lib().qmx_splitk_accumulate(_ptr(workspace), _ptr(out), M, N, splits, _dtype_code(out), _stream(out)),
           "qmx_splitk_accumulate")
    return out


def plan(M, N, K, bits=4, group_size=64, dtype=QMX_BF16, num_cus=0):
    """(route_name, splits) the dispatch policy picks (pure host call)."""
    if isinstance(dtype, torch.dtype):
        dtype = _TORCH_TO_QMX[dtype]
    route, splits = ctypes.c_int(-1), ctypes.c_int(-1)
    _check(lib().qmx_plan(M, N, K, bits, group_size, dtype, num_cus, ctypes.byref(route),
                          ctypes.byref(splits)), "qmx_plan")
    return ROUTE_NAMES[route.value], splits.value


def qmm_workspace_bytes(M, N, K, bits=4, group_size=64, dtype=QMX_BF16) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = _TORCH_TO_QMX[dtype]
    return lib().qmx_qmm_workspace_bytes(M, N, K, bits, group_size, dtype)


def qmm(w_packed, scales, biases, x, out=None, *, bits=4, group_size=64, workspace=None):
    """Policy-dispatched quantized matmul (qmx_qmm)."""
    M, N, K, out = _affine_args(w_packed, scales, biases, x, bits, group_size, out)
    need = qmm_workspace_bytes(M, N, K, bits, group_size, _dtype_code(x))
    if need and workspace is None:
        workspace = _workspace(x, need, None)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().qmx_qmm(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N, K, bits,
                         group_size, _dtype_code(x), ws_ptr, ws_bytes, _stream(x)), "qmx_qmm")
    return out


def plan_batched(batch, M, N, K, bits=4, group_size=64, dtype=QMX_BF16, num_cus=0):
    """(route_name, splits) the dispatch policy picks for a batch (pure host call)."""
    if isinstance(dtype, torch.dtype):
        dtype = _TORCH_TO_QMX[dtype]
    route, splits = ctypes.c_int(-1), ctypes.c_int(-1)
    _check(lib().qmx_plan_batched(batch, M, N, K, bits, group_size, dtype, num_cus, ctypes.byref(route),
                                  ctypes.byref(splits)), "qmx_plan_batched")
    return ROUTE_NAMES[route.value], splits.value


def qmm_batched(w_packed, scales, biases, x, out=None, *, bits=4, group_size=64, workspace=None):
    """Batched quantized matmul (qmx_qmm_batched).

    x: [B, M, K] with unit last stride; its batch and row strides and storage
    offset are passed as they are (rows need not be 16-byte aligned: the
    library then copies x into the workspace first).  w_packed [B, N, K*bits/32]
    and scales/biases [B, N, K/group_size], each matrix contiguous, or 2-D to
    share one matrix across the batch.  out: contiguous [B, M, N]."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [B, M, K] with a unit last stride")
    B, M, K = x.shape
    if w_packed.dtype not in _WORD_DTYPES:
        raise ValueError("w_packed must hold uint32 words (torch.int32 or torch.uint32)")
    if w_packed.dim() not in (2, 3) or (w_packed.dim() == 3 and w_packed.shape[0] != B):
        raise ValueError("w_packed must be [N, K*bits/32] or [B, N, K*bits/32]")
    N, words = w_packed.shape[-2], w_packed.shape[-1]
    if words * 32 != K * bits:
        raise ValueError(f"w_packed rows hold {words} words; K={K} at {bits} bits needs {K * bits / 32}")
    G = K // group_size if group_size else 0

    def batch_stride(t, inner, name):
        if t.dim() == 2:
            if tuple(t.shape) != inner:
                raise ValueError(f"{name} must be {inner} or {(B,) + inner}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            return 0
        if t.dim() != 3 or tuple(t.shape) != (B,) + inner:
            raise ValueError(f"{name} must be {inner} or {(B,) + inner}")
        if t.stride(2) != 1 or t.stride(1) != inner[1]:
            raise ValueError(f"each matrix of {name} must be contiguous")
        return t.stride(0) if B > 1 else 0

    wbs = batch_stride(w_packed, (N, K * bits // 32), "w_packed")
    sbs = batch_stride(scales, (N, G), "scales")
    if batch_stride(biases, (N, G), "biases") != sbs:
        raise ValueError("scales and biases must share their batch stride")
    for name, t in (("scales", scales), ("biases", biases)):
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype {x.dtype}")
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, M, N) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [B, M, N] = {(B, M, N)} of dtype {x.dtype}")
    for t in (w_packed, scales, biases, x, out):
        if not t.is_cuda or t.device != x.device:
            raise ValueError("all tensors must be on x's HIP device")
    xs = x.stride(0) if B > 1 else 0
    xr = x.stride(1) if M > 1 else K
    dt = _dtype_code(x)
    need = lib().qmx_qmm_batched_workspace_bytes(B, M, N, K, bits, group_size, dt, _ptr(x), xs, xr)
    if need and workspace is None:
        workspace = _workspace(x, need, None)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().qmx_qmm_batched(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), B, M, N, K,
                                 wbs, sbs, xs, xr, bits, group_size, dt, ws_ptr, ws_bytes, _stream(x)),
           "qmx_qmm_batched")
    return out


def gather_qmm(w_packed, scales, biases, x, w_index=None, x_index=None, out=None, *, bits=4, group_size=64,
               workspace=None, sorted_indices=False):
    """Gathered quantized matmul (qmx_qmm_gather): out[i] = x[x_index[i]] @
    dequant(W[w_index[i]]).T.  w_packed [E, N, K*bits/32] and scales/biases
    [E, N, K/group_size] (each matrix contiguous); x [X, M, K] with a unit last
    stride (any batch/row stride and offset); w_index, x_index: int32 device
    vectors of one length B (None: identity, then that operand has B matrices);
    out: contiguous [B, M, N].  sorted_indices: w_index holds runs of equal
    values (qmx_qmm_gather_sorted; the same results for any indices)."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [X, M, K] with a unit last stride")
    if w_packed.dim() != 3 or scales.dim() != 3 or biases.dim() != 3:
        raise ValueError("w_packed, scales and biases must be 3-D [E, ...]")
    if w_packed.dtype not in _WORD_DTYPES:
        raise ValueError("w_packed must hold uint32 words (torch.int32 or torch.uint32)")
    X, M, K = x.shape
    E, N, words = w_packed.shape
    if words * 32 != K * bits:
        raise ValueError(f"w_packed rows hold {words} words; K={K} at {bits} bits needs {K * bits / 32}")
    G = K // group_size if group_size else 0
    for name, t in (("scales", scales), ("biases", biases)):
        if tuple(t.shape) != (E, N, G) or t.stride(2) != 1 or t.stride(1) != G:
            raise ValueError(f"{name} must be [E, N, K/group_size] = {(E, N, G)} with contiguous matrices")
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype {x.dtype}")
    if w_packed.stride(2) != 1 or w_packed.stride(1) != words:
        raise ValueError("each matrix of w_packed must be contiguous")
    if scales.stride(0) != biases.stride(0):
        raise ValueError("scales and biases must share their batch stride")
    lengths = {t.shape[0] for t in (w_index, x_index) if t is not None}
    for t in (w_index, x_index):
        if t is not None and (t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous()):
            raise ValueError("indices must be contiguous int32 vectors")
    if len(lengths) > 1:
        raise ValueError("w_index and x_index must have one length")
    B = lengths.pop() if lengths else E
    if w_index is None and E != B:
        raise ValueError("without w_index, w_packed must hold one matrix per problem")
    if x_index is None and X != B:
        raise ValueError("without x_index, x must hold one matrix per problem")
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, M, N) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [B, M, N] = {(B, M, N)} of dtype {x.dtype}")
    for t in (w_packed, scales, biases, x, out, w_index, x_index):
        if t is not None and (not t.is_cuda or t.device != x.device):
            raise ValueError("all tensors must be on x's HIP device")
    xs = x.stride(0) if X > 1 else 0
    xr = x.stride(1) if M > 1 else K
    dt = _dtype_code(x)
    need = lib().qmx_qmm_gather_workspace_bytes(B, X, M, N, K, bits, group_size, dt, _ptr(x), xs, xr)
    if need and workspace is None:
        workspace = _workspace(x, need, None)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    name = "qmx_qmm_gather_sorted" if sorted_indices else "qmx_qmm_gather"
    _check(getattr(lib(), name)(_ptr(w_packed), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), _ptr(w_index),
                                _ptr(x_index), E, X, B, M, N, K, w_packed.stride(0) if E > 1 else 0,
                                scales.stride(0) if E > 1 else 0, xs, xr, bits, group_size, dt, ws_ptr, ws_bytes,
                                _stream(x)), name)
    return out


def _block_args(w_blocks, x, out, words_per_block, weights_per_block):
    if x.dim() != 1 or x.dtype != torch.float32:
        raise ValueError("x must be a float32 vector [K]")
    if w_blocks.dim() != 2 or w_blocks.dtype not in _WORD_DTYPES:
        raise ValueError("w_blocks must be uint32 words [N, blocks*words]")
    K = x.shape[0]
    N = w_blocks.shape[0]
    if w_blocks.shape[1] * weights_per_block != K * words_per_block:
        raise ValueError("w_blocks row length does not match K")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != (N,) or out.dtype != torch.float32:
        raise ValueError("out must be a float32 vector [N]")
    _need_cuda(w_blocks, x, out)
    return N, K, out


def matvec_q8_0(w_blocks, x, out=None):
    """out[N] = Q8_0 matvec (9 words per 32-weight block)."""
    N, K, out = _block_args(w_blocks, x, out, 9, 32)
    _check(lib().qmx_matvec_q8_0(_ptr(w_blocks), _ptr(x), _ptr(out), N, K, _stream(x)), "qmx_matvec_q8_0")
    return out


def matvec_q4_k(w_blocks, x, out=None):
    """out[N] = Q4_K matvec (36 words per 256-weight super-block)."""
    N, K, out = _block_args(w_blocks, x, out, 36, 256)
    _check(lib().qmx_matvec_q4_k(_ptr(w_blocks), _ptr(x), _ptr(out), N, K, _stream(x)), "qmx_matvec_q4_k")
    return out


def matvec_q8_i8(wq, xq, wd, out=None):
    """Integer-activation matvec: wq [N, K/4] and xq [K/4] int32 words holding
    four int8 each, wd float32 [N, K/32]; out float32 [N]."""
    if wq.dim() != 2 or xq.dim() != 1 or wq.dtype not in _WORD_DTYPES or xq.dtype not in _WORD_DTYPES:
        raise ValueError("wq must be [N, K/4] and xq [K/4] uint32 words (torch.int32 or torch.uint32)")
    N, K = wq.shape[0], 4 * xq.shape[0]
    if wq.shape[1] * 4 != K:
        raise ValueError("wq rows and xq must hold the same K")
    if wd.dtype != torch.float32 or tuple(wd.shape) != (N, K // 32):
        raise ValueError(f"wd must be float32 [N, K/32] = {(N, K // 32)}")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=xq.device)
    elif tuple(out.shape) != (N,) or out.dtype != torch.float32:
        raise ValueError("out must be a float32 vector [N]")
    _need_cuda(wq, xq, wd, out)
    _check(lib().qmx_matvec_q8_i8(_ptr(wq), _ptr(xq), _ptr(wd), _ptr(out), N, K, _stream(xq)), "qmx_matvec_q8_i8")
    return out


def words_tensor(a, device) -> torch.Tensor:
    """numpy uint32 array -> int32 tensor with the same bits on `device`."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)


def storage_tensor(a, dtype_code: int, device) -> torch.Tensor:
    """numpy storage array (float32, float16, or uint16 bf16 bits) -> torch tensor on `device`."""
    import numpy as np
    a = np.ascontiguousarray(a)
    if dtype_code == QMX_F32:
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if dtype_code == QMX_F16:
        return torch.from_numpy(a.astype(np.float16)).to(device)
    return torch.from_numpy(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def tensor_bits(t: torch.Tensor):
    """Device tensor -> numpy storage array (float32, float16 or uint16 bf16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


__all__ = ["qmv", "qmm_t", "qmm_t_splitk", "qmm_t_splitk_noalloc", "qmm", "qmm_batched", "gather_qmm", "plan", "plan_batched",
           "matvec_q8_0",
           "matvec_q4_k", "matvec_q8_i8",
           "splitk_workspace_bytes", "qmm_workspace_bytes", "strerror", "api_version", "lib",
           "QmxError", "words_tensor", "storage_tensor", "tensor_bits",
           "QMX_F32", "QMX_F16", "QMX_BF16"]
