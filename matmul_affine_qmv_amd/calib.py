"""ctypes binding of libqmx_calib.so (include/qmx_calib.h): streaming-read,
copy, matrix-core and empty-launch kernels that calibrate measurements.

Argument marshalling only; the kernels are in ``csrc/calib.hip``.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmx_calib.so")

EXPORTS = {
    "qmxc_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int,
                                 ctypes.c_void_p]),
    "qmxc_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]),
    "qmxc_mfma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "qmxc_mfma_valu": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p]),
    "qmxc_empty": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p]),
}
MFMA_VALU_FMAS = (0, 2, 4, 6, 8, 10, 12, 16)
FLOPS_PER_WAVE_ROUND = 8 * 2 * 16 * 16 * 32   # = 4 * 2 * 32 * 32 * 16

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m matmul_affine_qmv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed ({rc})")


def read(src: torch.Tensor, sink: torch.Tensor, blocks: int, never: int = 0x9E3779B9) -> None:
    """One streaming read of every byte of ``src`` (16-byte multiple)."""
    _check(lib().qmxc_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), never, blocks,
                           _stream()), "qmxc_read")


def copy(src: torch.Tensor, dst: torch.Tensor, blocks: int) -> None:
    _check(lib().qmxc_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), blocks, _stream()),
           "qmxc_copy")


def mfma(out: torch.Tensor, iters: int, blocks: int, shape: int = 32) -> None:
    """``blocks`` x 4 waves, each issuing ``iters`` rounds of bf16 MFMAs of the
    16x16x32 (shape 16) or 32x32x16 (shape 32) form (writes blocks*256 floats)."""
    _check(lib().qmxc_mfma(out.data_ptr(), iters, blocks, shape, _stream()), "qmxc_mfma")


def mfma_flops(iters: int, blocks: int) -> int:
    return blocks * 4 * iters * FLOPS_PER_WAVE_ROUND


def mfma_valu(out: torch.Tensor, iters: int, blocks: int, fmas: int, with_mfma: bool = True) -> None:
    """``blocks`` x 4 waves, each issuing ``iters`` rounds of four independent
    32x32x16 bf16 MFMAs, each followed by ``fmas`` independent float32 FMAs (or
    the FMAs alone); writes blocks*256 floats."""
    _check(lib().qmxc_mfma_valu(out.data_ptr(), iters, blocks, fmas, int(with_mfma), _stream()), "qmxc_mfma_valu")


def empty(blocks: int = 1) -> None:
    _check(lib().qmxc_empty(blocks, _stream()), "qmxc_empty")
