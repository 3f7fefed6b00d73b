"""Float64 CPU oracle for the quantized matvec / small-M matmul family.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``matmul_affine_qmv_amd``) never imports this package.

The arithmetic lives in ``qmx_oracle.c`` (plain C, float64, built with gcc
and OpenMP); this module only builds it, loads it with ctypes and marshals
numpy arrays.  ``oracle.brute`` holds an independent exact-rational brute
force for tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmx_oracle.c")
LIB = os.path.join(HERE, "libqmx_oracle.so")

F32, F16, BF16 = 0, 1, 2

_c_i32p = ctypes.POINTER(ctypes.c_int32)


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile the oracle with gcc (OpenMP); returns the library path."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out + ".tmp", "-lm", *extra]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built; run oracle.build()")
        self.lib = lib = ctypes.CDLL(path)
        vp, ip, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
        lib.oracle_affine_groups.argtypes = [vp, vp, vp, ip, vp, ip, ip, ip, ip, ip, ip,
                                             ip, ip, vp, ip, dp]
        lib.oracle_affine.argtypes = [vp, vp, vp, ip, vp, ip, ip, ip, ip, ip, ip, vp, ip, dp]
        lib.oracle_affine_hoisted.argtypes = [vp, vp, vp, ip, vp, ip, ip, ip, ip, ip, ip, dp]
        lib.oracle_q8_0.argtypes = [vp, vp, ip, ip, vp, ip, dp]
        lib.oracle_q4_k.argtypes = [vp, vp, ip, ip, vp, ip, dp]
        lib.oracle_q8_i8.argtypes = [vp, vp, vp, ip, ip, vp, ip, dp]
        lib.oracle_round.argtypes = [dp, ctypes.c_long, ip, dp]
        lib.oracle_decode.argtypes = [vp, ctypes.c_long, ip, dp]
        lib.oracle_set_num_threads.argtypes = [ip]
        for name in ("oracle_affine_groups", "oracle_affine", "oracle_affine_hoisted",
                     "oracle_q8_0", "oracle_q4_k", "oracle_q8_i8", "oracle_round", "oracle_decode",
                     "oracle_num_threads"):
            getattr(lib, name).restype = ctypes.c_int
        lib.oracle_set_num_threads.restype = None

    # -------------------------------------------------------------- helpers
    @staticmethod
    def _p(a):
        return a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _c(a, dtype=None):
        return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))

    @staticmethod
    def _check(rc, name):
        if rc != 0:
            raise ValueError(f"{name}: invalid arguments")

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    # -------------------------------------------------------------- affine
    def _affine_common(self, w, s, b, x, M, N, K, bits):
        w = self._c(w, np.uint32)
        s, b, x = self._c(s), self._c(b), self._c(x)
        if w.size != N * K * bits // 32:
            raise ValueError("w has the wrong size")
        return w, s, b, x

    def affine(self, w, s, b, sb_dt, x, x_dt, M, N, K, bits, gs, cols=None):
        """Float64 out[M, N] (or out[M, len(cols)]) of the affine definition."""
        w, s, b, x = self._affine_common(w, s, b, x, M, N, K, bits)
        if cols is not None:
            cols = self._c(cols, np.int32)
            nc = cols.size
        else:
            nc = N
        out = np.empty((M, nc), dtype=np.float64)
        rc = self.lib.oracle_affine(self._p(w), self._p(s), self._p(b), sb_dt, self._p(x), x_dt,
                                    M, N, K, bits, gs,
                                    self._p(cols) if cols is not None else None, nc, self._p(out))
        self._check(rc, "oracle_affine")
        return out

    def affine_groups(self, w, s, b, sb_dt, x, x_dt, M, N, K, bits, gs, g0, g1, cols=None):
        w, s, b, x = self._affine_common(w, s, b, x, M, N, K, bits)
        if cols is not None:
            cols = self._c(cols, np.int32)
            nc = cols.size
        else:
            nc = N
        out = np.empty((M, nc), dtype=np.float64)
        rc = self.lib.oracle_affine_groups(self._p(w), self._p(s), self._p(b), sb_dt, self._p(x),
                                           x_dt, M, N, K, bits, gs, g0, g1,
                                           self._p(cols) if cols is not None else None, nc,
                                           self._p(out))
        self._check(rc, "oracle_affine_groups")
        return out

    def affine_hoisted(self, w, s, b, sb_dt, x, x_dt, M, N, K, bits, gs):
        w, s, b, x = self._affine_common(w, s, b, x, M, N, K, bits)
        out = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_affine_hoisted(self._p(w), self._p(s), self._p(b), sb_dt, self._p(x),
                                            x_dt, M, N, K, bits, gs, self._p(out))
        self._check(rc, "oracle_affine_hoisted")
        return out

    def affine_case(self, case, cols=None):
        """Oracle of a ``qmx_inputs.affine_case`` dict."""
        return self.affine(case["w"], case["scales"], case["biases"], case["dtype"], case["x"],
                           case["dtype"], case["M"], case["N"], case["K"], case["bits"],
                           case["gs"], cols=cols)

    # -------------------------------------------------------------- blocks
    def q8_0(self, blocks, x, N, K, rows=None):
        blocks = self._c(blocks, np.uint32)
        x = self._c(x, np.float32)
        nr = N if rows is None else len(rows)
        rws = None if rows is None else self._c(rows, np.int32)
        out = np.empty(nr, dtype=np.float64)
        rc = self.lib.oracle_q8_0(self._p(blocks), self._p(x), N, K,
                                  None if rws is None else self._p(rws), nr, self._p(out))
        self._check(rc, "oracle_q8_0")
        return out

    def q4_k(self, blocks, x, N, K, rows=None):
        blocks = self._c(blocks, np.uint32)
        x = self._c(x, np.float32)
        nr = N if rows is None else len(rows)
        rws = None if rows is None else self._c(rows, np.int32)
        out = np.empty(nr, dtype=np.float64)
        rc = self.lib.oracle_q4_k(self._p(blocks), self._p(x), N, K,
                                  None if rws is None else self._p(rws), nr, self._p(out))
        self._check(rc, "oracle_q4_k")
        return out

    def q8_i8(self, wq, xq, wd, N, K, rows=None):
        """Integer-activation matvec: packed int8 weights and activations, float32 block scales."""
        wq = self._c(wq, np.uint32)
        xq = self._c(xq, np.uint32)
        wd = self._c(wd, np.float32)
        nr = N if rows is None else len(rows)
        rws = None if rows is None else self._c(rows, np.int32)
        out = np.empty(nr, dtype=np.float64)
        rc = self.lib.oracle_q8_i8(self._p(wq), self._p(xq), self._p(wd), N, K,
                                   None if rws is None else self._p(rws), nr, self._p(out))
        self._check(rc, "oracle_q8_i8")
        return out

    # -------------------------------------------------------------- rounding
    def round(self, v, dt):
        """Round float64 values to storage dtype ``dt`` (RNE); float64 result."""
        v = self._c(v, np.float64)
        out = np.empty_like(v)
        self._check(self.lib.oracle_round(self._p(v), v.size, dt, self._p(out)), "oracle_round")
        return out

    def decode(self, a, dt):
        a = self._c(a)
        out = np.empty(a.shape, dtype=np.float64)
        self._check(self.lib.oracle_decode(self._p(a), a.size, dt, self._p(out)), "oracle_decode")
        return out


_default = None


def load(path: str = LIB, rebuild_if_missing: bool = True) -> Oracle:
    """The oracle library next to this file (built on first use if missing)."""
    global _default
    if path == LIB and _default is not None:
        return _default
    if not os.path.exists(path) and rebuild_if_missing and path == LIB:
        build()
    o = Oracle(path)
    if path == LIB:
        _default = o
    return o
