"""Exact rational brute force for tiny inputs.

TEST INFRASTRUCTURE ONLY (used to pin the float64 oracle).  Pure-Python
loops with ``fractions.Fraction``: every stored value is a dyadic rational,
so the sums below are exact.  The bit fields are read differently from the
C oracle: each row (or block) is turned into one Python integer and fields
are cut out of it with shifts, and f16 values are decoded by numpy, not by
hand.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32, F16, BF16 = 0, 1, 2


def exact_values(a, dt):
    """Storage array -> flat list of Fractions."""
    a = np.asarray(a)
    if dt == F32:
        vals = a.astype(np.float32).ravel()
    elif dt == F16:
        vals = a.view(np.float16).ravel() if a.dtype != np.float16 else a.ravel()
    else:
        vals = (a.astype(np.uint32).ravel() << 16).view(np.float32)
    return [Fraction(float(v)) for v in vals]


def _row_int(words):
    """Row of uint32 words -> one integer, word 0 least significant."""
    v = 0
    for i, wd in enumerate(np.asarray(words, dtype=np.uint64).tolist()):
        v |= int(wd) << (32 * i)
    return v


def affine_exact(w, s, b, x, dt, M, N, K, bits, gs):
    """Exact out[m][n] = sum_k x[m,k] * (s[n,k//gs] * q[n,k] + b[n,k//gs])."""
    w = np.asarray(w, dtype=np.uint32).reshape(N, K * bits // 32)
    S, B, X = exact_values(s, dt), exact_values(b, dt), exact_values(x, dt)
    G = K // gs
    mask = (1 << bits) - 1
    out = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        stream = _row_int(w[n])
        q = [(stream >> (k * bits)) & mask for k in range(K)]
        for m in range(M):
            tot = Fraction(0)
            for k in range(K):
                g = k // gs
                tot += X[m * K + k] * (S[n * G + g] * q[k] + B[n * G + g])
            out[m][n] = tot
    return out


def q8_0_exact(blocks, x, N, K):
    blocks = np.asarray(blocks, dtype=np.uint32).reshape(N, K // 32, 9)
    X = [Fraction(float(v)) for v in np.asarray(x, dtype=np.float32)]
    out = []
    for n in range(N):
        tot = Fraction(0)
        for j in range(K // 32):
            wd = blocks[n, j]
            d = Fraction(float(np.array([wd[0] & 0xFFFF], dtype=np.uint16).view(np.float16)[0]))
            quants = _row_int(wd[1:]).to_bytes(32, "little")
            part = Fraction(0)
            for i, byte in enumerate(quants):
                qv = byte - 256 if byte >= 128 else byte
                part += qv * X[32 * j + i]
            tot += d * part
        out.append(tot)
    return out


def q8_i8_exact(wq, xq, wd, N, K):
    """Integer-activation matvec in exact rationals, from the raw words: signed
    bytes taken from each word's little-endian byte string."""
    wq = np.asarray(wq, dtype=np.uint32).reshape(N, K // 4)
    xbytes = b"".join(int(w).to_bytes(4, "little") for w in np.asarray(xq, dtype=np.uint32))
    xv = [v - 256 if v >= 128 else v for v in xbytes]
    scales = np.asarray(wd, dtype=np.float32).reshape(N, K // 32)
    out = []
    for n in range(N):
        wbytes = b"".join(int(w).to_bytes(4, "little") for w in wq[n])
        wv = [v - 256 if v >= 128 else v for v in wbytes]
        tot = Fraction(0)
        for b in range(K // 32):
            tot += Fraction(float(scales[n, b])) * sum(wv[i] * xv[i] for i in range(32 * b, 32 * b + 32))
        out.append(tot)
    return out


def q4_k_sub_scales(scale_bytes):
    """The eight (scale, min) 6-bit pairs of one Q4_K super-block.

    Written as a field map rather than as the page's byte formula: for
    sub-blocks 0-3 the scale and min are the low six bits of bytes j and j+4;
    for sub-blocks 4-7 the low four bits of the scale are the low nibble of
    byte j+4, the low four bits of the min its high nibble, and the top two
    bits of each come from the top two bits of bytes j-4 (scale) and j (min).
    """
    sb = list(scale_bytes)
    bitstr = [[(sb[i] >> t) & 1 for t in range(8)] for i in range(12)]

    def bits_to_int(lst):
        return sum(bit << t for t, bit in enumerate(lst))

    pairs = []
    for j in range(8):
        if j < 4:
            sc = bits_to_int(bitstr[j][0:6])
            mn = bits_to_int(bitstr[j + 4][0:6])
        else:
            sc = bits_to_int(bitstr[j + 4][0:4] + bitstr[j - 4][6:8])
            mn = bits_to_int(bitstr[j + 4][4:8] + bitstr[j][6:8])
        pairs.append((sc, mn))
    return pairs


def q4_k_weights_exact(block_words):
    """Dequantised weights (Fractions) of one 36-word Q4_K super-block, in element order."""
    raw = _row_int(block_words).to_bytes(144, "little")
    d = Fraction(float(np.frombuffer(raw[0:2], dtype="<f2")[0]))
    dmin = Fraction(float(np.frombuffer(raw[2:4], dtype="<f2")[0]))
    pairs = q4_k_sub_scales(raw[4:16])
    qs = raw[16:144]
    wts = [None] * 256
    for e in range(256):
        chunk, r = divmod(e, 64)          # 64 elements per 32 quant bytes
        hi, i = divmod(r, 32)             # first 32: low nibbles, next 32: high nibbles
        byte = qs[32 * chunk + i]
        qv = (byte >> 4) if hi else (byte & 15)
        sc, mn = pairs[2 * chunk + hi]
        wts[e] = d * sc * qv - dmin * mn
    return wts


def q4_k_exact(blocks, x, N, K):
    blocks = np.asarray(blocks, dtype=np.uint32).reshape(N, K // 256, 36)
    X = [Fraction(float(v)) for v in np.asarray(x, dtype=np.float32)]
    out = []
    for n in range(N):
        tot = Fraction(0)
        for blk in range(K // 256):
            wts = q4_k_weights_exact(blocks[n, blk])
            for e in range(256):
                tot += wts[e] * X[256 * blk + e]
        out.append(tot)
    return out
