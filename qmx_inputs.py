"""Seeded synthetic inputs shared by the tests, smoke() and bench.py.

This module only draws random numbers, rounds them to the storage dtypes and
lays integer codes out in the documented bit layouts.  It holds none of the
method's arithmetic: no dequantisation, no dot product, no reduction.  The
oracle and the HIP library each decode what is produced here on their own.

Layouts (pages: "metaltile-std src/mlx/quantized.rs", qmv kernel header and
int8 kernel comments; "hanzo-kernel src/quant.rs", Q8_0 packed layout and
Q4_K block comments):

* affine ``w_packed``: uint32 ``[N, K*bits/32]``; each row is a little-endian
  bit stream, element ``k`` occupies bits ``[k*bits, (k+1)*bits)`` of the row
  stream, so for 4-bit codes element ``i`` sits at bits ``4*(i%8)`` of word
  ``i//8`` (low nibble first) and for 8-bit codes byte ``j`` of a word holds
  element ``4*word + j``.  The same stream carries the other widths the
  staged loader of page "mlx PR 4682" takes (1, 3, 5 and 6 bits); 3-, 5- and
  6-bit fields may straddle two words.
* Q8_0: 9 uint32 per 32-weight block; word 0 holds the f16 scale in its low
  16 bits (high half zero), words 1..8 hold the 32 signed int8 quants, four
  per word, quant ``i`` at byte ``i%4`` of word ``1 + i//4``.
* Q4_K: 36 uint32 (144 bytes) per 256-weight super-block: bytes 0-1 f16
  ``d``, bytes 2-3 f16 ``dmin``, bytes 4-15 the 12 packed 6-bit scale/min
  bytes, bytes 16-143 the 128 bytes of 4-bit quants.

Random draws use numpy ``PCG64``; integer codes and quant bytes are random
bytes (b-bit codes are their low b bits, so every code value is equally
likely; Q8_0 bytes equal to -128 are drawn again); values are drawn in f32
and rounded round-to-nearest-even to the storage dtype.  Draw order: codes,
scales, bias jitter, x.
"""
from __future__ import annotations

import math

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
DTYPE_NAMES = {v: k for k, v in DTYPES.items()}
BASE_SEED = 20261202


def seed_for(config: int, case: int) -> int:
    """Seed of case ``case`` of workload family ``config``."""
    return BASE_SEED + 1000 * config + case


def dtype_code(dt) -> int:
    if isinstance(dt, str):
        return DTYPES[dt]
    return int(dt)


# ---------------------------------------------------------------- storage
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a_f32, dt) -> np.ndarray:
    """f32 values -> storage array: float32, float16, or uint16 bf16 bits."""
    dt = dtype_code(dt)
    a = np.asarray(a_f32, dtype=np.float32)
    if dt == F32:
        return a.copy()
    if dt == F16:
        return a.astype(np.float16)
    return f32_to_bf16_bits(a)


def storage_to_f64(a, dt) -> np.ndarray:
    """Decode a storage array to float64 (exact for all three dtypes)."""
    dt = dtype_code(dt)
    if dt == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


# ---------------------------------------------------------------- layouts
def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack unsigned codes ``[N, K]`` into row bit streams of uint32 words:
    element k at stream bits [k*bits, (k+1)*bits), word 0 holding stream bits
    0..31, so 3-, 5- and 6-bit fields may straddle two words."""
    codes = np.asarray(codes)
    n, k = codes.shape
    if not 1 <= bits <= 8:
        raise ValueError("bits must be 1..8")
    if (k * bits) % 32:
        raise ValueError("K*bits must be a multiple of 32")
    if 32 % bits == 0:
        per = 32 // bits
        out = np.zeros((n, k // per), dtype=np.uint32)
        for j in range(per):
            out |= codes[:, j::per].astype(np.uint32) << np.uint32(bits * j)
        return out
    # a period of P codes fills exactly P*bits/32 words; place element i of every period
    P = 32 // math.gcd(32, bits)
    out = np.zeros((n, k // P, P * bits // 32), dtype=np.uint64)
    for i in range(P):
        bit = i * bits
        v = codes[:, i::P].astype(np.uint64) << np.uint64(bit & 31)
        out[:, :, bit >> 5] |= v & np.uint64(0xFFFFFFFF)
        if (bit & 31) + bits > 32:
            out[:, :, (bit >> 5) + 1] |= v >> np.uint64(32)
    return out.reshape(n, k * bits // 32).astype(np.uint32)


def random_codes(rng, shape, bits: int) -> np.ndarray:
    """Codes uniform on 0..2^bits-1: the low ``bits`` bits of random bytes."""
    n = int(np.prod(shape))
    raw = np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape)
    return raw & np.uint8((1 << bits) - 1)


def random_bytes(rng, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def bytes_to_words(b) -> np.ndarray:
    """Little-endian bytes ``[..., 4*n]`` -> uint32 words ``[..., n]``."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return b.view("<u4").astype(np.uint32)


# ---------------------------------------------------------------- affine
def affine_case(M, N, K, bits, gs, dtype, seed, bias="jitter", x_dist="normal"):
    """Group-wise affine problem: uniform codes, scales U(0.002, 0.02),
    bias = -2^(bits-1)*scale*(1+U(-0.1,0.1)) ("jitter") or -2^(bits-1)*scale
    ("exact"), x ~ N(0, 1).  All of x, scales and biases share ``dtype``."""
    dt = dtype_code(dtype)
    if K % gs:
        raise ValueError("K must be a multiple of group_size")
    rng = np.random.Generator(np.random.PCG64(seed))
    G = K // gs
    codes = random_codes(rng, (N, K), bits)
    s32 = rng.uniform(0.002, 0.02, size=(N, G)).astype(np.float32)
    half = np.float32(1 << (bits - 1))
    if bias == "jitter":
        jit = rng.uniform(-0.1, 0.1, size=(N, G)).astype(np.float32)
        b32 = (-half * s32) * (np.float32(1) + jit)
    elif bias == "exact":
        b32 = -half * s32
    else:
        raise ValueError(bias)
    b32 = b32.astype(np.float32)
    if x_dist == "normal":
        x32 = rng.standard_normal((M, K)).astype(np.float32)
    else:
        raise ValueError(x_dist)
    return {
        "M": M, "N": N, "K": K, "bits": bits, "gs": gs, "dtype": dt,
        "codes": codes,
        "w": pack_codes(codes, bits),
        "scales": to_storage(s32, dt),
        "biases": to_storage(b32, dt),
        "x": to_storage(x32, dt),
        "seed": seed,
    }


# ---------------------------------------------------------------- int8 weights x int8 activations
def pack_i8(q) -> np.ndarray:
    """int8 values ``[..., 4n]`` -> uint32 words ``[..., n]`` (element i at byte i % 4)."""
    return bytes_to_words(np.ascontiguousarray(np.asarray(q, dtype=np.int8)).view(np.uint8))


def q8_i8_case(N, K, seed):
    """Integer-activation matvec: int8 weights and activations uniform over all
    256 values, float32 block scales U(0.001, 0.01)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.Generator(np.random.PCG64(seed))
    q = random_bytes(rng, (N, K)).view(np.int8)
    x = random_bytes(rng, (K,)).view(np.int8)
    wd = rng.uniform(0.001, 0.01, size=(N, K // 32)).astype(np.float32)
    return {"N": N, "K": K, "q": q, "xq_values": x, "wq": pack_i8(q), "xq": pack_i8(x), "wd": wd, "seed": seed}


def q8_i8_case_torch(N, K, seed, device):
    """The same distributions drawn on a torch device (seeded Philox)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    wq = torch.randint(-(2 ** 31), 2 ** 31, (N, K // 4), dtype=torch.int64, generator=g, device=device).to(torch.int32)
    xq = torch.randint(-(2 ** 31), 2 ** 31, (K // 4,), dtype=torch.int64, generator=g, device=device).to(torch.int32)
    wd = torch.rand((N, K // 32), generator=g, device=device, dtype=torch.float32) * 0.009 + 0.001
    return {"N": N, "K": K, "wq": wq, "xq": xq, "wd": wd, "seed": seed}


# ---------------------------------------------------------------- Q8_0
def q8_0_case(N, K, seed):
    """Q8_0 matvec: quants U{-127..127}, f16 block scale U(0.001, 0.01), x ~ N(0,1) f32."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = K // 32
    q = random_bytes(rng, (N, K)).view(np.int8)
    bad = q == -128                      # redraw -128 so quants are uniform on -127..127
    while bad.any():
        q[bad] = random_bytes(rng, (int(bad.sum()),)).view(np.int8)
        bad = q == -128
    d = rng.uniform(0.001, 0.01, size=(N, nb)).astype(np.float32).astype(np.float16)
    x = rng.standard_normal(K).astype(np.float32)
    return {"N": N, "K": K, "q": q, "d": d, "x": x,
            "blocks": q8_0_blocks(q, d), "seed": seed}


def q8_0_blocks(q, d) -> np.ndarray:
    """int8 quants ``[N, K]`` and f16 scales ``[N, K/32]`` -> uint32 ``[N, K/32*9]``."""
    q = np.asarray(q, dtype=np.int8)
    n, k = q.shape
    nb = k // 32
    words = np.zeros((n, nb, 9), dtype=np.uint32)
    words[:, :, 0] = np.asarray(d, dtype=np.float16).view(np.uint16).astype(np.uint32)
    words[:, :, 1:] = bytes_to_words(q.view(np.uint8).reshape(n, nb, 32))
    return words.reshape(n, nb * 9)


# ---------------------------------------------------------------- Q4_K
def q4_k_case(N, K, seed):
    """Q4_K matvec: random quant and packed scale bytes (so every 6-bit scale
    and min is uniform on 0..63 and every quant uniform on 0..15), f16
    d ~ U[0.002, 0.052), f16 dmin ~ U[0, 0.025), x ~ N(0,1) f32."""
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = K // 256
    qs = random_bytes(rng, (N, nb, 128))
    sc = random_bytes(rng, (N, nb, 12))
    d = rng.uniform(0.002, 0.052, size=(N, nb)).astype(np.float32).astype(np.float16)
    dmin = rng.uniform(0.0, 0.025, size=(N, nb)).astype(np.float32).astype(np.float16)
    x = rng.standard_normal(K).astype(np.float32)
    return {"N": N, "K": K, "qs": qs, "scale_bytes": sc, "d": d, "dmin": dmin,
            "x": x, "blocks": q4_k_blocks(d, dmin, sc, qs), "seed": seed}


def q4_k_blocks(d, dmin, scale_bytes, qs) -> np.ndarray:
    """Assemble 144-byte super-blocks; returns uint32 ``[N, nb*36]``."""
    d = np.asarray(d, dtype=np.float16)
    n, nb = d.shape
    raw = np.zeros((n, nb, 144), dtype=np.uint8)
    raw[:, :, 0:2] = d.view(np.uint8).reshape(n, nb, 2)
    raw[:, :, 2:4] = np.asarray(dmin, dtype=np.float16).view(np.uint8).reshape(n, nb, 2)
    raw[:, :, 4:16] = scale_bytes
    raw[:, :, 16:144] = qs
    return bytes_to_words(raw).reshape(n, nb * 36)


# ---------------------------------------------------------------- device-side draws (bench)
def affine_case_torch(M, N, K, bits, gs, dtype, seed, device, bias="jitter"):
    """The affine workload drawn directly on a torch device (seeded Philox).

    Same distributions as ``affine_case``: packed words are random 32-bit
    words, so every b-bit code is uniform; scales U(0.002, 0.02) and the bias
    rule in f32, rounded to ``dtype``; x ~ N(0, 1).  Returns device tensors
    ``w`` (int32 bits), ``scales``, ``biases``, ``x``.
    """
    import torch
    dt = dtype_code(dtype)
    tdt = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dt]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    G = K // gs
    w = torch.randint(-(2 ** 31), 2 ** 31, (N, K * bits // 32), dtype=torch.int64, generator=g,
                      device=device).to(torch.int32)
    s32 = torch.rand((N, G), generator=g, device=device, dtype=torch.float32) * 0.018 + 0.002
    half = float(1 << (bits - 1))
    if bias == "jitter":
        jit = torch.rand((N, G), generator=g, device=device, dtype=torch.float32) * 0.2 - 0.1
        b32 = (-half * s32) * (1.0 + jit)
    else:
        b32 = -half * s32
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    return {"M": M, "N": N, "K": K, "bits": bits, "gs": gs, "dtype": dt, "seed": seed,
            "w": w, "scales": s32.to(tdt), "biases": b32.to(tdt), "x": x.to(tdt)}


def q8_0_case_torch(N, K, seed, device):
    """Q8_0 blocks drawn on a device: quants U{-127..127}, f16 d U(0.001, 0.01), x ~ N(0,1)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nb = K // 32
    q = torch.randint(-127, 128, (N, nb, 32), dtype=torch.int32, generator=g, device=device)
    b = (q & 0xFF).reshape(N, nb, 8, 4)
    words = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    d = (torch.rand((N, nb), generator=g, device=device) * 0.009 + 0.001).to(torch.float16)
    d_word = d.view(torch.int16).to(torch.int32) & 0xFFFF
    blocks = torch.cat([d_word.unsqueeze(-1), words], dim=-1).reshape(N, nb * 9).contiguous()
    x = torch.randn(K, generator=g, device=device, dtype=torch.float32)
    return {"N": N, "K": K, "blocks": blocks, "x": x, "seed": seed}


def q4_k_case_torch(N, K, seed, device):
    """Q4_K super-blocks drawn on a device: random scale/quant bytes, f16 d U[0.002, 0.052),
    f16 dmin U[0, 0.025), x ~ N(0,1)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nb = K // 256
    body = torch.randint(-(2 ** 31), 2 ** 31, (N, nb, 35), dtype=torch.int64, generator=g,
                         device=device).to(torch.int32)
    d = (torch.rand((N, nb), generator=g, device=device) * 0.05 + 0.002).to(torch.float16)
    dmin = (torch.rand((N, nb), generator=g, device=device) * 0.025).to(torch.float16)
    w0 = (d.view(torch.int16).to(torch.int32) & 0xFFFF) | (dmin.view(torch.int16).to(torch.int32) << 16)
    blocks = torch.cat([w0.unsqueeze(-1), body], dim=-1).reshape(N, nb * 36).contiguous()
    x = torch.randn(K, generator=g, device=device, dtype=torch.float32)
    return {"N": N, "K": K, "blocks": blocks, "x": x, "seed": seed}
