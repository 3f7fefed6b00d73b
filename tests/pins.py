"""Pins of the float64 oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages and the mathematics fix:
layouts the pages state, IEEE-754 decodes, hand-worked blocks, exact rational
brute force, a dense numpy dequantise-then-matmul, closed forms and special
cases.  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` plants mistakes in copies of the oracle source and
checks that some pin fails for each.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import qmx_inputs as qi
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32, F16, BF16 = qi.F32, qi.F16, qi.BF16


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _h(s):
    return int(s, 16)


def _ev(expr):
    """Evaluate a tiny fixture expression such as '1 + 3*2**-8' or 'inf'."""
    if expr in ("inf", "-inf"):
        return float(expr)
    return float(eval(expr, {"__builtins__": {}}, {}))  # fixture text is ours, arithmetic only


def dense_weights(case):
    """numpy dequantisation from the generator's raw codes: W[n,k] = s*q + b (f64)."""
    s = qi.storage_to_f64(case["scales"], case["dtype"])
    b = qi.storage_to_f64(case["biases"], case["dtype"])
    gs = case["gs"]
    q = case["codes"].astype(np.float64)
    return s.repeat(gs, axis=1) * q + b.repeat(gs, axis=1)


def _onehot_codes(o, words, bits, K):
    """Codes the oracle reads from one row, probed with scale 1, bias 0, x = e_k."""
    w = np.array([_h(x) if isinstance(x, str) else x for x in words], dtype=np.uint32)[None, :]
    G = 1
    gs = K
    s = np.ones((1, G), np.float32)
    b = np.zeros((1, G), np.float32)
    x = np.eye(K, dtype=np.float32)
    out = o.affine(w, s, b, F32, x, F32, K, 1, K, bits, gs)
    return out[:, 0]


# ---------------------------------------------------------------- layouts and decodes
def pin_layouts(o):
    for c in _golden("layouts.json")["cases"]:
        K = len(c["codes"])
        got = _onehot_codes(o, c["words"], c["bits"], K)
        assert np.array_equal(got, np.array(c["codes"], dtype=np.float64)), (c, got)


def pin_half_decode(o):
    g = _golden("halfprec.json")
    for name, dt in (("f16", F16), ("bf16", BF16)):
        bits = np.array([_h(b) for b, _ in g[name]], dtype=np.uint16)
        want = np.array([_ev(v) for _, v in g[name]])
        got = o.decode(bits, dt)
        assert np.array_equal(got, want), (name, got, want)


def pin_rounding(o):
    g = _golden("halfprec.json")
    for name, dt in (("round_bf16", BF16), ("round_f16", F16)):
        v = np.array([_ev(a) for a, _ in g[name]])
        want = np.array([_ev(b) for _, b in g[name]])
        got = o.round(v, dt)
        assert np.array_equal(got, want), (name, got, want)
    # library routines: numpy's float64 -> float16 and -> float32 casts round to nearest even
    rng = np.random.Generator(np.random.PCG64(7))
    v = rng.standard_normal(4096) * np.exp2(rng.integers(-30, 15, 4096))
    assert np.array_equal(o.round(v, F16), v.astype(np.float16).astype(np.float64))
    assert np.array_equal(o.round(v, F32), v.astype(np.float32).astype(np.float64))
    # bf16 of float32-representable values: the generator's bit rounding is RNE from f32
    v32 = v.astype(np.float32)
    want = qi.bf16_bits_to_f32(qi.f32_to_bf16_bits(v32)).astype(np.float64)
    assert np.array_equal(o.round(v32.astype(np.float64), BF16), want)


def pin_q8_0_golden(o):
    g = _golden("q8_0_block.json")
    blk = np.array([_h(w) for w in g["words"]], dtype=np.uint32)[None, :]
    x = np.array(g["x"], dtype=np.float32)
    got = o.q8_0(blk, x, 1, 32)
    assert got[0] == g["out"], got


def _q4k_golden_block():
    g = _golden("q4_k_block.json")
    raw = np.zeros(144, dtype=np.uint8)
    raw[0:2] = np.array([_h(g["d_bits"])], np.uint16).view(np.uint8)
    raw[2:4] = np.array([_h(g["dmin_bits"])], np.uint16).view(np.uint8)
    raw[4:16] = [_h(b) for b in g["scale_bytes"]]
    for idx, val in g["qs_nonzero"].items():
        raw[16 + int(idx)] = _h(val)
    return g, qi.bytes_to_words(raw)[None, :]


def pin_q4_k_golden(o):
    g, blk = _q4k_golden_block()
    x = np.zeros(256, dtype=np.float32)
    for p in g["probes"]:
        x[:] = 0
        x[p["element"]] = 1
        got = o.q4_k(blk, x, 1, 256)[0]
        assert got == p["weight"], (p, got)
    # the independent field-map decoder agrees with the hand-derived sub-block table
    raw_scales = [_h(b) for b in g["scale_bytes"]]
    assert [list(t) for t in brute.q4_k_sub_scales(raw_scales)] == g["sub_scales"]


# ---------------------------------------------------------------- brute force
def _rel_err(got, exact_fracs):
    num = max(abs(Fraction(float(gv)) - e) for gv, e in zip(got, exact_fracs))
    den = max(max(abs(e) for e in exact_fracs), Fraction(1, 10**30))
    return float(num / den)


def pin_affine_brute(o):
    shapes = [(1, 1, 32, 32), (2, 3, 64, 32), (3, 2, 256, 64), (1, 8, 512, 128), (2, 2, 128, 128)]
    case_id = 0
    for bits in (1, 2, 3, 4, 5, 6, 8):
        for dt in (F32, F16, BF16):
            for (M, N, K, gs) in (shapes if bits in (2, 4, 8) else shapes[:3]):
                if (K * bits) % 32:
                    continue
                case_id += 1
                c = qi.affine_case(M, N, K, bits, gs, dt, seed=900 + case_id)
                got = o.affine_case(c)
                ex = brute.affine_exact(c["w"], c["scales"], c["biases"], c["x"], dt, M, N, K, bits, gs)
                flat_e = [v for row in ex for v in row]
                assert _rel_err(got.ravel(), flat_e) < 1e-14, (bits, dt, M, N, K, gs)


def pin_q8_0_brute(o):
    for i, (N, K) in enumerate([(1, 32), (3, 64), (2, 128)]):
        c = qi.q8_0_case(N, K, seed=950 + i)
        got = o.q8_0(c["blocks"], c["x"], N, K)
        ex = brute.q8_0_exact(c["blocks"], c["x"], N, K)
        assert _rel_err(got, ex) < 1e-14


def pin_q4_k_brute(o):
    for i, (N, K) in enumerate([(1, 256), (2, 512)]):
        c = qi.q4_k_case(N, K, seed=960 + i)
        got = o.q4_k(c["blocks"], c["x"], N, K)
        ex = brute.q4_k_exact(c["blocks"], c["x"], N, K)
        assert _rel_err(got, ex) < 1e-14


def pin_q8_i8_brute(o):
    for i, (N, K) in enumerate([(1, 32), (3, 64), (2, 128)]):
        c = qi.q8_i8_case(N, K, seed=965 + i)
        got = o.q8_i8(c["wq"], c["xq"], c["wd"], N, K)
        ex = brute.q8_i8_exact(c["wq"], c["xq"], c["wd"], N, K)
        assert _rel_err(got, ex) < 1e-14


def pin_q8_i8_layout(o):
    """One-hot activations read single weights back through the packed layout."""
    g = _golden("int8_layout.json")
    for case in g["cases"]:
        words = np.array([int(w, 16) for w in case["words"]], dtype=np.uint32)
        K = 4 * len(words)
        Kp = 32 * ((K + 31) // 32)
        wq = np.zeros((1, Kp // 4), dtype=np.uint32)
        wq[0, :len(words)] = words
        wd = np.ones((1, Kp // 32), dtype=np.float32)
        for i, v in enumerate(case["values"]):
            onehot = np.zeros(Kp, dtype=np.int8)
            onehot[i] = 1
            got = o.q8_i8(wq, qi.pack_i8(onehot), wd, 1, Kp)[0]
            assert got == v, (case, i, got)


def pin_q8_i8_integer_gemv(o):
    """Unit block scales: the exact integer matrix-vector product (numpy int64)."""
    c = qi.q8_i8_case(7, 256, seed=968)
    ones = np.ones_like(c["wd"])
    got = o.q8_i8(c["wq"], c["xq"], ones, 7, 256)
    want = c["q"].astype(np.int64) @ c["xq_values"].astype(np.int64)
    assert np.array_equal(got, want.astype(np.float64))


# ---------------------------------------------------------------- identities and library routines
def pin_dense_numpy(o):
    """Dequantise from the raw codes with numpy, then x @ W.T in float64."""
    for i, (M, N, K, bits, gs, dt) in enumerate([(3, 16, 1024, 4, 64, BF16), (2, 9, 512, 2, 32, F16),
                                                (4, 7, 384, 8, 128, F32), (1, 33, 4096, 4, 64, F32),
                                                (2, 5, 384, 3, 64, BF16), (3, 6, 256, 5, 32, F16),
                                                (1, 7, 192, 6, 64, F32), (2, 4, 256, 1, 128, BF16)]):
        c = qi.affine_case(M, N, K, bits, gs, dt, seed=970 + i)
        W = dense_weights(c)
        X = qi.storage_to_f64(c["x"], dt)
        want = X @ W.T
        got = o.affine_case(c)
        scale = np.abs(X) @ np.abs(W).T
        assert np.all(np.abs(got - want) <= 1e-12 * scale + 1e-300), (M, N, K, bits, gs, dt)


def pin_hoist_identity(o):
    """The bias-hoisted form equals the dequantise-then-dot form."""
    for i, (M, N, K, bits, gs, dt) in enumerate([(3, 16, 2048, 4, 64, BF16), (2, 8, 1024, 2, 32, F16),
                                                (2, 8, 1024, 8, 128, F32)]):
        c = qi.affine_case(M, N, K, bits, gs, dt, seed=980 + i)
        d = o.affine_case(c)
        h = o.affine_hoisted(c["w"], c["scales"], c["biases"], dt, c["x"], dt, M, N, K, bits, gs)
        scale = np.abs(qi.storage_to_f64(c["x"], dt)) @ np.abs(dense_weights(c)).T
        assert np.all(np.abs(d - h) <= 1e-12 * scale)


def pin_special_cases(o):
    M, N, K, bits, gs = 3, 5, 256, 4, 64
    c = qi.affine_case(M, N, K, bits, gs, F32, seed=990)
    X = qi.storage_to_f64(c["x"], F32)
    b = qi.storage_to_f64(c["biases"], F32)
    G = K // gs
    # all codes zero -> out = sum_g b[n,g] * sum_{i in g} x[m,i]
    zero_w = np.zeros_like(c["w"])
    got = o.affine(zero_w, c["scales"], c["biases"], F32, c["x"], F32, M, N, K, bits, gs)
    xs = X.reshape(M, G, gs).sum(axis=2)
    assert np.allclose(got, xs @ b.T, rtol=1e-13, atol=1e-13)
    # scale 1, bias 0, integer x -> exact integer GEMV of the codes
    xi = np.random.Generator(np.random.PCG64(991)).integers(-50, 51, size=(M, K))
    ones = np.ones_like(c["scales"])
    zeros = np.zeros_like(c["biases"])
    got = o.affine(c["w"], ones, zeros, F32, xi.astype(np.float32), F32, M, N, K, bits, gs)
    want = xi.astype(np.int64) @ c["codes"].astype(np.int64).T
    assert np.array_equal(got, want.astype(np.float64))
    # linearity in powers of two is exact
    for j in (-3, 5):
        x2 = (X * 2.0 ** j).astype(np.float32)
        got2 = o.affine(c["w"], c["scales"], c["biases"], F32, x2, F32, M, N, K, bits, gs)
        base = o.affine_case(c)
        assert np.array_equal(got2, base * 2.0 ** j)
    # one group spanning the whole row with 8-bit codes -> per-row affine int8 GEMV
    c8 = qi.affine_case(2, 4, 128, 8, 128, F32, seed=992)
    W = (qi.storage_to_f64(c8["scales"], F32) * c8["codes"].astype(np.float64)
         + qi.storage_to_f64(c8["biases"], F32))
    want = qi.storage_to_f64(c8["x"], F32) @ W.T
    assert np.allclose(o.affine_case(c8), want, rtol=1e-13, atol=1e-12)


def pin_split_additivity(o):
    """Per-partition oracles over whole groups add up to the full oracle."""
    M, N, K, bits, gs = 2, 6, 1024, 4, 64
    c = qi.affine_case(M, N, K, bits, gs, BF16, seed=995)
    full = o.affine_case(c)
    G = K // gs
    for S in (2, 3, 4):
        parts = [o.affine_groups(c["w"], c["scales"], c["biases"], BF16, c["x"], BF16, M, N, K,
                                 bits, gs, (p * G) // S, ((p + 1) * G) // S) for p in range(S)]
        assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-12)
    # a partition is the oracle of the matching slice of the problem
    g0, g1 = 3, 11
    part = o.affine_groups(c["w"], c["scales"], c["biases"], BF16, c["x"], BF16, M, N, K, bits, gs,
                           g0, g1)
    W = dense_weights(c)[:, g0 * gs:g1 * gs]
    X = qi.storage_to_f64(c["x"], BF16)[:, g0 * gs:g1 * gs]
    assert np.allclose(part, X @ W.T, rtol=1e-12, atol=1e-12)


def pin_columns_subset(o):
    c = qi.affine_case(2, 40, 512, 4, 64, F16, seed=996)
    full = o.affine_case(c)
    cols = np.array([39, 0, 17, 17, 5], dtype=np.int32)
    assert np.array_equal(o.affine_case(c, cols=cols), full[:, cols])


def pin_q8_0_dense(o):
    c = qi.q8_0_case(17, 640, seed=997)
    W = c["d"].astype(np.float64).repeat(32, axis=1) * c["q"].astype(np.float64)
    want = W @ c["x"].astype(np.float64)
    got = o.q8_0(c["blocks"], c["x"], 17, 640)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    # unit scale and integer x -> exact int8 dot
    d1 = np.ones_like(c["d"])
    xi = np.random.Generator(np.random.PCG64(998)).integers(-9, 10, size=640).astype(np.float32)
    got = o.q8_0(qi.q8_0_blocks(c["q"], d1), xi, 17, 640)
    assert np.array_equal(got, (c["q"].astype(np.int64) @ xi.astype(np.int64)).astype(np.float64))
    rows = np.array([16, 3, 3], dtype=np.int32)
    assert np.array_equal(o.q8_0(c["blocks"], c["x"], 17, 640, rows=rows), o.q8_0(c["blocks"], c["x"], 17, 640)[rows])


def pin_q4_k_dense(o):
    """Dense dequantisation built from the independent field-map decoder, then numpy matvec."""
    c = qi.q4_k_case(5, 768, seed=999)
    N, K = 5, 768
    W = np.zeros((N, K))
    for n in range(N):
        for blk in range(K // 256):
            W[n, 256 * blk:256 * (blk + 1)] = [float(v) for v in
                                               brute.q4_k_weights_exact(c["blocks"][n, 36 * blk:36 * (blk + 1)])]
    want = W @ c["x"].astype(np.float64)
    got = o.q4_k(c["blocks"], c["x"], N, K)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


ALL_PINS = [pin_layouts, pin_half_decode, pin_rounding, pin_q8_0_golden, pin_q4_k_golden,
            pin_q8_i8_brute, pin_q8_i8_layout, pin_q8_i8_integer_gemv,
            pin_affine_brute, pin_q8_0_brute, pin_q4_k_brute, pin_dense_numpy, pin_hoist_identity,
            pin_special_cases, pin_split_additivity, pin_columns_subset, pin_q8_0_dense,
            pin_q4_k_dense]


def failing_pins(o):
    """Names of the pins that fail (or crash) on oracle ``o``."""
    bad = []
    for p in ALL_PINS:
        try:
            p(o)
        except Exception:  # noqa: BLE001 - any failure counts
            bad.append(p.__name__)
    return bad


__all__ = ["ALL_PINS", "failing_pins", "dense_weights"] + [p.__name__ for p in ALL_PINS]
