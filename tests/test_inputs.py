"""The seeded generators: layouts against the pages' statements, value ranges, determinism."""
import json
import os

import numpy as np

import qmx_inputs as qi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pack_matches_stated_layouts():
    cases = json.load(open(os.path.join(GOLDEN, "layouts.json")))["cases"]
    for c in cases:
        codes = np.array(c["codes"], dtype=np.uint8)[None, :]
        words = qi.pack_codes(codes, c["bits"])
        assert [int(w) for w in words[0]] == [int(w, 16) for w in c["words"]], c


def test_affine_distributions_and_determinism():
    a = qi.affine_case(2, 64, 4096, 4, 64, "f32", seed=qi.seed_for(1, 0))
    b = qi.affine_case(2, 64, 4096, 4, 64, "f32", seed=qi.seed_for(1, 0))
    for k in ("w", "scales", "biases", "x"):
        assert np.array_equal(a[k], b[k])
    s, bb = a["scales"], a["biases"]
    assert s.min() > 0.002 and s.max() < 0.02
    ratio = -bb / (8 * s)
    assert ratio.min() >= 0.9 - 1e-6 and ratio.max() <= 1.1 + 1e-6
    assert a["codes"].max() == 15 and a["codes"].min() == 0
    assert abs(a["x"].mean()) < 0.05 and abs(a["x"].std() - 1) < 0.05


def test_exact_bias_is_power_of_two_multiple():
    for bits in (2, 4, 8):
        c = qi.affine_case(1, 16, 256, bits, 32, "bf16", seed=5, bias="exact")
        s = qi.storage_to_f64(c["scales"], qi.BF16)
        b = qi.storage_to_f64(c["biases"], qi.BF16)
        assert np.array_equal(b, -(2.0 ** (bits - 1)) * s)
        assert c["codes"].max() == (1 << bits) - 1


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1); 1 + 3*2^-8 -> 1 + 2^-6
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert list(qi.f32_to_bf16_bits(v)) == [0x3F80, 0x3F82, 0xBF80]


def test_q8_0_blocks():
    c = qi.q8_0_case(3, 96, seed=1)
    blk = c["blocks"].reshape(3, 3, 9)
    assert np.all(blk[:, :, 0] >> 16 == 0)
    assert np.array_equal((blk[:, :, 0] & 0xFFFF).astype(np.uint16).view(np.float16), c["d"])
    q = blk[:, :, 1:].copy().view(np.uint8).reshape(3, 96).view(np.int8)
    assert np.array_equal(q, c["q"])
    assert c["q"].min() >= -127 and c["q"].max() <= 127


def test_q4_k_blocks():
    c = qi.q4_k_case(2, 512, seed=2)
    raw = c["blocks"].reshape(2, 2, 36).copy().view(np.uint8).reshape(2, 2, 144)
    assert np.array_equal(raw[:, :, 0:2].copy().view(np.float16)[..., 0], c["d"])
    assert np.array_equal(raw[:, :, 2:4].copy().view(np.float16)[..., 0], c["dmin"])
    assert np.array_equal(raw[:, :, 4:16], c["scale_bytes"])
    assert np.array_equal(raw[:, :, 16:], c["qs"])
    d = c["d"].astype(np.float64)
    assert d.min() >= 0.0019 and d.max() <= 0.0521
