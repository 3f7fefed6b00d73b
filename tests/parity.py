"""Comparison of device outputs with the float64 oracle.

Tolerance (the contract: rel-L2 <= 1e-3 and max-abs <= 2 bf16 ulps of the
reference for f16/bf16 outputs, <= 1e-5 relative for f32), read as:

* 16-bit outputs: ``rel_l2 = ||out - round(ref)|| / ||round(ref)||`` with
  ``round`` the oracle's round-to-nearest-even to the output dtype (a
  perfectly rounded bf16 output is already ~1.6e-3 from the unrounded
  reference, so the literal unrounded reading would reject exact results),
  gate 1e-3; and ``max|out - ref| <= 2 * ulp_bf16(max|ref|)``, a norm-wise
  bound.
* float32 outputs: ``rel_l2 = ||out - ref|| / ||ref|| <= 1e-5`` and
  ``max|out - ref| <= 1e-5 * max|ref|``.
"""
from __future__ import annotations

import math

import numpy as np

F32, F16, BF16 = 0, 1, 2


def ulp_bf16(v: float) -> float:
    if v == 0:
        return 2.0 ** -133
    return 2.0 ** (math.floor(math.log2(abs(v))) - 7)


def compare(out64, ref64, dt, orc):
    """Metrics of ``out64`` (decoded device output) against ``ref64``."""
    out64 = np.asarray(out64, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    assert out64.shape == ref64.shape, (out64.shape, ref64.shape)
    if out64.size == 0:
        return {"rel_l2": 0.0, "max_abs": 0.0, "bound": 0.0, "ok": True, "n": 0}
    refT = orc.round(ref64, dt) if dt != F32 else ref64
    base = refT if dt != F32 else ref64
    den = float(np.linalg.norm(base))
    rel = float(np.linalg.norm(out64 - base)) / den if den > 0 else float(np.linalg.norm(out64))
    max_abs = float(np.max(np.abs(out64 - ref64)))
    amax = float(np.max(np.abs(ref64)))
    if dt == F32:
        bound, rel_gate = 1e-5 * amax, 1e-5
    else:
        bound, rel_gate = 2 * ulp_bf16(amax), 1e-3
    exact = float(np.mean(out64 == refT)) if dt != F32 else float("nan")
    ok = bool(np.all(np.isfinite(out64))) and rel <= rel_gate and max_abs <= bound
    return {"rel_l2": rel, "max_abs": max_abs, "bound": bound, "rel_gate": rel_gate,
            "frac_exact": exact, "ok": ok, "n": int(out64.size)}


def assert_close(out64, ref64, dt, orc, what=""):
    m = compare(out64, ref64, dt, orc)
    assert m["ok"], f"{what}: {m}"
    return m
