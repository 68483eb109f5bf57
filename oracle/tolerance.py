"""Element-wise comparison rules between a device result and the oracle -- TEST INFRASTRUCTURE.

Used only by the tests, the smoke check and the benchmark's sampled parity check.

Rules (per element, ``ref`` is the unrounded float64 oracle value):

* fp16 outputs: ``|y - ref| <= max(2e-3, ulp16(ref))``.  2e-3 is the stated bound; it cannot
  hold where the fp16 grid itself is coarser (|ref| >= 8, where half a spacing already exceeds
  2e-3), so there one spacing of the fp16 grid at |ref| is allowed.
* bf16 outputs: ``|y - ref| / max(|ref|, 1e-2) <= 1e-2`` (relative, with a floor so that
  outputs that are near zero through cancellation are judged in absolute terms).
* fp32 outputs: ``|y - ref| <= 1e-5``.

NaN in the result where the reference is finite, or vice versa, always fails.
"""
from __future__ import annotations

import math

import numpy as np

FP16_ABS = 2e-3
BF16_REL = 1e-2
BF16_FLOOR = 1e-2
FP32_ABS = 1e-5

# The rules above as text, for reports.
RULE_TEXT = {
    "f16": "|y - ref| <= max(2e-3, ulp16(ref))",
    "bf16": "|y - ref| / max(|ref|, 1e-2) <= 1e-2",
    "f32": "|y - ref| <= 1e-5",
}


def ulp16(v) -> np.ndarray:
    """Spacing of the binary16 grid in the binade of |v| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -30)))
    e = np.maximum(e, -14.0)
    return np.ldexp(1.0, (e - 10).astype(np.int64))


def _as64(y) -> np.ndarray:
    if hasattr(y, "detach"):
        import torch
        y = y.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(y, dtype=np.float64)


def compare(y, ref, kind: str) -> dict:
    """Compare a result with the oracle under the rule for ``kind`` ('f16', 'bf16', 'f32').

    Returns a dict with ok, n_bad, max_abs, max_excess (worst err / allowed), worst index.
    """
    y = _as64(y)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    err = np.abs(y - ref)
    if kind in ("f16", "fp16"):
        allowed = np.maximum(FP16_ABS, ulp16(ref))
    elif kind == "bf16":
        allowed = BF16_REL * np.maximum(np.abs(ref), BF16_FLOOR)
    elif kind in ("f32", "fp32"):
        allowed = np.full_like(ref, FP32_ABS)
    else:
        raise ValueError(kind)
    nan_mismatch = np.isnan(y) != np.isnan(ref)
    both_nan = np.isnan(y) & np.isnan(ref)
    err = np.where(both_nan, 0.0, err)
    bad = (err > allowed) | nan_mismatch
    ratio = np.where(allowed > 0, err / allowed, np.inf)
    ratio = np.where(nan_mismatch, np.inf, ratio)
    worst = int(np.argmax(ratio)) if ratio.size else -1
    return {
        "ok": bool(not bad.any()),
        "n_bad": int(bad.sum()),
        "n": int(y.size),
        "max_abs": float(np.max(np.where(np.isnan(err), 0.0, err))) if err.size else 0.0,
        "max_excess": float(ratio.flat[worst]) if ratio.size else 0.0,
        "worst": np.unravel_index(worst, y.shape) if ratio.size else None,
        "rule": kind,
    }


def assert_close(y, ref, kind: str, what: str = "") -> dict:
    r = compare(y, ref, kind)
    if not r["ok"]:
        w = r["worst"]
        yv = _as64(y)[w] if w is not None else math.nan
        rv = np.asarray(ref)[w] if w is not None else math.nan
        raise AssertionError(
            f"{what}: {r['n_bad']}/{r['n']} elements outside the {kind} rule; max_abs={r['max_abs']:.3e} "
            f"worst at {w}: got {yv!r} want {rv!r} ({r['max_excess']:.2f}x allowed)")
    return r
