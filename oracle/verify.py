"""Compare a GPU result with the oracle's fp64 sums (test infrastructure).

Two checks, both element by element:

* exact(out32, ref64): out32 must equal ref64 rounded to fp32 (round to nearest
  even), compared by value (so -0 == +0); any NaN fails. This is the bar for
  integer-valued inputs: with |a|, |b| <= 4 integers every product and partial sum
  is an integer below 2**24 (for K < 10**6), so every fp32 operation is exact in
  any order and any correct kernel reproduces the oracle bit for bit.
* within_tol(out32, ref64, mag64, rel=1e-5): |out32 - ref64| <= rel * mag64 per
  element, evaluated in fp64, where mag64 = sum |a*b| over the same products; NaN
  or Inf anywhere fails. Where mag64 == 0 every product is zero and the result
  must be exactly 0.

Both return a Report; Report.ok is the verdict and str(Report) names the first
failing element.
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class Report:
    ok: bool
    n: int
    bad: int
    worst: float          # largest |err| / allowed (exact mode: largest |err|)
    first_bad: tuple      # index of the first failing element, or ()
    detail: str = ""

    def __bool__(self):
        return self.ok

    def __str__(self):
        if self.ok:
            return f"ok: {self.n} elements, worst ratio {self.worst:.3g}"
        return (f"FAIL: {self.bad}/{self.n} elements; first at {self.first_bad}; "
                f"worst {self.worst:.3g}; {self.detail}")


def _first(mask):
    idx = np.argwhere(mask)
    return tuple(int(v) for v in idx[0]) if idx.size else ()


def exact(out32, ref64) -> Report:
    out32 = np.asarray(out32)
    ref64 = np.asarray(ref64)
    if out32.shape != ref64.shape:
        raise ValueError(f"shape mismatch {out32.shape} vs {ref64.shape}")
    want = ref64.astype(np.float32)
    bad = ~(out32 == want)           # NaN compares unequal, so NaN is caught here
    nbad = int(bad.sum())
    diff = np.abs(out32.astype(np.float64) - want.astype(np.float64))
    worst = float(np.nanmax(diff)) if diff.size else 0.0
    if np.isnan(diff).any():
        worst = float("nan")
    detail = ""
    if nbad:
        f = _first(bad)
        detail = f"got {out32[f]!r}, want {want[f]!r}"
    return Report(nbad == 0, int(out32.size), nbad, worst, _first(bad), detail)


def within_tol(out32, ref64, mag64, rel: float = 1e-5) -> Report:
    out32 = np.asarray(out32)
    ref64 = np.asarray(ref64)
    mag64 = np.asarray(mag64)
    if not (out32.shape == ref64.shape == mag64.shape):
        raise ValueError(f"shape mismatch {out32.shape}, {ref64.shape}, {mag64.shape}")
    got = out32.astype(np.float64)
    err = np.abs(got - ref64)
    allowed = rel * mag64
    finite = np.isfinite(got)
    bad = ~finite | (err > allowed)
    nbad = int(bad.sum())
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allowed > 0, err / allowed, np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio[finite])) if finite.any() else float("inf")
    detail = ""
    if nbad:
        f = _first(bad)
        detail = f"got {got[f]!r}, want {ref64[f]!r} +- {allowed[f]!r}"
    return Report(nbad == 0, int(out32.size), nbad, worst, _first(bad), detail)
