"""Element-wise parity bounds for attention outputs against the fp64 oracle.

Test infrastructure (imported by the tests only).

Two gates apply to every 16-bit output compared with the oracle:

* the absolute tolerance of the workload descriptions: max-abs 2e-2 for f16 /
  bf16 KV and 1e-5 for float32 KV;
* a bound scaled to the output, from the kernel's error budget, that a dropped,
  repeated or misrouted 16-token block (or a 512-token partition at 32K
  tokens) does not meet:

      |got - want| <= K * u * (|want| + rms(want row)) + floor

  u is the unit roundoff of the KV element type (2^-8 bf16, 2^-11 f16; 2^-20
  for float32, which covers the float32 logits, exp2 and accumulation).  The
  two terms of the budget: the output is rounded once to the element type
  (<= u |want|), and every softmax weight is rounded to the element type
  before the P.V product while the running sum adds the same rounded weights,
  so the result is a convex combination of V rows whose weights carry
  independent relative errors <= u: the output moves by sum_t w_t d_t
  (v_t - out), of standard deviation <= u / sqrt(3) * rms(v - out) *
  sqrt(sum_t w_t^2).  The rms of the output row scales like sqrt(sum_t w_t^2)
  for N(0, 1) values, so K = 4 leaves about 5 standard deviations of that
  term plus the store (checked against an emulation of the kernel's rounding
  in tests/test_parity_bounds.py, which also shows that a dropped block or
  partition breaks the bound).
"""
from __future__ import annotations

import json
import os

import numpy as np

ABS_TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
UNIT = {"f32": 2.0 ** -20, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
K_SCALED = 4.0
FLOOR = {"f32": 1e-7, "f16": 1e-6, "bf16": 1e-6}


def logit_gates(dtype: str, xmax: float, vmax: float) -> dict:
    """Gates for logits of magnitude up to xmax (natural units): float32 logits
    carry an absolute error of about 2^-21 xmax (the rounding of the q.k
    dot product and of the scale), which moves every weight by that much
    relatively, and the output by that times at most 2 vmax.  With N(0, 1)
    logits this is below the float32 tolerance; logits of 100 or a common
    offset of 1000 make it the larger term."""
    e = 2.0 ** -21 * xmax
    return {"abs_tol": ABS_TOL[dtype] + 2.0 * vmax * e, "unit": UNIT[dtype] + e}


def quantised_gates(dtype: str, qmag: float, vmax: float) -> dict:
    """Gates for quantised keys: the B operand of their logit products is
    q' = q * s rounded to f16 (relative error <= 2^-11 per element, whatever
    the value type), so a logit is off by at most
    e = 2^-11 * scale * sum_c |q_c s_c code_c| (qmag = the largest such sum
    over the call, natural units); each weight then moves by about e
    relatively, the output by at most 2 vmax e."""
    e = 2.0 ** -11 * qmag
    return {"abs_tol": ABS_TOL[dtype] + 2.0 * vmax * e, "unit": UNIT[dtype] + e}


def scaled_bound(want: np.ndarray, dtype: str, unit: float | None = None) -> np.ndarray:
    """Per-element bound of the same shape as ``want`` (rows = last axis)."""
    want = np.asarray(want, dtype=np.float64)
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    u = UNIT[dtype] if unit is None else unit
    return K_SCALED * u * (np.abs(want) + rms) + FLOOR[dtype]


def violations(got: np.ndarray, want: np.ndarray, dtype: str, abs_tol: float | None = None,
               unit: float | None = None):
    """(number of elements outside either gate, max-abs error, max ratio of
    the error to the scaled bound)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bound = scaled_bound(want, dtype, unit)
    tol = ABS_TOL[dtype] if abs_tol is None else abs_tol
    bad = ~np.isfinite(got) | (err > tol) | (err > bound)
    ratio = float(np.max(err / bound, initial=0.0))
    return int(bad.sum()), float(err.max(initial=0.0)), ratio


def assert_parity(got, want, dtype: str, what: str, abs_tol: float | None = None,
                  unit: float | None = None) -> dict:
    """Both gates on every element; prints and returns the achieved figures."""
    n_bad, max_abs, ratio = violations(got, want, dtype, abs_tol, unit)
    print(f"[parity] {what}: max-abs {max_abs:.3e}, max err/scaled-bound {ratio:.3f}, "
          f"{np.asarray(want).size} elements", flush=True)
    log = os.environ.get("PA_PARITY_LOG")  # optional record of the achieved errors
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"what": what, "dtype": dtype, "elements": int(np.asarray(want).size),
                                "max_abs": max_abs, "err_over_bound": ratio,
                                "pass": n_bad == 0}) + "\n")
    if n_bad:
        got = np.asarray(got, dtype=np.float64)
        err = np.abs(got - np.asarray(want, dtype=np.float64))
        worst = np.unravel_index(np.nanargmax(np.where(np.isfinite(err), err, np.inf)), err.shape)
        raise AssertionError(f"{what}: {n_bad} elements outside the bounds (max-abs {max_abs:.3e}, "
                             f"err/bound {ratio:.3f}, worst at {worst})")
    return {"max_abs": max_abs, "ratio": ratio}
