"""Tolerances and comparison helpers shared by the parity tests.

Bars (attention output compared in fp64 against the fp64 oracle):

* fp32 inputs:       max-abs <= 1e-5, relative L2 <= 1e-6.
* fp16 inputs:       max-abs <= 2e-2, mean-abs <= 2e-3, relative L2 <= 1e-3.
* bf16 inputs:       max-abs <= 2e-2, mean-abs <= 2e-3, relative L2 <= 5e-3.

The max-abs / mean-abs bars are the project's stated targets. Under these input
distributions the outputs are small (|out| of order 1e-2), so those two bars alone would
accept an all-zero output; the relative-L2 bar is derived from the output rounding: an
output stored in a 16-bit type carries at most half an ulp of relative error (2^-9 for
bf16, 2^-11 for fp16), whose RMS is about 0.58 of that, and fp32 accumulation adds far
less. 5e-3 and 1e-3 leave a factor of about 4-8 over that rounding; 1e-6 for fp32 leaves a
factor of about 10 over the accumulation error of sums of a few hundred fp32 terms.
"""

from __future__ import annotations

import numpy as np

BARS = {
    "f32": {"max_abs": 1e-5, "mean_abs": None, "rel_l2": 1e-6},
    "f16": {"max_abs": 2e-2, "mean_abs": 2e-3, "rel_l2": 1e-3},
    "bf16": {"max_abs": 2e-2, "mean_abs": 2e-3, "rel_l2": 5e-3},
}


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    if not np.all(np.isfinite(got)):
        return {"max_abs": np.inf, "mean_abs": np.inf, "rel_l2": np.inf, "finite": False}
    return {
        "max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "mean_abs": float(np.mean(np.abs(diff))) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)),
        "finite": True,
    }


def within(got, ref, dtype: str) -> tuple[bool, dict]:
    e = errors(got, ref)
    bar = BARS[dtype]
    ok = e["finite"] and e["max_abs"] <= bar["max_abs"] and e["rel_l2"] <= bar["rel_l2"]
    if bar["mean_abs"] is not None:
        ok = ok and e["mean_abs"] <= bar["mean_abs"]
    return ok, e


def assert_close(got, ref, dtype: str, what: str = "") -> dict:
    ok, e = within(got, ref, dtype)
    assert ok, f"{what}: parity failed for {dtype}: {e} vs bars {BARS[dtype]}"
    return e
