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

import os

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


# Every comparison made through assert_close in this session: the test, what was compared,
# the achieved errors and the bars. conftest.py writes them as a table at the end of the
# session when PKV_PARITY_RECORD names a file.
RECORDS: list[dict] = []


def assert_close(got, ref, dtype: str, what: str = "") -> dict:
    ok, e = within(got, ref, dtype)
    RECORDS.append({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
                    "what": what, "dtype": dtype, "elements": int(np.asarray(got).size),
                    "ok": bool(ok), **{k: e[k] for k in ("max_abs", "mean_abs", "rel_l2")}})
    assert ok, f"{what}: parity failed for {dtype}: {e} vs bars {BARS[dtype]}"
    return e


# How each test module's kernels form the weighted sum of V (the pages fix no precision;
# the matrix-core forms round the softmax weights first).
PATHS = {
    "test_gpu_parity": "single-query: fp32 weights, P.V on the vector ALU",
    "test_gpu_step": "single-query: fp32 weights, P.V on the vector ALU",
    "test_zz_no_alloc": "single-query: fp32 weights, P.V on the vector ALU",
    "test_gpu_limits": "single-query: fp32 weights, P.V on the vector ALU",
    "test_gpu_multi_query": "multi-query: weights rounded to the dtype, P.V on the matrix cores",
    "test_gpu_mq_step": "multi-query: weights rounded to the dtype, P.V on the matrix cores",
    "test_gpu_shared_prefix": "shared prefix: prefix tasks with weights rounded to the dtype on "
                              "the matrix cores, private blocks in fp32",
    "test_gpu_quant": "8-bit cache: weights (times the V scale for bf16) rounded to the dtype, "
                      "P.V on the matrix cores",
    "test_block_manager": "single-query: fp32 weights, P.V on the vector ALU",
}


def records_table() -> str:
    """Markdown table of RECORDS, grouped by test module, with the bars."""
    lines = ["| test | compared | dtype | elements | max-abs | mean-abs | rel-L2 | bars "
             "(max-abs / mean-abs / rel-L2) | ok |", "|---|---|---|---|---|---|---|---|---|"]
    by_path: dict[str, list] = {}
    for r in RECORDS:
        mod = r["test"].split("::")[0].rsplit("/", 1)[-1].removesuffix(".py")
        by_path.setdefault(PATHS.get(mod, mod), []).append(r)
        b = BARS[r["dtype"]]
        bars = f"{b['max_abs']:g} / {b['mean_abs'] if b['mean_abs'] is not None else '-'} / " \
               f"{b['rel_l2']:g}"
        lines.append(f"| `{r['test'].split('/')[-1]}` | {r['what']} | {r['dtype']} | "
                     f"{r['elements']} | {r['max_abs']:.3e} | {r['mean_abs']:.3e} | "
                     f"{r['rel_l2']:.3e} | {bars} | {'yes' if r['ok'] else 'NO'} |")
    summary = ["| weighted-sum path | comparisons | dtype | worst max-abs | worst mean-abs | "
               "worst rel-L2 |", "|---|---|---|---|---|---|"]
    for path, rs in by_path.items():
        for dt in sorted({r["dtype"] for r in rs}):
            sel = [r for r in rs if r["dtype"] == dt]
            summary.append(f"| {path} | {len(sel)} | {dt} | "
                           f"{max(r['max_abs'] for r in sel):.3e} | "
                           f"{max(r['mean_abs'] for r in sel):.3e} | "
                           f"{max(r['rel_l2'] for r in sel):.3e} |")
    return "\n".join(summary) + "\n\n" + "\n".join(lines) + "\n"
