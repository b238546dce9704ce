"""Helpers for the GPU tests: moving the seeded numpy inputs to the device and
comparing device results with the oracle under the stated tolerances.

Every check returns its error summary: max-abs and max-rel error and `tol_used`, the
largest fraction of the elementwise tolerance any element uses (1.0 = at the bound).
`record()` prints a summary and, when MI_ATTN_PARITY_LOG names a file, appends it there as
one JSON line, so that the margins of a run can be kept."""
import json
import os

import numpy as np

F32_MAX_ABS = 1e-4             # fp32 inputs: max-abs error against the fp64 oracle
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2  # bf16 inputs: |gpu - ref| <= atol + rtol * |ref| elementwise
# fp16 inputs are held to the same 16-bit bound (fp16 keeps 3 more mantissa bits than
# bf16, so this bound is looser for it than for bf16)


def to_gpu(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> dict:
    """Assert the tolerance of `dtype` and return the error summary."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0
    if dtype == "f32":
        tol_used = max_abs / F32_MAX_ABS
        assert max_abs <= F32_MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
        ratio = err / bound
        tol_used = float(ratio.max()) if err.size else 0.0
        bad = err > bound
        if bad.any():
            idx = np.unravel_index(np.argmax(err - bound), err.shape)
            raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {idx}: "
                                 f"gpu {got[idx]:.6f} ref {ref[idx]:.6f} (max abs {max_abs:.3e})")
    return {"max_abs": max_abs, "max_rel": max_rel, "tol_used": tol_used, "elements": int(err.size)}


def record(what: str, summary: dict) -> dict:
    """Print a check's error summary and append it to $MI_ATTN_PARITY_LOG (JSON lines)."""
    line = {"what": what, **summary}
    print(f"[parity] {what}: max_abs {summary['max_abs']:.3e} max_rel {summary['max_rel']:.3e} "
          f"tol_used {summary['tol_used']:.3f} over {summary['elements']} elements", flush=True)
    path = os.environ.get("MI_ATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")
    return summary
