"""Comparison metrics between a GPU result and the fp64 oracle.

Test infrastructure (used by the test suite and the smoke check only).

* rel_l2: ||o - ref||_F / ||ref||_F over the whole tensor.
* allclose_report: the per-element gate |o - ref| <= atol + rtol * |ref|
  (the atol/rtol pair is the one the PyPTO BSA README states for its
  forward; section 1 and 6.1 of that page).
* row_gain: per output row, <o - ref, ref> / <ref, ref>, the coherent part of
  the error (flash-attention SM100 sparse-MLA page, "measurement" section).
* bf16_floor: the rms row gain of bf16(ref) - ref, i.e. what rounding the
  exact output to bf16 alone produces (same section).
* check_result: the per-element ratio gate of the ops-transformer pytest page
  (section 7), reported as a secondary metric.
"""
import numpy as np


def _a(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rel_l2(o, ref) -> float:
    o, ref = _a(o), _a(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((o - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def allclose_report(o, ref, atol, rtol) -> dict:
    """Per-element gate; returns fail fraction, worst violation ratio, max abs diff."""
    o, ref = _a(o), _a(ref)
    d = np.abs(o - ref)
    tol = atol + rtol * np.abs(ref)
    fail = d > tol
    n = d.size
    return {
        "fail_frac": float(fail.sum() / n) if n else 0.0,
        "n_fail": int(fail.sum()),
        "worst_ratio": float((d / tol).max()) if n else 0.0,
        "max_abs": float(d.max()) if n else 0.0,
        "nan": int(np.isnan(o).sum()),
    }


def lse_report(lse, ref) -> dict:
    """Max |lse - ref| over rows with a finite reference, plus the count of rows
    where the -inf pattern differs (an empty row must be -inf on both sides)."""
    lse, ref = _a(lse).ravel(), _a(ref).ravel()
    fin = np.isfinite(ref)
    mism = int(np.sum(np.isneginf(ref) != np.isneginf(lse)))
    err = float(np.abs(lse[fin] - ref[fin]).max()) if fin.any() else 0.0
    return {"max_abs": err, "neginf_mismatch": mism, "nan": int(np.isnan(lse).sum())}


def row_gain(o, ref) -> np.ndarray:
    """g_r = <o_r - ref_r, ref_r> / <ref_r, ref_r> for rows with a nonzero ref."""
    o, ref = _a(o), _a(ref)
    o = o.reshape(-1, o.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    den = np.einsum("rd,rd->r", ref, ref)
    keep = den > 0
    return np.einsum("rd,rd->r", o[keep] - ref[keep], ref[keep]) / den[keep]


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def round_to(ref, dtype):
    """Round-to-nearest-even of an fp64 array to a torch dtype, back in fp64."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(_a(ref)))
    return t.to(torch.float32).to(dtype).to(torch.float64).numpy()


def bf16_floor(ref) -> float:
    """rms row gain that rounding the exact output to bf16 alone produces."""
    import torch
    return rms(row_gain(round_to(ref, torch.bfloat16), ref))


def check_result(o, ref) -> dict:
    """ops-transformer pytest page, section 7: an element violates when
    |a - b| > max(max(|a|, |b|) * 0.005, 2.5e-5); the case fails when the
    violator ratio exceeds 0.005 or the max difference exceeds 0.1."""
    a, b = _a(o).ravel(), _a(ref).ravel()
    d = np.abs(a - b)
    thr = np.maximum(np.maximum(np.abs(a), np.abs(b)) * 0.005, 2.5e-5)
    ratio = float((d > thr).mean()) if d.size else 0.0
    dmax = float(d.max()) if d.size else 0.0
    return {"violator_ratio": ratio, "diff_max": dmax, "diff_sum": float(d.sum()),
            "passed": bool(ratio <= 0.005 and dmax <= 0.1)}
