"""Shared helpers of the GPU parity tests: upload, tolerance gates, reports.

Gates, against the unrounded fp64 oracle:
  rel-L2 <= 3e-3 for fp16/bf16, <= 1e-5 for fp32;
  per element |o - ref| <= 1e-4 + 7.8125e-3 |ref| + u_P * sum_j P_j |v_j|;
  the plain per-element gate |o - ref| <= 1e-4 + 7.8125e-3 |ref| on a
  fraction of elements of at least 1 - plain_cap: plain_cap = 0 (every
  element, the literal gate) for fp32 and for the full-size fp16 workloads,
  1e-3 for small fp16 cases (rows with a handful of keys, where rounding P
  alone can exceed the literal gate); for bf16 the cap is asserted on the
  full-size workloads it is derived for (2% for causal S=4096 and S=8192,
  0.6% for the top-k MLA workload) and reported elsewhere;
  |lse - ref| <= 1e-4 on rows with keys; rows without keys are -inf on both
  sides.
The atol/rtol pair is the forward tolerance of the PyPTO BSA README
(sections 1 and 6.1). The third term is the exact bound of the error that
rounding P to the 16-bit dtype (unit roundoff u_P: 2^-8 bf16, 2^-11 fp16,
2^-24 fp32) introduces before P.V: each p_j carries a relative error <= u_P
and enters O with weight |v_j| / l. sum_j P_j |v_j| is the oracle's output
with |V| in place of V.

Why bf16 cannot meet the literal gate everywhere and what caps it: the
output's own rounding (relative 2^-9) stays inside rtol = 2^-7, but rounding
P to bf16 adds an error of standard deviation about u_P |v| / sqrt(3 n) to a
row with n effective keys, comparable to atol + rtol |o| for n in the
hundreds. A bit-exact numpy emulation of this pipeline on the full causal
bf16 S=4096 output fails the literal gate on 1.07% of the elements (and on
0.20-0.30% of the top-k MLA output); the caps of 2% and 0.6% allow for the
row mix of a sample. Longer rows (S=8192) average the P-rounding errors over
more keys, so the S=4096 cap covers them. Short rows fail more often (a few
percent at 300 keys), which is why small bf16 cases only report the fraction.
A kernel with a real fault (a dropped tile, a wrong row, a lost rescale)
fails the derived gate above by orders of magnitude.
"""
import json
import math
import os
import sys

import numpy as np
import torch

from oracle import metrics

TOL = {
    torch.float32: dict(rel_l2=1e-5, atol=1e-4, rtol=7.8125e-3, u_p=2.0 ** -24, plain_cap=0.0),
    torch.float16: dict(rel_l2=3e-3, atol=1e-4, rtol=7.8125e-3, u_p=2.0 ** -11, plain_cap=1e-3),
    torch.bfloat16: dict(rel_l2=3e-3, atol=1e-4, rtol=7.8125e-3, u_p=2.0 ** -8, plain_cap=None),
}
LSE_TOL = 1e-4


def f32(x: float) -> float:
    """The float32 value the GPU receives for a Python float."""
    return float(np.float32(x))


def gpu(*ts):
    out = tuple(None if t is None else t.cuda() for t in ts)
    return out if len(out) > 1 else out[0]


def log(case: str, rep: dict):
    line = json.dumps({"case": case, **rep}, default=float)
    print(line)
    sys.stdout.flush()
    d = os.environ.get("FA_TEST_LOG_DIR")
    if d:
        with open(os.path.join(d, "parity.jsonl"), "a") as f:
            f.write(line + "\n")


def check(case, o, lse, o_ref, lse_ref, dtype, o_abs, extra=None, plain_cap=None, page_gate=False):
    """Compares GPU outputs (torch, any device) with the oracle (numpy fp64);
    o_abs is the oracle output with |V| (the P-rounding bound's weights).
    plain_cap overrides the dtype's cap on the fraction of elements failing
    the literal atol/rtol gate (0 = every element must pass it). page_gate
    also asserts the ops-transformer pytest page's comparison (section 7:
    at most 0.5% of elements off by more than 0.005 relative, none by more
    than 0.1), which the full-size fp16 workloads meet.
    Asserts the gates and returns the report."""
    o = o.detach().float().cpu().numpy().astype(np.float64)
    lse = lse.detach().cpu().numpy().astype(np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64).reshape(o.shape)
    o_abs = np.asarray(o_abs, dtype=np.float64).reshape(o.shape)
    lse_ref = np.asarray(lse_ref, dtype=np.float64).reshape(lse.shape)
    tol = TOL[dtype]
    cap = tol["plain_cap"] if plain_cap is None else plain_cap
    rep = {"dtype": str(dtype).replace("torch.", ""), "rows": int(lse.size)}
    rep["rel_l2"] = metrics.rel_l2(o, o_ref)
    d = np.abs(o - o_ref)
    gate = tol["atol"] + tol["rtol"] * np.abs(o_ref) + tol["u_p"] * o_abs
    n_fail = int((d > gate).sum())
    plain = metrics.allclose_report(o, o_ref, tol["atol"], tol["rtol"])
    rep.update({"fail_frac": n_fail / max(d.size, 1), "worst_ratio": float((d / gate).max()) if d.size else 0.0,
                "max_abs": plain["max_abs"], "nan": plain["nan"], "plain_gate_fail_frac": plain["fail_frac"],
                "plain_worst_ratio": plain["worst_ratio"], "plain_cap": cap})
    lr = metrics.lse_report(lse, lse_ref)
    rep.update({"lse_max_abs": lr["max_abs"], "lse_neginf_mismatch": lr["neginf_mismatch"],
                "lse_nan": lr["nan"]})
    cr = metrics.check_result(o, o_ref)
    rep["check_result"] = cr["violator_ratio"]
    if extra:
        rep.update(extra)
    log(case, rep)
    assert rep["nan"] == 0 and rep["lse_nan"] == 0, rep
    assert rep["rel_l2"] <= tol["rel_l2"], rep
    assert n_fail == 0, rep
    if cap == 0.0:
        assert plain["n_fail"] == 0, rep
    elif cap is not None:
        assert plain["fail_frac"] <= cap, rep
    assert rep["lse_max_abs"] <= LSE_TOL, rep
    assert rep["lse_neginf_mismatch"] == 0, rep
    if page_gate:
        assert cr["passed"], (rep, cr)
    return rep


def sample_rows(g, n_total, n, must=()):
    """Sorted distinct row ids: n random ones plus the ids in ``must``."""
    r = g.choice(n_total, size=min(n, n_total), replace=False)
    return np.unique(np.concatenate([r, np.asarray(list(must), dtype=np.int64)])).astype(np.int64)


def absv(v):
    """|V| in the oracle's input dtype (exact)."""
    return v.abs() if hasattr(v, "abs") else np.abs(v)
