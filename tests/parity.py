"""Shared helpers of the GPU parity tests: tolerances and error reports.

The bars, applied to the raw error of every element: out max abs error
<= 1e-3 (fp16; the accuracy check of the "optimizing-attention-flash" skill
page, §3 workflow one, compares the whole output against standard attention
with a 1e-3 bound) and <= 8e-3 (bf16); lse relative error <= 1e-4, read as
|Δlse| <= 1e-4 * max(1, |lse|); -inf must match -inf exactly.

Every report also carries the error net of half an ulp of the output type at
the oracle value ("max_net_err") and the number of elements whose raw error is
over the bar but whose net error is not ("rounding_limited"): the part of an
error that the final rounding of out alone can cause.  These are reported, not
allowed: an element over the raw bar fails the check.

Every report is kept in REPORTS; tests/conftest.py prints a summary of them at
the end of the session (also under -q) and, when the environment variable
FA_PARITY_REPORT names a file, writes them there as JSON.
"""

from __future__ import annotations

import numpy as np
import torch

TOL = {torch.float16: 1e-3, torch.bfloat16: 8e-3}
MANT = {torch.float16: 10, torch.bfloat16: 7}
LSE_REL = 1e-4

REPORTS: list[dict] = []


def half_ulp(ref: np.ndarray, dtype) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    emin = -14 if dtype == torch.float16 else -126
    e = np.maximum(e, emin)
    return 0.5 * np.exp2(e - MANT[dtype])


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def check(out, lse, ref_out, ref_lse, dtype, label=""):
    """Assert the GPU (out, lse) meet the raw bars against the oracle; return the report."""
    o = to64(out)
    r = np.asarray(ref_out, dtype=np.float64)
    assert o.shape == r.shape, (label, o.shape, r.shape)
    assert np.isfinite(o).all(), f"{label}: non-finite values in out"
    err = np.abs(o - r)
    tol = TOL[dtype]
    over = err > tol
    net = err - half_ulp(r, dtype)
    i = int(np.argmax(err)) if err.size else 0
    rep = dict(label=label, dtype=str(dtype).replace("torch.", ""), n=int(err.size), bar=tol,
               max_abs_err=float(err.max(initial=0.0)), ref_at_max=float(r.flat[i]) if err.size else 0.0,
               max_net_err=float(np.maximum(net, 0).max(initial=0.0)), over_bar=int(over.sum()),
               rounding_limited=int((over & (net <= tol)).sum()), max_abs_ref=float(np.abs(r).max(initial=0.0)))
    if lse is not None:
        lg = to64(lse)
        lr = np.asarray(ref_lse, dtype=np.float64)
        assert lg.shape == lr.shape, (label, lg.shape, lr.shape)
        ninf_r = np.isneginf(lr)
        rep["lse_neginf_match"] = bool((np.isneginf(lg) == ninf_r).all())
        fin = ~ninf_r
        rep["lse_finite"] = bool(np.isfinite(lg[fin]).all())
        lerr = np.abs(lg[fin] - lr[fin]) / np.maximum(1.0, np.abs(lr[fin]))
        rep["lse_rel_err"] = float(np.nan_to_num(lerr, nan=np.inf).max(initial=0.0))
    REPORTS.append(rep)
    if over.any():
        idx = np.unravel_index(i, err.shape)
        raise AssertionError(f"{label}: {rep['over_bar']} elements over {tol}; max err {rep['max_abs_err']:.3e} at "
                             f"index {tuple(int(x) for x in idx)} (oracle {rep['ref_at_max']:.6f}, net of half an "
                             f"ulp {rep['max_net_err']:.3e}, {rep['rounding_limited']} rounding-limited)")
    if lse is not None:
        assert rep["lse_neginf_match"], f"{label}: -inf pattern of lse differs"
        assert rep["lse_finite"], f"{label}: non-finite lse"
        assert rep["lse_rel_err"] <= LSE_REL, f"{label}: lse rel err {rep['lse_rel_err']:.3e}"
    print("parity", rep, flush=True)
    return rep
