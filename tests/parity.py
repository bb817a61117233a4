"""Shared helpers of the GPU parity tests: tolerances and error reports.

The bars: out max abs error <= 1e-3 (fp16; the accuracy check of the
"optimizing-attention-flash" skill page, §3 workflow one) and <= 8e-3 (bf16);
lse relative error <= 1e-4, read as |Δlse| <= 1e-4 * max(1, |lse|); -inf must
match -inf exactly.

Output rounding: the kernel's out is rounded to fp16/bf16, while the oracle is
exact float64.  Where |out| >= 2 (fp16) half an ulp of the output type is
already ~1e-3, so an element can exceed the raw bound from its own final
rounding alone.  Such elements are reported as "rounding-limited" and accepted
only if the error net of half an ulp of the oracle value is within the bound;
every other element must meet the raw bound.
"""

from __future__ import annotations

import numpy as np
import torch

TOL = {torch.float16: 1e-3, torch.bfloat16: 8e-3}
MANT = {torch.float16: 10, torch.bfloat16: 7}
LSE_REL = 1e-4


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


def check(out, lse, ref_out, ref_lse, dtype, label="", max_limited_frac=1e-3):
    """Assert the GPU (out, lse) meet the bars against the oracle; return a report dict."""
    o = to64(out)
    r = np.asarray(ref_out, dtype=np.float64)
    assert o.shape == r.shape, (label, o.shape, r.shape)
    assert np.isfinite(o).all(), f"{label}: non-finite values in out"
    err = np.abs(o - r)
    tol = TOL[dtype]
    raw_bad = err > tol
    net = err - half_ulp(r, dtype)
    hard = raw_bad & (net > tol)
    limited = raw_bad & ~hard
    rep = dict(label=label, max_abs_err=float(err.max(initial=0.0)),
               max_net_err=float(np.maximum(net, 0).max(initial=0.0)),
               rounding_limited=int(limited.sum()), n=int(err.size))
    assert not hard.any(), f"{label}: {int(hard.sum())} elements over {tol} (max err {err.max():.3e})"
    assert limited.sum() <= max(1, max_limited_frac * err.size), f"{label}: too many rounding-limited elements {rep}"
    if lse is not None:
        lg = to64(lse)
        lr = np.asarray(ref_lse, dtype=np.float64)
        assert lg.shape == lr.shape, (label, lg.shape, lr.shape)
        ninf_r = np.isneginf(lr)
        assert (np.isneginf(lg) == ninf_r).all(), f"{label}: -inf pattern of lse differs"
        fin = ~ninf_r
        assert np.isfinite(lg[fin]).all(), f"{label}: non-finite lse"
        lerr = np.abs(lg[fin] - lr[fin]) / np.maximum(1.0, np.abs(lr[fin]))
        rep["lse_rel_err"] = float(lerr.max(initial=0.0))
        assert rep["lse_rel_err"] <= LSE_REL, f"{label}: lse rel err {rep['lse_rel_err']:.3e}"
    print("parity", rep, flush=True)
    return rep
