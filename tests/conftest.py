import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work of more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, when no GPU is visible, except when the
    # gpu marker was selected explicitly (then a missing GPU is an error).
    selected = config.getoption("-m") or ""
    if "gpu" in selected and "not gpu" not in selected:
        return
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


# Labels of the workloads the benchmark times and the pages' configurations,
# whose parity figures are printed one per line at the end of the session.
_HEADLINE = ("c1_", "c2_", "c3_", "c4_", "c5_", "fp8 c3")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One summary of every parity check of the session (also under -q): the
    largest raw error per dtype against its bar, then one line per headline
    workload.  With FA_PARITY_REPORT=<file> the reports are also written as JSON."""
    try:
        import parity
    except ImportError:
        return
    reps = parity.REPORTS
    if not reps:
        return
    import json
    path = os.environ.get("FA_PARITY_REPORT")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(reps, f, indent=1)
    tr = terminalreporter
    tr.section("parity against the float64 oracle (raw max abs error vs bar)")
    for dt in sorted({r["dtype"] for r in reps}):
        rs = [r for r in reps if r["dtype"] == dt]
        worst = max(rs, key=lambda r: r["max_abs_err"] / r["bar"])
        lse = max((r.get("lse_rel_err", 0.0) for r in rs), default=0.0)
        tr.write_line(f"{dt}: {len(rs)} checks, {sum(r['n'] for r in rs)} elements, max raw err "
                      f"{worst['max_abs_err']:.3e} (bar {worst['bar']:g}, in {worst['label']!r}), over bar "
                      f"{sum(r['over_bar'] for r in rs)}, rounding-limited {sum(r['rounding_limited'] for r in rs)}, "
                      f"max lse rel err {lse:.2e}")
    for r in reps:
        if str(r["label"]).startswith(_HEADLINE):
            tr.write_line(f"{r['label']}: n={r['n']} max_abs_err={r['max_abs_err']:.3e} (bar {r['bar']:g}) "
                          f"max_net_err={r['max_net_err']:.3e} over_bar={r['over_bar']} "
                          f"rounding_limited={r['rounding_limited']} lse_rel_err={r.get('lse_rel_err', 0.0):.2e}")
