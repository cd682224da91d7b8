import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library; parity via the C ABI")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Print the worst GPU-vs-oracle errors each parity test recorded (tests/gpu_helpers.py), so that the session's
    output keeps the margins to the bounds: one line per test function (worst over its parameters), then the overall
    worst. The per-case figures also go to parity_margins.json in the run's output folder when it can be written."""
    try:
        from tests.gpu_helpers import MARGINS
    except Exception:
        return
    if not MARGINS:
        return
    import json

    def fmt(m):
        parts = []
        for key, label in (("out32", "fp32-out"), ("out", "out"), ("lse", "lse"), ("rel", "bound-used")):
            if key in m:
                parts.append(f"{label} {m[key]:.2e}" if key != "rel" else f"{label} {m[key]:.2f}")
        return "  ".join(parts)

    by_fn = {}
    for tid, m in MARGINS.items():
        fn = tid.split("::")[-1].split("[")[0]
        agg = by_fn.setdefault(fn, {"cases": 0})
        agg["cases"] += 1
        for k, v in m.items():
            agg[k] = max(agg.get(k, 0.0), v)
    tr = terminalreporter
    tr.write_sep("-", "parity margins: worst |gpu - oracle| (bounds: fp32 out 2e-3; out 2e-3 + 1e-2|ref|; lse 1e-4; "
                      "bound-used = worst |d| / elementwise bound)")
    for fn in sorted(by_fn):
        agg = by_fn[fn]
        tr.write_line(f"{fn} ({agg['cases']} cases): {fmt(agg)}")
    overall = {}
    for m in MARGINS.values():
        for k, v in m.items():
            overall[k] = max(overall.get(k, 0.0), v)
    tr.write_line(f"ALL {len(MARGINS)} cases: {fmt(overall)}")
    try:
        out_dir = os.path.join(ROOT, "gpurun_out")
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "parity_margins.json"), "w") as fh:
            json.dump(MARGINS, fh, indent=1, sort_keys=True)
    except OSError:
        pass
