import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path)")
    config.addinivalue_line("markers", "slow: long CPU oracle run")


def report_err(name, got, want):
    """Max abs, mean abs and max relative error, printed and returned."""
    import numpy as np
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = np.abs(got - want)
    max_abs = float(diff.max()) if diff.size else 0.0
    mean_abs = float(diff.mean()) if diff.size else 0.0
    rel = diff / np.maximum(np.abs(want), 1e-30)
    max_rel = float(rel.max()) if rel.size else 0.0
    print(f"[{name}] max_abs={max_abs:.3e} mean_abs={mean_abs:.3e} "
          f"max_rel={max_rel:.3e} n={diff.size}", flush=True)
    return max_abs, mean_abs, max_rel
