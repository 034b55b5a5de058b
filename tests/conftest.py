import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a ``key = value`` fixture; integer lists become lists of ints."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            parts = val.split()
            nums = [int(p) for p in parts]
            out[key] = nums if len(nums) > 1 else nums[0]
    return out


@pytest.fixture
def golden():
    return load_golden


def pytest_sessionfinish(session, exitstatus):
    """With FF_PARITY_SUMMARY=<path>, write the error statistics of every GPU
    parity case of the session (max |dO|, relative Frobenius, LSE, control
    ratio) as a markdown table."""
    path = os.environ.get("FF_PARITY_SUMMARY")
    if not path:
        return
    try:
        from ffharness import RECORDS
    except Exception:
        return
    if not RECORDS:
        return
    with open(path, "w") as f:
        f.write("| case | calls | bank checks | max abs dO | max (abs dO / gate) | max rel. Frobenius | "
                "max abs dLSE | min control ratio |\n")
        f.write("|---|---|---|---|---|---|---|---|\n")
        for name, st in RECORDS:
            ctl = "-" if st.min_control_ratio == float("inf") else f"{st.min_control_ratio:.1f}"
            f.write(f"| {name} | {st.calls} | {st.bank_checks} | {st.max_abs:.3e} | {st.max_gate_use:.3f} | "
                    f"{st.max_rel_fro:.3e} | {st.max_lse:.3e} | {ctl} |\n")
