import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Tie-band records of the mask checks (tests/parity_utils.py), one per checked
# token: printed at the end of the run so that the counts of channels inside
# the 1e-3 band around the k-th value (or tau_s), and of channels where the
# GPU mask differs from the oracle's, are visible in the run's output even
# under -q.
BAND_RECORDS = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    if not BAND_RECORDS:
        return
    by = {}
    for r in BAND_RECORDS:
        d = by.setdefault(r["case"], dict(tokens=0, band=0, band_max=0, diff=0, diff_max=0))
        d["tokens"] += 1
        d["band"] += r["band"]
        d["band_max"] = max(d["band_max"], r["band"])
        d["diff"] += r["diff"]
        d["diff_max"] = max(d["diff_max"], r["diff"])
    tr = terminalreporter
    tr.write_sep("-", "mask tie bands (GPU vs oracle)")
    tot_t = sum(d["tokens"] for d in by.values())
    tot_d = sum(d["diff"] for d in by.values())
    for case, d in sorted(by.items()):
        tr.write_line(f"{case}: {d['tokens']} tokens, band {d['band']} (max {d['band_max']}), "
                      f"differing {d['diff']} (max {d['diff_max']})")
    tr.write_line(f"all: {tot_t} tokens checked, {tot_d} channels differing (all inside the band)")


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(os.path.join(ROOT, "tests", "golden", name)) as f:
            return json.load(f)
    return load
