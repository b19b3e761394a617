import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle cases that take tens of seconds on the CPU")


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


def pytest_terminal_summary(terminalreporter):
    """Per-comparison parity counts (codes and scales against the oracle), so
    that they stay in the output of every run, not only under -s."""
    from tests import parity

    if not parity.RESULTS:
        return
    tr = terminalreporter
    tr.section("parity counts (codes/scales vs oracle)")
    tr.write_line(f"{'comparison':44s} {'elements':>11s} {'mism':>5s} {'+0/-0':>5s} {'out-1e-6':>8s} "
                  f"{'1e-6 set':>8s} {'free':>6s} {'free blk':>8s} {'mism/elem':>9s}")
    for r in parity.RESULTS:
        tr.write_line(f"{r['label'][:44]:44s} {r['elements']:11d} {r['mismatches']:5d} {r['signed_zero']:5d} "
                      f"{r['mismatches_outside_literal']:8d} {r['literal_exempt']:8d} {r['free']:6d} "
                      f"{r['free_blocks']:8d} {r['mismatches'] / r['elements']:9.1e}")
    out = os.environ.get("BATQ_PARITY_JSON")  # optional: also keep the counts as JSON at this path
    if out:
        import json

        with open(out, "w") as f:
            json.dump(parity.RESULTS, f, indent=1)
