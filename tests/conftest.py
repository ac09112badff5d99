import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def hand_code(state):
    """Weight value of a trellis state from the hand-derived golden fixture (not the oracle)."""
    import numpy as np
    for row in golden_rows("code_hand_values.txt"):
        if int(row[0], 16) == state:
            return float(np.array([int(row[7], 16)], np.uint16).view(np.float16)[0])
    raise KeyError(state)
