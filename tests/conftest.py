import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def rel_l2(got, ref) -> float:
    """||got - ref||_2 / ||ref||_2 in float64."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(s):
    return float.fromhex(s) if "0x" in s else float(s)


def golden_q8_blocks():
    """The hand-worked int8 blocks of tests/golden/q8_blocks.txt: a list of
    {"name", "scale", "x" (32 floats), "codes" (32 ints)}."""
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, "q8_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("block"):
                cur = {"name": line.split()[1], "x": [], "codes": []}
                blocks.append(cur)
            elif line.startswith("scale"):
                cur["scale"] = _num(line.split()[1])
            else:
                a, b = line.split("->")
                cur["x"].append(_num(a.strip()))
                cur["codes"].append(int(b))
    return blocks
