import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a golden fixture: non-comment lines of `key values | key values | ...`.

    Returns a list of dicts mapping each key to its list of tokens; a `->` splits
    a line into `lhs` and `rhs` token lists instead.
    """
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if "->" in line:
                lhs, rhs = line.split("->")
                toks = lhs.split()
                rows.append({"key": toks[0], "lhs": toks[1:], "rhs": rhs.split()})
                continue
            row = {}
            for part in line.split("|"):
                toks = part.split()
                row[toks[0]] = toks[1:]
            rows.append(row)
    return rows


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.load()
    return oracle
