import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a whitespace fixture: ``key v1 v2 ...`` lines, '#' comments."""
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def read_run_cases(name):
    """Parse ``case``/``run``/``end`` blocks of derived run fixtures."""
    cases, cur = {}, None
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"runs": []}
                cases[vals[0]] = cur
            elif key == "end":
                cur = None
            elif key == "run":
                cur["runs"].append([int(v) for v in vals])
            else:
                cur[key] = [int(v) for v in vals]
    return cases


@pytest.fixture(scope="session")
def golden():
    return read_golden
