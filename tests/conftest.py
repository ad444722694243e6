"""Shared pytest configuration.

Markers:
  gpu -- needs a real MI355X (run with ``-m gpu``); everything else runs on
         the CPU (``-m "not gpu"``).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X GPU")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a golden fixture: '#' comments, then 'key: value' lines.

    Values may continue on following lines that start with whitespace.
    """
    path = os.path.join(GOLDEN, name)
    out = {}
    key = None
    with open(path) as fh:
        for raw in fh:
            line = raw.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            if line[0] in " \t" and key is not None:
                out[key] += " " + line.strip()
                continue
            key, _, val = line.partition(":")
            key = key.strip()
            out[key] = val.strip()
    return out


def hex_u16(s):
    import numpy as np
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint16)


def hex_bytes(s):
    import numpy as np
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)
