import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name):
    """Parse a tests/golden/*.txt record file into {record: {key: value}}."""
    recs = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *kvs = line.split()
            rec = {}
            for kv in kvs:
                k, v = kv.split("=", 1)
                rec[k] = [float(x) if "." in x else int(x) for x in v.split(",")] if "," in v \
                    else (float(v) if "." in v else int(v))
            recs[head] = rec
    return recs
