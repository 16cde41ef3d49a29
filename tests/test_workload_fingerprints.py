"""The seeded input generator reproduces the recorded fingerprints of all
six workloads (tests/golden/workload_sha256.txt, written by
tests/golden/make_workload_sha256.py)."""
import importlib.util
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "workload_sha256.txt")


def _maker():
    spec = importlib.util.spec_from_file_location("make_workload_sha256",
                                                  os.path.join(HERE, "golden", "make_workload_sha256.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _recorded():
    rec = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, arr, shape, h = line.split()
            rec.setdefault(name, {})[arr] = (shape, h)
    return rec


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_workload_arrays_match_fingerprints(cfg):
    mk = _maker()
    rec = _recorded()
    rows = mk.fingerprints(cfg)
    name = rows[0][0]
    assert set(rec[name]) == {r[1] for r in rows}
    for _, arr, shape, h in rows:
        assert rec[name][arr] == ("x".join(map(str, shape)), h), (name, arr)
