"""Seeded input generators: pinned to the published SplitMix64 outputs and to
the workload recipes (grid, faces, coefficient field, right-hand sides)."""
import math
import os

import numpy as np
import pytest

from matrix_free_pcg_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_vectors.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                s, t, v = line.split()
                rows.append((int(s), int(t), int(v)))
    return rows


def test_splitmix64_matches_published_outputs():
    rows = _golden()
    assert len(rows) >= 7
    for seed, t, v in rows:
        got = W.splitmix64_stream(seed, t + 1)[t]
        assert int(got) == v, (seed, t)


def test_uniform01_is_counter_based_and_in_range():
    c = np.arange(1000, dtype=np.uint64)
    u = W.uniform01(7, c)
    assert u.min() >= 0.0 and u.max() < 1.0
    # counter form == sequential stream (output t uses counter t)
    s = W.splitmix64_stream(7, 1000)
    assert np.array_equal((s >> np.uint64(11)).astype(np.float64) * 2.0 ** -53, u)


def test_field_value_depends_on_cell_not_layout():
    nx, ny, nz, seed = 5, 3, 4, 11
    f = W.uniform_field(nx, ny, nz, seed)
    assert f.shape == (ny, nz, nx)
    for (i, j, k) in [(0, 0, 0), (4, 2, 3), (1, 2, 0), (3, 0, 2)]:
        c = i + nx * (j + ny * k)
        assert f[j, k, i] == -1.0 + 2.0 * W.uniform01(seed, np.array([c], dtype=np.uint64))[0]


def test_gaussian_field_moments():
    g = W.gaussian_field(64, 64, 64, 2)
    assert abs(g.mean()) < 5e-3
    assert abs(g.std() - 1.0) < 5e-3


def test_config_recipes():
    p1 = W.config_problem(1)
    assert (p1.nx, p1.ny, p1.nz) == (32, 32, 16) and p1.delta == 1e-2
    assert p1.alpha_z_face[0] == 0 and p1.alpha_z_face[-1] == 0
    assert np.all(p1.alpha_z_face[1:-1] == 1e3)
    p2 = W.config_problem(2)
    nz = p2.nz
    assert p2.alpha_z_face[1] == pytest.approx(1e3 * (1 + 1 / nz) ** 2)
    assert p2.alpha_z_face[nz - 1] == pytest.approx(1e3 * (1 + (nz - 1) / nz) ** 2)
    p4 = W.config_problem(4, scale_xy=(16, 8), nz=8)
    ah = p4.alpha_h_field()
    assert ah.shape == (8, 16)
    i, j = 3, 5
    assert ah[j, i] == pytest.approx(1 + 0.5 * math.sin(2 * math.pi * i / 16) * math.cos(2 * math.pi * j / 8))
    assert p4.alpha_z_face[4] == pytest.approx(1e4 * (1 + 2 * 4 / 8) ** 2)
    w2 = W.make_workload(2, scale_xy=(16, 16), nz=8)
    assert abs(w2.rhs.mean()) < 1e-15
    w3 = W.make_workload(3, scale_xy=(16, 16), nz=8)
    assert w3.rhs is None and w3.x_true.shape == (16, 8, 16)
    assert np.abs(w3.x_true).max() <= 8.0
    w5 = W.make_workload(5, scale_xy=(8, 8), nz=4)
    assert w5.fixed_iterations and w5.maxit == 50 and w5.tol == 0.0
