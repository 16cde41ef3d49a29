"""Shared helpers of the GPU parity tests (HIP library through the C ABI vs
the CPU oracle on the same seeded inputs)."""
from __future__ import annotations

import os

import numpy as np
import pytest

EPS = np.finfo(np.float64).eps


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from matrix_free_pcg_amd import build as hipbuild
    if not os.path.exists(hipbuild.LIB):
        raise RuntimeError("libmfpcg.so is not built; build it before running GPU tests")
    return torch.device("cuda:0")


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dev)


def to_host(t):
    return t.detach().cpu().numpy()


def stencil_scale(prob, x):
    """S = (delta + 8 max alpha_h + 4 max alpha_z) * ||x||_inf: bounds the sum of
    the magnitudes of the terms of (A x) in any cell."""
    return (prob.delta + 8 * prob.alpha_h_field().max() + 4 * prob.alpha_z_face.max()) * np.abs(x).max()


def apply_tol(prob, x):
    """|y_gpu - y_oracle| per cell: each side rounds 7 products and 13 sums
    or differences whose partial sums are bounded by S, so each is within
    ~8 eps S of the exact value; 16 eps S covers both."""
    return 16 * EPS * stencil_scale(prob, x)


def column_cond_bound(prob):
    """Gershgorin bound of the condition number of the column matrices M_T:
    (delta + aT_max + 4 max alpha_z) / (delta + aT_min)."""
    ah = prob.alpha_h_field()
    ax = 0.5 * (ah + np.roll(ah, -1, axis=1))
    ay = 0.5 * (ah + np.roll(ah, -1, axis=0))
    aT = ax + np.roll(ax, 1, axis=1) + ay + np.roll(ay, 1, axis=0)
    return (prob.delta + aT.max() + 4 * prob.alpha_z_face.max()) / (prob.delta + aT.min())


def precond_tol(prob, z_ref):
    """Both sides run a backward-stable elimination of each column matrix;
    their difference is bounded by 64 eps cond(M_T) ||z||_inf."""
    return 64 * EPS * column_cond_bound(prob) * np.abs(z_ref).max()


def gen_scale(gp, x):
    """Bound on the sum of the term magnitudes of the general stencil in any
    cell, |T| a + d (sum of the cell's edges) + 4 |T| beta, times ||x||_inf."""
    T = gp.area
    hor = gp.d.max() * (gp.alpha_x + np.roll(gp.alpha_x, 1, axis=1) + gp.alpha_y + np.roll(gp.alpha_y, 1, axis=0)).max()
    return (T.max() * gp.a.max() + hor + 4 * T.max() * gp.beta_face.max()) * np.abs(x).max()


def gen_column_cond(gp):
    """Gershgorin bound of the condition number of the general operator's
    column matrices."""
    aT = gp.alpha_x + np.roll(gp.alpha_x, 1, axis=1) + gp.alpha_y + np.roll(gp.alpha_y, 1, axis=0)
    lo = (gp.area[:, None, :] * gp.a[None, :, None] + gp.d[None, :, None] * aT[:, None, :]).min()
    vert = gp.beta_face[:-1] + gp.beta_face[1:]
    hi = (gp.area[:, None, :] * (gp.a + 2 * vert)[None, :, None] + gp.d[None, :, None] * aT[:, None, :]).max()
    return hi / lo
