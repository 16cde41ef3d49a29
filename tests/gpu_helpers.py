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


def first_below(hist, level):
    """First step k with hist[k] < level * hist[0] (or None)."""
    h = np.asarray(hist)
    k = np.flatnonzero(h < level * h[0])
    return int(k[0]) if k.size else None


def check_mixed_against_oracle(label, hg, iters_g, ho, iters_o, h64, iters_64):
    """The bars of the mixed-precision solve (binary64 CG, binary32 column
    solve) against the oracle's mixed solve (ho, iters_o) and its binary64
    solve (h64, iters_64).  Two binary32 column solves that round differently
    follow the binary64 trajectory until the residual reaches the level where
    the preconditioner's binary32 rounding dominates; there the run can stall
    for some steps before it crosses tol (on tiny-32x32x16 the oracle's stalls
    between 1.2e-10 and 2.4e-10 for 14 steps, binary32 arithmetic rounded
    like the GPU's does not).  So:
      * while ||r_k|| >= 1e-8 ||r_0||, the GPU history deviates from the
        oracle's mixed one by at most twice the oracle's own binary64-vs-mixed
        deviation over the same steps, plus 1e-6;
      * the first step below 1e-6, 1e-7 and 1e-8 of ||r_0|| is at most one
        step further from the oracle's mixed run than the oracle's own
        binary64 run is (where the residual is monotone they coincide; where
        it oscillates near a level the first crossing moves with rounding:
        on cfg4-128x24x64 the two oracle runs differ by up to 88 % in history
        there);
      * the step count at tol lies between the binary64 and the oracle's
        mixed count, within 1 (the stall lasts between none and the oracle's
        number of steps: 15 on tiny-32x32x16, 9-15 under rounding-level
        perturbations of b, none at 1024x1024x128)."""
    hg, ho, h64 = (np.asarray(v, dtype=np.float64) for v in (hg, ho, h64))
    n = min(len(hg), len(ho), len(h64))
    big = ho[:n] >= 1e-8 * ho[0]
    dev_g = float(np.max(np.abs(hg[:n][big] - ho[:n][big]) / ho[:n][big]))
    dev_64 = float(np.max(np.abs(h64[:n][big] - ho[:n][big]) / ho[:n][big]))
    cross = {lev: (first_below(hg, lev), first_below(ho, lev), first_below(h64, lev)) for lev in (1e-6, 1e-7, 1e-8)}
    print(f"{label} mixed: steps gpu {iters_g} oracle {iters_o} binary64 {iters_64}; history deviation "
          f"{dev_g:.2e} (oracle binary64-vs-mixed {dev_64:.2e}); crossings {cross}", flush=True)
    assert dev_g <= 2 * dev_64 + 1e-6, (label, dev_g, dev_64)
    for lev, (kg, ko, k64) in cross.items():
        assert kg is not None and ko is not None and k64 is not None, (label, lev, kg, ko, k64)
        assert abs(kg - ko) <= abs(k64 - ko) + 1, (label, lev, kg, ko, k64)
    lo, hi = min(iters_o, iters_64), max(iters_o, iters_64)
    assert lo - 1 <= iters_g <= hi + 1, (label, iters_g, iters_o, iters_64)
