"""GPU parity of the single-precision paths against the oracle's binary32
functions: the binary32 stencil and column solve, PCG in binary32, and binary64
PCG with the column preconditioner in binary32 (the paper's section 7 runs
the solver in both precisions).

Tolerances, derived from the arithmetic (each side is a plain binary32
computation of the same formula; the GPU contracts into FMAs and groups the
column solve into segments):
  * stencil: |y_gpu - y_orc| <= 16 eps32 S, as for binary64;
  * column solve: the forward error of a binary32 Thomas solve on the stiff
    columns here can reach 1e-3 relative (the oracle's own binary32 solve
    shows it), so it is judged by what the method fixes: the backward error
    |r - M z_gpu| <= 4 (L + P) eps32 (|M| |z_gpu|) per element -- the
    segmented elimination takes each value through a local sweep of L levels
    and two scans over the P segments (the oracle's sequential sweep stays
    below 1 eps32) -- and the GPU's distance to the binary64 solve at most 4x
    the oracle's binary32 distance (+ 16 eps32 ||z||);
  * binary32 PCG: step counts within 2, distance to the converged binary64
    solution within 1.5x the oracle's (+ 1e-6); residual histories (while
    ||r|| >= 1e-3 ||r0||) and fixed-step iterates within max(1e-4, 10 f),
    where f is the oracle's binary32 column-solve forward error on the
    right-hand side of the same workload: two correct binary32 runs that
    round the column solve differently diverge by that much per step;
  * mixed PCG: converged with the true residual ||b - A x||/||b|| <= 10 tol
    (binary64, evaluated by the oracle), within 1e-8 of the oracle's mixed
    solution, and the history, level crossings and step count held by
    check_mixed_against_oracle: the step count lies between the oracle's
    binary64 and mixed counts, within 1 (rounding in the binary32
    preconditioner can stall the run near tol for some steps: on the
    32x32x16 workload the oracle's mixed run stalls for 15 steps, 92 against
    77 in binary64, and the GPU's for none).
"""
import numpy as np
import pytest

import matrix_free_pcg_amd as mf
import oracle
from gpu_helpers import check_mixed_against_oracle, require_gpu, stencil_scale, to_host
from matrix_free_pcg_amd import workloads as W

pytestmark = pytest.mark.gpu

EPS32 = float(np.finfo(np.float32).eps)

GRIDS = [
    ("cfg1-32x32x16", lambda: W.config_problem(1)),
    ("cfg2-128x128x64", lambda: W.config_problem(2)),
    ("cfg4-70x45x40", lambda: W.config_problem(4, scale_xy=(70, 45), nz=40)),
    ("cfg4-128x24x64", lambda: W.config_problem(4, scale_xy=(128, 24), nz=64)),
    ("cfg4-65x4x130", lambda: W.config_problem(4, scale_xy=(65, 4), nz=130)),
    ("cfg4-5x3x300", lambda: W.config_problem(4, scale_xy=(5, 3), nz=300)),
    ("cfg3-1x1x7", lambda: W.config_problem(3, scale_xy=(1, 1), nz=7)),
    ("cfg4-2x2x1", lambda: W.config_problem(4, scale_xy=(2, 2), nz=1)),
    ("cfg4-64x2x512", lambda: W.config_problem(4, scale_xy=(64, 2), nz=512)),
]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def to_dev32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_dev64(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dev)


def column_coeffs(prob):
    """alpha_T per column and the faces below / above every level (binary64)."""
    ah = prob.alpha_h_field()
    ax = 0.5 * (ah + np.roll(ah, -1, axis=1))
    ay = 0.5 * (ah + np.roll(ah, -1, axis=0))
    aT = ax + np.roll(ax, 1, axis=1) + ay + np.roll(ay, 1, axis=0)      # [ny, nx]
    lo = prob.alpha_z_face[:-1][None, :, None]                           # face below level k
    up = prob.alpha_z_face[1:][None, :, None]                            # face above level k
    return aT[:, None, :], lo, up


def segment_geometry(nz):
    """Segment length L and count P of the 64-column preconditioner pass (the
    smallest L of 8, 16, 32 with 64 * ceil(nz / L) <= 1024 threads)."""
    for L in (8, 16, 32):
        if 64 * -(-nz // L) <= 1024:
            return L, -(-nz // L)
    raise ValueError(nz)


def precond_f32_forward_error(prob, r):
    """The oracle's binary32 column solve against its binary64 one, relative."""
    z64 = oracle.precond(prob, np.asarray(r, dtype=np.float64))
    z32 = oracle.precond_f32(prob, np.asarray(r, dtype=np.float32)).astype(np.float64)
    return np.abs(z32 - z64).max() / np.abs(z64).max()


def backward_error(prob, r, z):
    """max_l |r - M z|_l / (|M| |z|)_l with M the column matrices (eq. (19))."""
    aT, lo, up = column_coeffs(prob)
    zm = np.concatenate([z[:, :1, :], z[:, :-1, :]], axis=1)      # level k-1 (face 0 carries 0)
    zp = np.concatenate([z[:, 1:, :], z[:, -1:, :]], axis=1)      # level k+1 (face nz carries 0)
    diag = prob.delta + aT + lo + up
    Mz = diag * z - lo * zm - up * zp
    absMz = diag * np.abs(z) + lo * np.abs(zm) + up * np.abs(zp)
    return np.max(np.abs(r - Mz) / np.maximum(absMz, 1e-300))


@pytest.mark.parametrize("label,make", GRIDS, ids=[g[0] for g in GRIDS])
def test_apply_A_f32_matches_oracle(dev, label, make):
    import torch
    prob = make()
    x = W.uniform_field(prob.nx, prob.ny, prob.nz, 101).astype(np.float32)
    h = mf.pcg_create(prob)
    try:
        xd = to_dev32(x, dev)
        yd = torch.full_like(xd, float("nan"))
        mf.pcg_apply_A_f32(h, xd, yd)
        torch.cuda.synchronize()
        y = to_host(yd)
    finally:
        mf.pcg_destroy(h)
    ref = oracle.apply_A_f32(prob, x)
    err = np.abs(y.astype(np.float64) - ref).max()
    assert np.isfinite(y).all()
    assert err <= 16 * EPS32 * stencil_scale(prob, x), (label, err)


@pytest.mark.parametrize("label,make", GRIDS, ids=[g[0] for g in GRIDS])
def test_precond_f32_matches_oracle(dev, label, make):
    import torch
    prob = make()
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 202).astype(np.float32)
    h = mf.pcg_create(prob)
    try:
        rd = to_dev32(r, dev)
        zd = torch.full_like(rd, float("nan"))
        mf.pcg_precond_f32(h, rd, zd)
        torch.cuda.synchronize()
        z = to_host(zd).astype(np.float64)
    finally:
        mf.pcg_destroy(h)
    r64 = r.astype(np.float64)
    z64 = oracle.precond(prob, r64)
    zo = oracle.precond_f32(prob, r).astype(np.float64)
    assert np.isfinite(z).all()
    be = backward_error(prob, r64, z)
    L, P = segment_geometry(prob.nz)
    assert be <= 4 * (L + P) * EPS32, (label, "backward error", be, L, P)
    fg = np.abs(z - z64).max()
    fo = np.abs(zo - z64).max()
    assert fg <= 4 * fo + 16 * EPS32 * np.abs(z64).max(), (label, fg, fo)
    # the two binary32 column solves against each other, per application on
    # the same r: both sum the pivots' diagonal in the same order; they
    # differ in the segment scans (the GPU's elimination is split into
    # segments) and in fused multiply-adds
    # (measured: 0.07-0.39 of the binary32 rounding |z_orc32 - z_orc64| on the
    # variable-coefficient grids, 1.16 on the constant one, where both are at
    # the rounding floor); a systematic difference, such as pivots summed in
    # another order, exceeds it
    dz = np.abs(z - zo).max()
    print(f"{label}: |z_gpu32 - z_orc32| {dz:.2e}, |z_orc32 - z_orc64| {fo:.2e} (ratio {dz / max(fo, 1e-300):.2f})")
    assert dz <= 2 * fo + 4 * EPS32 * np.abs(z64).max(), (label, dz, fo)


SOLVES = [
    ("cfg1", lambda: W.make_workload(1)),
    ("cfg2", lambda: W.make_workload(2)),
    ("cfg4-70x45x40", lambda: W.make_workload(4, scale_xy=(70, 45), nz=40)),
    ("cfg4-128x24x64", lambda: W.make_workload(4, scale_xy=(128, 24), nz=64)),
]


def _gpu_solve(fn, prob, b, tol, maxit, dev, conv):
    import torch
    h = mf.pcg_create(prob)
    try:
        bd = conv(b, dev)
        xd = torch.zeros_like(bd)
        res = fn(h, bd, xd, tol, maxit)
        torch.cuda.synchronize()
        return res, to_host(xd).astype(np.float64)
    finally:
        mf.pcg_destroy(h)


@pytest.mark.parametrize("label,make", SOLVES, ids=[c[0] for c in SOLVES])
def test_solve_f32_matches_oracle(dev, label, make):
    w = make()
    prob, tol = w.problem, 1e-5
    b32 = w.rhs.astype(np.float32)
    res, xg = _gpu_solve(mf.pcg_solve_f32, prob, b32, tol, 5000, dev, to_dev32)
    ref = oracle.pcg_f32(prob, b32, tol=tol, maxit=5000)
    assert res["status"] == ref["status"] == 0, (label, res, ref["status"])
    assert abs(res["iters"] - ref["iters"]) <= 2, (label, res["iters"], ref["iters"])
    xs = oracle.pcg(prob, b32.astype(np.float64), tol=1e-13, maxit=20000)["x"]
    ns = np.linalg.norm(xs)
    eg = np.linalg.norm(xg - xs) / ns
    eo = np.linalg.norm(ref["x"].astype(np.float64) - xs) / ns
    print(f"{label} f32: iters gpu {res['iters']} oracle {ref['iters']}; to x*: gpu {eg:.2e} oracle {eo:.2e}")
    assert eg <= 1.5 * eo + 1e-6, (label, eg, eo)
    # histories, against the binary32 rounding level of the column solve
    f = precond_f32_forward_error(prob, b32)
    n = min(len(res["hist"]), len(ref["hist"]))
    hg, ho = res["hist"][:n], ref["hist"][:n]
    assert abs(hg[0] - ho[0]) <= 1e-6 * ho[0]
    big = ho >= 1e-3 * ho[0]
    dev_g = np.max(np.abs(hg[big] - ho[big]) / ho[big])
    print(f"{label} f32: history deviation {dev_g:.2e} (binary32 column-solve error {f:.2e})")
    assert dev_g <= max(1e-4, 10 * f), (label, dev_g, f)


@pytest.mark.parametrize("label,make", SOLVES, ids=[c[0] for c in SOLVES])
def test_solve_mixed_matches_oracle(dev, label, make):
    w = make()
    prob, tol = w.problem, w.tol
    res, xg = _gpu_solve(mf.pcg_solve_mixed, prob, w.rhs, tol, w.maxit, dev, to_dev64)
    ref = oracle.pcg_mixed(prob, w.rhs, tol=tol, maxit=w.maxit)
    r64 = oracle.pcg(prob, w.rhs, tol=tol, maxit=w.maxit)
    assert res["status"] == ref["status"] == 0, (label, res, ref["status"])
    check_mixed_against_oracle(label, res["hist"], res["iters"], ref["hist"], ref["iters"], r64["hist"],
                               r64["iters"])
    tr = np.linalg.norm(w.rhs - oracle.apply_A(prob, xg)) / np.linalg.norm(w.rhs)
    rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
    print(f"{label} mixed: iters gpu {res['iters']} oracle {ref['iters']} (binary64 {r64['iters']}); "
          f"true residual {tr:.2e}; rel-L2 to oracle {rel:.2e}")
    assert tr <= 10 * tol, (label, tr)
    assert rel <= 1e-8, (label, rel)


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_f32_and_mixed_first_steps(dev, steps):
    """Fixed step counts (tol = 0): the iterates after k steps against the
    oracle's, within the binary32 rounding of k steps on this workload."""
    w = W.make_workload(4, scale_xy=(70, 45), nz=40)
    prob = w.problem
    b32 = w.rhs.astype(np.float32)
    bound = max(1e-4, 10 * precond_f32_forward_error(prob, b32))
    res, xg = _gpu_solve(mf.pcg_solve_f32, prob, b32, 0.0, steps, dev, to_dev32)
    ref = oracle.pcg_f32(prob, b32, tol=0.0, maxit=steps)
    assert res["iters"] == ref["iters"] == steps and res["status"] == 1
    rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
    print(f"steps {steps}: f32 rel-L2 {rel:.2e} (bound {bound:.2e})")
    assert rel <= bound, ("f32", steps, rel, bound)
    res, xg = _gpu_solve(mf.pcg_solve_mixed, prob, w.rhs, 0.0, steps, dev, to_dev64)
    ref = oracle.pcg_mixed(prob, w.rhs, tol=0.0, maxit=steps)
    assert res["iters"] == ref["iters"] == steps and res["status"] == 1
    rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
    hist = np.max(np.abs(res["hist"] - ref["hist"]) / ref["hist"])
    print(f"steps {steps}: mixed rel-L2 {rel:.2e}, history {hist:.2e}")
    assert rel <= bound and hist <= bound, ("mixed", steps, rel, hist, bound)


def test_f32_edge_cases(dev):
    import torch
    w = W.make_workload(4, scale_xy=(33, 5), nz=9)
    prob = w.problem
    h = mf.pcg_create(prob)
    try:
        b = torch.zeros(prob.ny, prob.nz, prob.nx, dtype=torch.float32, device=dev)
        x = torch.zeros_like(b)
        res = mf.pcg_solve_f32(h, b, x, 1e-5, 50)
        assert res["status"] == mf.PCG_OK and res["iters"] == 0
        with pytest.raises(TypeError):
            mf.pcg_solve_f32(h, b.double(), x.double(), 1e-5, 50)
        with pytest.raises(mf.PcgError):
            mf.pcg_solve_f32(h, b, b, 1e-5, 50)
        bad = w.rhs.astype(np.float32)
        bad[1, 2, 3] = np.nan
        res = mf.pcg_solve_f32(h, to_dev32(bad, dev), torch.zeros_like(b), 1e-5, 50)
        assert res["status"] == mf.PCG_ERR_BREAKDOWN
        bad64 = w.rhs.copy()
        bad64[1, 2, 3] = np.inf
        res = mf.pcg_solve_mixed(h, to_dev64(bad64, dev), torch.zeros_like(b).double(), 1e-10, 50)
        assert res["status"] == mf.PCG_ERR_BREAKDOWN
    finally:
        mf.pcg_destroy(h)


RANDOM_SHAPES = [(64, 4, 64), (24, 16, 16), (128, 12, 33), (55, 16, 48), (64, 8, 16), (109, 6, 128),
                 (128, 8, 64), (192, 4, 116)]


@pytest.mark.parametrize("nx,ny,nz", RANDOM_SHAPES, ids=lambda v: str(v))
def test_f32_and_mixed_random_shapes(dev, nx, ny, nz):
    """Two fixed steps of the binary32 and mixed solves against the oracle's
    on grid shapes that mix whole and ragged tiles (the binary32 stencil
    passes take 8-row tiles where ny allows, the others 4), within the
    binary32 rounding bound of the other fixed-step tests."""
    prob = W.config_problem(4, scale_xy=(nx, ny), nz=nz)
    b64 = W.uniform_field(nx, ny, nz, 61)
    b32 = b64.astype(np.float32)
    bound = max(1e-4, 10 * precond_f32_forward_error(prob, b32))
    res, xg = _gpu_solve(mf.pcg_solve_f32, prob, b32, 0.0, 2, dev, to_dev32)
    ref = oracle.pcg_f32(prob, b32, tol=0.0, maxit=2)
    assert res["iters"] == ref["iters"] == 2
    assert np.linalg.norm(xg - ref["x"]) <= bound * np.linalg.norm(ref["x"]), "f32"
    res, xg = _gpu_solve(mf.pcg_solve_mixed, prob, b64, 0.0, 2, dev, to_dev64)
    ref = oracle.pcg_mixed(prob, b64, tol=0.0, maxit=2)
    assert res["iters"] == ref["iters"] == 2
    assert np.linalg.norm(xg - ref["x"]) <= bound * np.linalg.norm(ref["x"]), "mixed"
