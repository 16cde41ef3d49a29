"""GPU parity of the tensor-product multigrid preconditioner (horizontal
Galerkin coarsening with piecewise-constant transfers, damped column-block
smoother, V(nu, nu) cycle, damped or Chebyshev-accelerated coarsest sweeps)
against the oracle's multigrid functions (pinned by M1-M7).

Tolerances:
  * coarse coefficients: bit-exact (both sides sum the same binary64 values
    in the same order, additions only);
  * one V-cycle z = B r: every sweep is a stencil pass and a column solve
    whose GPU and oracle results differ by rounding, and the coarsest
    single column (no horizontal coupling left: |T| (a_k + vertical
    Laplacian), condition ~4e7 for the general operators) turns a pivot
    rounded differently into a difference of eps * kappa.  The bar is
    therefore the oracle's own spread when every coefficient is perturbed
    by one ulp (the GPU's result is that of a problem rounded a few ulps
    apart): |z_gpu - z_orc| <= max(1e-11, 8 spread) ||z_orc||_inf.  The
    full-depth cycles measure 4e-10 to 1.3e-9 for that spread (1e-16 for
    a perturbed r: the sensitivity is the matrix's, not the input's) and
    4e-10 to 1.4e-9 for the GPU; the others 1e-13 and below 6e-13;
  * solves: as the other solve tests (iterations within 1, final iterates
    within rel-L2 1e-9, residual histories within 10x the oracle's own
    spread under an ulp-level perturbation of b, floor 1e-6);
  * at full size, where the oracle is too slow, properties that hold at any
    size: B is symmetric (<B u, v> = <u, B v>) and positive, and the solve
    converges with a true residual within 10 tol."""
import dataclasses

import numpy as np
import pytest

import matrix_free_pcg_amd as mf
import oracle
from gpu_helpers import require_gpu, to_dev, to_host
from matrix_free_pcg_amd import workloads as W
from oracle_pins import general_from_special, random_general

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def as_general(prob):
    return prob if isinstance(prob, W.GeneralProblem) else general_from_special(prob)


def coefficient_spread(gp, r, mg, seeds=(700, 701)):
    """Largest relative change of the oracle's V-cycle when every
    coefficient (a, d, beta, |T|, alpha_x, alpha_y) is multiplied by
    1 + 2^-52 u, u uniform in [-1, 1]: how far apart two correct cycles on
    operators rounded one ulp apart lie."""
    zo = oracle.mg_vcycle(gp, r, **mg)
    spread = 0.0
    for seed in seeds:
        rng = np.random.default_rng(seed)
        kw = {}
        for name in ("a", "d", "beta_face", "area", "alpha_x", "alpha_y"):
            v = np.asarray(getattr(gp, name), dtype=np.float64)
            kw[name] = np.ascontiguousarray(v * (1.0 + 2.0 ** -52 * rng.uniform(-1.0, 1.0, size=v.shape)))
        zp = oracle.mg_vcycle(dataclasses.replace(gp, **kw), r, **mg)
        spread = max(spread, float(np.abs(zp - zo).max() / np.abs(zo).max()))
    return zo, spread


GRIDS = [
    ("general-128x64x16", lambda: W.general_problem(128, 64, 16, 6)),
    ("varying-96x40x12", lambda: W.config_problem(4, scale_xy=(96, 40), nz=12)),
    ("random-8x2x5", lambda: random_general(8, 2, 5, seed=21)),
    ("random-1x16x6", lambda: random_general(1, 16, 6, seed=22)),
    ("random-6x10x9", lambda: random_general(6, 10, 9, seed=23)),
    ("random-1x1x7", lambda: random_general(1, 1, 7, seed=24)),
    ("random-5x3x4", lambda: random_general(5, 3, 4, seed=25)),
    ("general-64x64x128", lambda: W.general_problem(64, 64, 128, 6)),
    # 16- and 32-level segments (nz > 128): the two-pass sweeps
    ("general-64x8x256", lambda: W.general_problem(64, 8, 256, 6)),
    ("random-4x4x300", lambda: random_general(4, 4, 300, seed=26)),
]
PARAMS = [
    dict(nu=1, omega=0.8, max_levels=0, coarse_sweeps=2),
    dict(nu=2, omega=0.7, max_levels=3, coarse_sweeps=3),
    dict(nu=1, omega=1.0, max_levels=2, coarse_sweeps=1),
    # Chebyshev-accelerated coarsest sweeps on [coarse_lo, 2]: a three-level
    # hierarchy, the grid alone (every step of the solve is the Chebyshev
    # iteration, its last step forming the dot products) and nu = 2
    dict(nu=1, omega=0.9, max_levels=3, coarse_sweeps=8, coarse_lo=0.02),
    dict(nu=1, omega=0.9, max_levels=1, coarse_sweeps=6, coarse_lo=0.1),
    dict(nu=2, omega=0.8, max_levels=2, coarse_sweeps=16, coarse_lo=0.02),
]


def _pid(i):
    p = PARAMS[i]
    tag = "nu{nu}-w{omega}-L{max_levels}-cs{coarse_sweeps}".format(**p)
    return tag + (f"-lo{p['coarse_lo']}" if p.get("coarse_lo") else "")


@pytest.mark.parametrize("label,make", GRIDS, ids=[g[0] for g in GRIDS])
def test_mg_levels_match_oracle(dev, label, make):
    prob = make()
    gp = as_general(prob)
    h = mf.pcg_create(prob)
    try:
        mf.pcg_mg_setup(h)
        nlev = mf.pcg_mg_num_levels(h)
        levels = [mf.pcg_mg_level(h, l) for l in range(nlev)]
    finally:
        mf.pcg_destroy(h)
    assert nlev == oracle.mg_num_levels(gp.nx, gp.ny), (label, nlev)
    # level 0 is the operator in general form as the oracle's side builds it
    # (edge = mean of the two cells' alpha_h: one addition and one halving,
    # identical in binary64), and every coarser level is the oracle's
    # coarsening of the level above, bit for bit (the same additions in the
    # same order)
    nx0, ny0, area0, ax0, ay0 = levels[0]
    assert (nx0, ny0) == (gp.nx, gp.ny), label
    assert np.array_equal(area0, gp.area) and np.array_equal(ax0, gp.alpha_x) and \
        np.array_equal(ay0, gp.alpha_y), label
    cur = gp
    for l in range(1, nlev):
        cur = oracle.mg_coarsen(cur)
        nx, ny, area, ax, ay = levels[l]
        assert (nx, ny) == (cur.nx, cur.ny), (label, l)
        assert np.array_equal(area, cur.area) and np.array_equal(ax, cur.alpha_x) and \
            np.array_equal(ay, cur.alpha_y), (label, l)
    assert cur.nx * cur.ny == 1 or oracle.mg_coarsen(cur) is None, label


@pytest.mark.parametrize("pi", range(len(PARAMS)), ids=_pid)
@pytest.mark.parametrize("label,make", GRIDS, ids=[g[0] for g in GRIDS])
def test_vcycle_matches_oracle(dev, label, make, pi):
    import torch
    prob = make()
    gp = as_general(prob)
    mg = PARAMS[pi]
    r = W.gaussian_field(gp.nx, gp.ny, gp.nz, 303)
    h = mf.pcg_create(prob)
    try:
        mf.pcg_mg_setup(h, **mg)
        rd = to_dev(r, dev)
        zd = torch.full_like(rd, float("nan"))
        mf.pcg_mg_vcycle(h, rd, zd)
        # a second cycle on the same workspace gives the same result
        zd2 = torch.full_like(rd, float("nan"))
        ws = torch.full((mf.pcg_mg_workspace_bytes(h, 0),), 255, dtype=torch.uint8, device=dev)
        mf.pcg_mg_vcycle(h, rd, zd2, ws)
        torch.cuda.synchronize()
        z, z2 = to_host(zd), to_host(zd2)
    finally:
        mf.pcg_destroy(h)
    zo, spread = coefficient_spread(gp, r, mg)
    err = np.abs(z - zo).max() / np.abs(zo).max()
    bar = max(1e-11, 8.0 * spread)
    print(f"{label} {mg}: rel max err {err:.2e} (coefficient spread {spread:.2e}, bar {bar:.2e})")
    assert np.all(np.isfinite(z)) and err <= bar, (label, mg, err, spread)
    assert np.array_equal(z, z2), label




def test_first_sweep_segments_agree(dev, monkeypatch):
    """On the finest level the first sweep takes the 16-level segments of the
    column passes (nz = 128 over the 8-level multiplier table); with
    MFPCG_COL_LF=8 (read at pcg_create) it takes the table's 8-level ones.
    The same elimination either way: a V-cycle (first sweep without q) and 5
    steps of the multigrid solve (first sweep with r -= alpha q) agree to
    rounding."""
    import torch
    prob = W.general_problem(128, 64, 128, 8)
    mg = dict(nu=1, omega=0.9, max_levels=3, coarse_sweeps=8, coarse_lo=0.02)
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 305)
    b = W.uniform_field(prob.nx, prob.ny, prob.nz, 306)

    def run(lf):
        if lf is None:
            monkeypatch.delenv("MFPCG_COL_LF", raising=False)
        else:
            monkeypatch.setenv("MFPCG_COL_LF", lf)
        h = mf.pcg_create(prob)
        try:
            mf.pcg_mg_setup(h, **mg)
            rd = to_dev(r, dev)
            zd = torch.full_like(rd, float("nan"))
            mf.pcg_mg_vcycle(h, rd, zd)
            bd = to_dev(b, dev)
            xd = torch.zeros_like(bd)
            res = mf.pcg_solve_mg(h, bd, xd, 0.0, 5)
            torch.cuda.synchronize()
            return to_host(zd), to_host(xd), np.asarray(res["hist"]), mf.pcg_tuning_overrides(h)
        finally:
            mf.pcg_destroy(h)
            monkeypatch.delenv("MFPCG_COL_LF", raising=False)

    z16, x16, h16, ov16 = run(None)
    z8, x8, h8, ov8 = run("8")
    assert ov16 == 0 and ov8 & 0x004, (ov16, ov8)
    dz = np.abs(z16 - z8).max() / np.abs(z8).max()
    print(f"first sweep 16 vs 8 levels: V-cycle {dz:.2e}, histories {np.abs(h16 / h8 - 1).max():.2e}")
    assert np.isfinite(z16).all() and dz <= 1e-11, dz
    assert np.allclose(h16, h8, rtol=1e-11, atol=0)
    assert np.linalg.norm(x16 - x8) <= 1e-11 * np.linalg.norm(x8)

@pytest.mark.parametrize("width", ["16", "32", "64", "48"])
def test_coarsest_tile_width(dev, monkeypatch, width):
    """The coarsest level's tile width (MFPCG_MG_COARSE_C, read by
    pcg_mg_setup): 16, 32 and 64 columns per workgroup give the oracle's
    V-cycle within the V-cycle bar, the width the default rule picks (16 on
    this 32 x 16-column coarsest level, which has fewer tiles than the chip
    has CUs) gives the default's bits, the handle reports the override, and
    any other width is refused."""
    import torch
    prob = W.general_problem(128, 64, 16, 6)
    mg = dict(nu=1, omega=0.8, max_levels=3, coarse_sweeps=5)
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 304)

    def cycle(env):
        if env is None:
            monkeypatch.delenv("MFPCG_MG_COARSE_C", raising=False)
        else:
            monkeypatch.setenv("MFPCG_MG_COARSE_C", env)
        h = mf.pcg_create(prob)
        try:
            mf.pcg_mg_setup(h, **mg)
            rd = to_dev(r, dev)
            zd = torch.full_like(rd, float("nan"))
            mf.pcg_mg_vcycle(h, rd, zd)
            torch.cuda.synchronize()
            return to_host(zd), mf.pcg_tuning_overrides(h)
        finally:
            mf.pcg_destroy(h)
            monkeypatch.delenv("MFPCG_MG_COARSE_C", raising=False)

    if width == "48":
        with pytest.raises(mf.PcgError) as e:
            cycle(width)
        assert e.value.code == mf.PCG_ERR_INVALID
        return
    z_def, ov_def = cycle(None)
    z, ov = cycle(width)
    assert ov_def == 0 and ov & 0x400, (ov_def, ov)
    zo, spread = coefficient_spread(prob, r, mg)
    err = np.abs(z - zo).max() / np.abs(zo).max()
    bar = max(1e-11, 8.0 * spread)
    print(f"coarsest tiles of {width} columns: rel max err {err:.2e} (bar {bar:.2e})")
    assert np.all(np.isfinite(z)) and err <= bar, (width, err, bar)
    if width == "16":
        assert np.array_equal(z, z_def)

SOLVES = [
    ("general-128x64x16", lambda: W.general_problem(128, 64, 16, 6), 6),
    ("varying-96x40x12", lambda: W.config_problem(4, scale_xy=(96, 40), nz=12), 4),
    ("random-6x10x9", lambda: random_general(6, 10, 9, seed=23), 8),
    ("general-64x32x32", lambda: W.general_problem(64, 32, 32, 6), 6),
]


@pytest.mark.parametrize("pi", [0, 1, 3, 4], ids=["default", "nu2-L3", "cheb-L3", "cheb-L1"])
@pytest.mark.parametrize("label,make,seed", SOLVES, ids=[c[0] for c in SOLVES])
def test_solve_mg_matches_oracle(dev, label, make, seed, pi):
    import torch
    prob = make()
    gp = as_general(prob)
    mg = PARAMS[pi]
    b = W.uniform_field(gp.nx, gp.ny, gp.nz, seed)
    h = mf.pcg_create(prob)
    try:
        mf.pcg_mg_setup(h, **mg)
        bd = to_dev(b, dev)
        xd = torch.zeros_like(bd)
        res = mf.pcg_solve_mg(h, bd, xd, 1e-10, 500)
        torch.cuda.synchronize()
        xg = to_host(xd)
    finally:
        mf.pcg_destroy(h)
    ref = oracle.pcg_mg(gp, b, tol=1e-10, maxit=500, **mg)
    assert res["status"] == ref["status"] == 0, (label, res, ref["status"])
    assert abs(res["iters"] - ref["iters"]) <= 1, (label, res["iters"], ref["iters"])
    rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
    u = np.random.default_rng(4242).uniform(-1.0, 1.0, size=b.shape)
    spread = oracle.pcg_mg(gp, b * (1.0 + 2.0 ** -52 * u), tol=1e-10, maxit=500, **mg)["hist"]
    n = min(len(res["hist"]), len(ref["hist"]), len(spread))
    hg, ho, hs = res["hist"][:n], ref["hist"][:n], spread[:n]
    big = ho >= 1e-6 * ho[0]
    dg = np.max(np.abs(hg[big] - ho[big]) / ho[big])
    ds = np.max(np.abs(hs[big] - ho[big]) / ho[big])
    col = oracle.pcg_gen(gp, b, tol=1e-10, maxit=5000)["iters"]
    print(f"{label} {mg}: iters gpu {res['iters']} oracle {ref['iters']} (column PCG {col}) rel-L2 {rel:.2e} "
          f"history {dg:.2e} (self {ds:.2e})")
    assert rel <= 1e-9, (label, rel)
    assert dg <= max(1e-6, 10 * ds), (label, dg, ds)


def test_mg_setup_rejects_and_requires(dev):
    import torch
    prob = W.config_problem(1, scale_xy=(8, 8), nz=4)
    h = mf.pcg_create(prob)
    try:
        bd = to_dev(np.ones((8, 4, 8)), dev)
        xd = torch.zeros_like(bd)
        with pytest.raises(mf.PcgError):
            mf.pcg_solve_mg(h, bd, xd, 1e-8, 10, workspace=torch.empty(1 << 20, dtype=torch.uint8, device=dev))
        for bad in (dict(nu=0), dict(omega=0.0), dict(omega=1.5), dict(max_levels=-1), dict(coarse_sweeps=0),
                    dict(coarse_lo=-0.1), dict(coarse_lo=2.0), dict(coarse_lo=float("nan"))):
            with pytest.raises(mf.PcgError) as e:
                mf.pcg_mg_setup(h, **bad)
            assert e.value.code == mf.PCG_ERR_INVALID
        mf.pcg_mg_setup(h, max_levels=2)
        assert mf.pcg_mg_num_levels(h) == 2
        mf.pcg_mg_setup(h)
        assert mf.pcg_mg_num_levels(h) == 4
        with pytest.raises(mf.PcgError):
            mf.pcg_mg_level(h, 4)
    finally:
        mf.pcg_destroy(h)


@pytest.mark.parametrize("cfg", [4, 6])
def test_mg_full_size(dev, cfg):
    """The 1024 x 1024 x 128 workloads: B symmetric and positive on random
    vectors, and the solve converges (true residual within 10 tol)."""
    import torch
    wl = W.make_workload(cfg)
    prob = wl.problem
    n = prob.n
    h = mf.pcg_create(prob)
    try:
        mf.pcg_mg_setup(h)
        g = torch.Generator(device=dev).manual_seed(7)
        u = torch.randn(n, dtype=torch.float64, device=dev, generator=g)
        v = torch.randn(n, dtype=torch.float64, device=dev, generator=g)
        Bu, Bv = torch.empty_like(u), torch.empty_like(v)
        ws = torch.empty(mf.pcg_mg_workspace_bytes(h, 0), dtype=torch.uint8, device=dev)
        mf.pcg_mg_vcycle(h, u, Bu, ws)
        mf.pcg_mg_vcycle(h, v, Bv, ws)
        a, b_ = float(torch.dot(Bu, v)), float(torch.dot(u, Bv))
        uBu = float(torch.dot(u, Bu))
        assert abs(a - b_) <= 1e-10 * (float(Bu.norm()) * float(v.norm())), (a, b_)
        assert uBu > 0.0
        del u, v, Bu, Bv, ws
        bd = to_dev(wl.rhs, dev).reshape(-1)
        xd = torch.zeros_like(bd)
        res = mf.pcg_solve_mg(h, bd, xd, wl.tol, 300)
        y = torch.empty_like(xd)
        mf.pcg_apply_A(h, xd, y)
        true_rel = float((bd - y).norm() / bd.norm())
        torch.cuda.synchronize()
    finally:
        mf.pcg_destroy(h)
    print(f"cfg {cfg}: {res['iters']} steps, final {res['final_rel_res']:.2e}, true {true_rel:.2e}")
    assert res["status"] == 0 and res["iters"] <= 150, res
    assert true_rel <= 10 * wl.tol, true_rel


def test_mg_solve_edge_cases(dev):
    """b = 0, maxit = 0, a warm start from a seeded x0, tol = 0 (fixed steps)
    and bitwise determinism of two runs."""
    import torch
    prob = W.config_problem(4, scale_xy=(64, 32), nz=16)
    gp = as_general(prob)
    b = W.uniform_field(64, 32, 16, 44)
    h = mf.pcg_create(prob)
    try:
        mf.pcg_mg_setup(h)
        bd = to_dev(b, dev)
        x = torch.zeros_like(bd)
        res = mf.pcg_solve_mg(h, torch.zeros_like(bd), x, 1e-10, 100)
        assert res["status"] == mf.PCG_OK and res["iters"] == 0 and float(x.abs().max()) == 0.0
        res = mf.pcg_solve_mg(h, bd, x, 1e-10, 0)
        assert res["status"] == mf.PCG_NOT_CONVERGED and res["iters"] == 0 and len(res["hist"]) == 1
        x0 = W.uniform_field(64, 32, 16, 45)
        x = to_dev(x0, dev)
        warm = mf.pcg_solve_mg(h, bd, x, 1e-10, 200)
        assert warm["status"] == mf.PCG_OK
        x1 = x.clone()
        xa, xb = torch.zeros_like(bd), torch.zeros_like(bd)
        ra = mf.pcg_solve_mg(h, bd, xa, 0.0, 7)
        rb = mf.pcg_solve_mg(h, bd, xb, 0.0, 7)
        torch.cuda.synchronize()
        assert ra["status"] == rb["status"] == mf.PCG_NOT_CONVERGED and ra["iters"] == 7
        assert torch.equal(xa, xb) and np.array_equal(ra["hist"], rb["hist"])
        xg7, x1h = to_host(xa), to_host(x1)
    finally:
        mf.pcg_destroy(h)
    # seven fixed steps against the oracle's, with the bounds of the solve
    # comparisons: x within rel-L2 1e-9, the history within max(1e-6, 10x the
    # oracle's spread under an ulp-level perturbation of b).  A cycle's
    # rounding is not that of a perturbed b: the residual t = f - A z cancels
    # terms ~1e4 times larger than itself and the coarse columns are far
    # worse conditioned than the fine ones, so two correct cycles differ by
    # up to a few 1e-10 relative (measured 4.6e-10 in x after 7 steps, 7.6e-8
    # in the 7th residual norm, while the perturbed-b spread is 2e-16)
    ref = oracle.pcg_mg(gp, b, tol=0.0, maxit=7)
    u = np.random.default_rng(4242).uniform(-1.0, 1.0, size=b.shape)
    sp = oracle.pcg_mg(gp, b * (1.0 + 2.0 ** -52 * u), tol=0.0, maxit=7)
    nx_ = np.linalg.norm(ref["x"])
    dx, sx = np.linalg.norm(xg7 - ref["x"]) / nx_, np.linalg.norm(sp["x"] - ref["x"]) / nx_
    dh = np.max(np.abs(ra["hist"] - ref["hist"]) / ref["hist"])
    sh = np.max(np.abs(sp["hist"] - ref["hist"]) / ref["hist"])
    print(f"7 steps: x {dx:.2e} (oracle spread {sx:.2e}), history {dh:.2e} (spread {sh:.2e})")
    assert dx <= max(1e-9, 10 * sx), (dx, sx)
    assert dh <= max(1e-6, 10 * sh), (dh, sh)
    full = oracle.pcg_mg(gp, b, x0=x0, tol=1e-10, maxit=200)
    assert abs(warm["iters"] - full["iters"]) <= 1, (warm["iters"], full["iters"])
    assert np.linalg.norm(x1h - full["x"]) <= 1e-9 * np.linalg.norm(full["x"])
