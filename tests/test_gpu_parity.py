"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle on
the same seeded inputs, at sizes the oracle finishes in seconds.  Grids are
chosen to span several 64-column tiles with a ragged tail, 1 to 16 column
segments, and the degenerate 1- and 2-cell directions."""
import math

import numpy as np
import pytest

import matrix_free_pcg_amd as mf
import oracle
from gpu_helpers import apply_tol, gen_scale, precond_tol, require_gpu, to_dev, to_host
from matrix_free_pcg_amd import workloads as W

pytestmark = pytest.mark.gpu

# (label, problem factory); the problems exercise constant and varying alpha_h,
# constant and graded alpha_z, and every segment length (nz -> L = 4, 8, 16, 32)
GRIDS = [
    ("cfg1-32x32x16", lambda: W.config_problem(1)),
    ("cfg2-128x128x64", lambda: W.config_problem(2)),
    ("cfg4-70x45x40", lambda: W.config_problem(4, scale_xy=(70, 45), nz=40)),
    ("cfg4-129x3x128", lambda: W.config_problem(4, scale_xy=(129, 3), nz=128)),
    ("cfg4-65x4x130", lambda: W.config_problem(4, scale_xy=(65, 4), nz=130)),
    ("cfg4-5x3x300", lambda: W.config_problem(4, scale_xy=(5, 3), nz=300)),
    ("cfg3-1x1x7", lambda: W.config_problem(3, scale_xy=(1, 1), nz=7)),
    ("cfg4-2x2x1", lambda: W.config_problem(4, scale_xy=(2, 2), nz=1)),
    ("cfg2-3x1x2", lambda: W.config_problem(2, scale_xy=(3, 1), nz=2)),
    ("cfg4-64x2x33", lambda: W.config_problem(4, scale_xy=(64, 2), nz=33)),
    # whole tiles (nx a multiple of 64, nz of the segment length): the
    # straight-line kernels, with 8, 1, 16 and 16 segments of 16, 8, 16, 32
    # levels (the first over the multiplier table of 8-level segments)
    ("cfg4-128x3x128", lambda: W.config_problem(4, scale_xy=(128, 3), nz=128)),
    ("cfg4-64x1x8", lambda: W.config_problem(4, scale_xy=(64, 1), nz=8)),
    ("cfg2-192x2x256", lambda: W.config_problem(2, scale_xy=(192, 2), nz=256)),
    ("cfg4-64x2x512", lambda: W.config_problem(4, scale_xy=(64, 2), nz=512)),
]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("label,make", GRIDS, ids=[g[0] for g in GRIDS])
def test_apply_A_matches_oracle(dev, label, make):
    import torch
    prob = make()
    x = W.uniform_field(prob.nx, prob.ny, prob.nz, 101)
    h = mf.pcg_create(prob)
    try:
        xd = to_dev(x, dev)
        yd = torch.full_like(xd, float("nan"))
        mf.pcg_apply_A(h, xd, yd)
        torch.cuda.synchronize()
    finally:
        mf.pcg_destroy(h)
    y = to_host(yd)
    ref = oracle.apply_A(prob, x)
    err = np.abs(y - ref).max()
    assert np.isfinite(y).all()
    assert err <= apply_tol(prob, x), (label, err, apply_tol(prob, x))


@pytest.mark.parametrize("label,make", GRIDS, ids=[g[0] for g in GRIDS])
def test_precond_matches_oracle(dev, label, make):
    import torch
    prob = make()
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 202)
    h = mf.pcg_create(prob)
    try:
        rd = to_dev(r, dev)
        zd = torch.full_like(rd, float("nan"))
        mf.pcg_precond(h, rd, zd)
        torch.cuda.synchronize()
    finally:
        mf.pcg_destroy(h)
    z = to_host(zd)
    ref = oracle.precond(prob, r)
    err = np.abs(z - ref).max()
    assert np.isfinite(z).all()
    assert err <= precond_tol(prob, ref), (label, err, precond_tol(prob, ref))
    assert np.array_equal(to_host(rd), r)   # input untouched


SOLVERS = {"interleaved": mf.pcg_solve, "no_q": mf.pcg_solve_no_q,
           "standard": mf.pcg_solve_standard}
VARIANTS = list(SOLVERS)


def _solve_both(prob, b, tol, maxit, dev, variant="interleaved", x0=None):
    import torch
    h = mf.pcg_create(prob)
    try:
        bd = to_dev(b, dev)
        xd = to_dev(np.zeros_like(b) if x0 is None else x0, dev)
        res = SOLVERS[variant](h, bd, xd, tol, maxit)
        torch.cuda.synchronize()
        xg = to_host(xd)
    finally:
        mf.pcg_destroy(h)
    ref = oracle.pcg(prob, b, x0=x0, tol=tol, maxit=maxit)
    return res, xg, ref


def _check_solution(label, res, xg, ref, spread, drift=None):
    """Iterations within +-1 and final iterates within rel-L2 1e-9.

    drift=(prob, b): for an ill-conditioned case where two correct float64
    runs can end further apart than 1e-9, the bar is instead that the GPU
    iterate is as close to the converged solution x* (oracle, tol 1e-14) as
    the oracle's own iterate is (within a factor 2) -- i.e. the difference is
    rounding amplified by the conditioning, not an error.  Both distances are
    printed."""
    assert res["status"] == ref["status"] == 0, (label, res, ref["status"])
    assert abs(res["iters"] - ref["iters"]) <= 1, (label, res["iters"], ref["iters"])
    rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
    if drift is not None and rel > 1e-9:
        prob, b = drift
        xs = oracle.pcg(prob, b, tol=1e-14, maxit=20000)["x"]
        ns = np.linalg.norm(xs)
        e_gpu = np.linalg.norm(xg - xs) / ns
        e_orc = np.linalg.norm(ref["x"] - xs) / ns
        print(f"{label}: gpu-oracle {rel:.2e}; to x*: gpu {e_gpu:.2e} oracle {e_orc:.2e}")
        assert e_gpu <= 2.0 * max(e_orc, 1e-9), (label, rel, e_gpu, e_orc)
    else:
        assert rel <= 1e-9, (label, rel)
    check_histories(label, res["hist"], ref["hist"], res["iters"], spread)
    return rel


def oracle_spread(prob, b, tol, maxit, x0=None):
    """The oracle's own rounding-level sensitivity: its residual history for
    b perturbed by one ulp-scale relative amount, b*(1 + 2^-52 u), u ~ U[-1,1]."""
    u = np.random.default_rng(4242).uniform(-1.0, 1.0, size=b.shape)
    return oracle.pcg(prob, b * (1.0 + 2.0 ** -52 * u), x0=x0, tol=tol, maxit=maxit)["hist"]


def check_histories(label, hg_all, ho_all, iters, spread, factor=10.0):
    """Residual histories agree while the residual is well above the stopping
    tolerance: for every step with |r_k| >= 1e-6 |r_0|, the relative deviation
    is at most max(1e-6, factor x the oracle's own deviation when b is
    perturbed at the rounding level).  Closer to the tolerance the residual is
    made of the components most sensitive to rounding and two correct float64
    runs can differ by tens of percent there, so the tail is not compared step
    by step (the iteration counts and final iterates are)."""
    assert len(hg_all) == iters + 1
    n = min(len(hg_all), len(ho_all), len(spread))
    hg, ho, hs = hg_all[:n], ho_all[:n], spread[:n]
    h0 = ho[0]
    assert abs(hg[0] - h0) <= 1e-12 * h0
    big = ho >= 1e-6 * h0
    rel = np.max(np.abs(hg[big] - ho[big]) / ho[big])
    rel_self = np.max(np.abs(hs[big] - ho[big]) / ho[big])
    tail = np.max(np.abs(hg - ho) / ho)
    print(f"{label}: history rel dev {rel:.2e} while |r|>1e-6|r0| (oracle self {rel_self:.2e}); "
          f"max over all steps {tail:.2e}")
    assert rel <= max(1e-6, factor * rel_self), (label, rel, rel_self)


# (label, workload factory, compare-to-x* allowed): only the manufactured
# case (alpha_z/alpha_h = 1e4, delta = 1e-3, |b| ~ 1e3 |x|) is ill-conditioned
# enough for run-to-run rounding to exceed 1e-9 in x.
SOLVE_CASES = [
    ("cfg1", lambda: W.make_workload(1), False),
    ("cfg2", lambda: W.make_workload(2), False),
    ("cfg3-64x48x32", lambda: W.make_workload(3, scale_xy=(64, 48), nz=32), True),
    ("cfg4-70x45x40", lambda: W.make_workload(4, scale_xy=(70, 45), nz=40), False),
    ("cfg4-130x20x128", lambda: W.make_workload(4, scale_xy=(130, 20), nz=128), False),
    ("cfg4-128x24x64", lambda: W.make_workload(4, scale_xy=(128, 24), nz=64), False),
]


def _rhs(w):
    if w.rhs is not None:
        return w.rhs
    return oracle.apply_A(w.problem, w.x_true)   # oracle side builds its b; the same b is given to both


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("label,make,drift", SOLVE_CASES, ids=[c[0] for c in SOLVE_CASES])
def test_solve_matches_oracle(dev, label, make, drift, variant):
    w = make()
    b = _rhs(w)
    res, xg, ref = _solve_both(w.problem, b, w.tol, w.maxit, dev, variant)
    spread = oracle_spread(w.problem, b, w.tol, w.maxit)
    rel = _check_solution(label, res, xg, ref, spread, drift=(w.problem, b) if drift else None)
    print(f"{label} {variant}: iters gpu={res['iters']} oracle={ref['iters']} rel-L2={rel:.2e}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("steps", [0, 1, 2, 3, 4, 5, 7, 8])
def test_first_steps_match_oracle(dev, steps, variant):
    """Fixed step counts (tol = 0): iterate and history after k steps, tight.
    The interleaved loop applies the x updates every fourth step, so these
    counts stop it with 1, 2, 3 and 4 updates pending."""
    w = W.make_workload(4, scale_xy=(70, 45), nz=40)
    res, xg, ref = _solve_both(w.problem, w.rhs, 0.0, steps, dev, variant)
    assert res["status"] == ref["status"] == 1
    assert res["iters"] == ref["iters"] == steps
    assert np.allclose(res["hist"], ref["hist"], rtol=1e-11, atol=0)
    if steps == 0:
        assert np.array_equal(xg, np.zeros_like(xg))
    else:
        rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
        assert rel <= 1e-11, rel


def test_warm_start_matches_oracle(dev):
    w = W.make_workload(4, scale_xy=(70, 45), nz=40)
    x0 = W.uniform_field(70, 45, 40, 77)
    res, xg, ref = _solve_both(w.problem, w.rhs, w.tol, w.maxit, dev, x0=x0)
    _check_solution("warm", res, xg, ref, oracle_spread(w.problem, w.rhs, w.tol, w.maxit, x0=x0))


def test_solve_is_deterministic(dev):
    import torch
    w = W.make_workload(4, scale_xy=(130, 20), nz=128)
    h = mf.pcg_create(w.problem)
    try:
        outs = []
        for _ in range(2):
            bd = to_dev(w.rhs, dev)
            xd = torch.zeros_like(bd)
            res = mf.pcg_solve(h, bd, xd, w.tol, w.maxit)
            torch.cuda.synchronize()
            outs.append((to_host(xd), res["hist"], res["iters"]))
    finally:
        mf.pcg_destroy(h)
    assert outs[0][2] == outs[1][2]
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][0], outs[1][0])


@pytest.mark.parametrize("variant", VARIANTS)
def test_edge_cases(dev, variant):
    import torch
    w = W.make_workload(4, scale_xy=(33, 5), nz=9)
    prob = w.problem
    fn = SOLVERS[variant]
    h = mf.pcg_create(prob)
    try:
        # r0 = 0: no steps, x = x0, converged
        bd = torch.zeros(prob.ny, prob.nz, prob.nx, dtype=torch.float64, device=dev)
        xd = torch.zeros_like(bd)
        res = fn(h, bd, xd, 1e-10, 50)
        assert res["status"] == mf.PCG_OK and res["iters"] == 0
        assert torch.count_nonzero(xd).item() == 0
        # maxit = 0: no steps, not converged, history [||r0||]
        bd = to_dev(w.rhs, dev)
        xd = torch.zeros_like(bd)
        res = fn(h, bd, xd, 1e-10, 0)
        assert res["status"] == mf.PCG_NOT_CONVERGED and res["iters"] == 0
        assert len(res["hist"]) == 1 and abs(res["hist"][0] - np.linalg.norm(w.rhs)) <= 1e-12 * np.linalg.norm(w.rhs)
        assert torch.count_nonzero(xd).item() == 0
        # NaN in b: breakdown
        bad = w.rhs.copy()
        bad[2, 3, 4] = np.nan
        res = fn(h, to_dev(bad, dev), torch.zeros_like(bd), 1e-10, 50)
        assert res["status"] == mf.PCG_ERR_BREAKDOWN
        # invalid: workspace too small, x aliasing b, wrong dtype
        ws = torch.empty(16, dtype=torch.uint8, device=dev)
        with pytest.raises(ValueError):
            fn(h, bd, xd, 1e-10, 50, workspace=ws)
        with pytest.raises(mf.PcgError):
            fn(h, bd, bd, 1e-10, 50)
        with pytest.raises(TypeError):
            fn(h, bd.float(), xd, 1e-10, 50)
        with pytest.raises(mf.PcgError):
            fn(h, bd, xd, float("nan"), 50)
    finally:
        mf.pcg_destroy(h)


def test_converges_in_one_step_when_M_equals_A(dev):
    """alpha_h = 0 makes M = A (pin K3 of the oracle), on the GPU path."""
    prob = W.Problem(70, 6, 33, 1.0, W.graded_faces(33, 10.0, 1.0), 0.0)
    b = W.uniform_field(70, 6, 33, 5)
    res, xg, ref = _solve_both(prob, b, 1e-10, 20, dev)
    assert res["status"] == 0 and res["iters"] == 1 and ref["iters"] == 1
    assert np.linalg.norm(xg - ref["x"]) <= 1e-12 * np.linalg.norm(ref["x"])


def test_profile_counts_launches(dev):
    import torch
    w = W.make_workload(4, scale_xy=(70, 45), nz=40)
    h = mf.pcg_create(w.problem)
    try:
        mf.pcg_profile_enable(h, True)
        bd = to_dev(w.rhs, dev)
        xd = torch.zeros_like(bd)
        res = mf.pcg_solve(h, bd, xd, 0.0, 7)
        ms_p, n_p = mf.pcg_profile_read(h, mf.PCG_KID_FUSED_PREC)
        ms_s, n_s = mf.pcg_profile_read(h, mf.PCG_KID_FUSED_SPMV)
        assert res["iters"] == 7
        assert n_p == 8 and n_s == 7     # the last stencil pass (launched before the stop test was read) is not counted
        assert ms_p > 0 and ms_s > 0 and math.isfinite(ms_p + ms_s)
        mf.pcg_profile_reset(h)
        assert mf.pcg_profile_read(h, mf.PCG_KID_FUSED_PREC) == (0.0, 0)
        # sampled: the passes of steps k with k mod 8 < 4 only (k = 0..3, 8..11;
        # the stencil pass of the last step, k = 11, is not counted)
        mf.pcg_profile_enable(h, 8)
        xd.zero_()
        res = mf.pcg_solve(h, bd, xd, 0.0, 11)
        _, n_p = mf.pcg_profile_read(h, mf.PCG_KID_FUSED_PREC)
        _, n_s = mf.pcg_profile_read(h, mf.PCG_KID_FUSED_SPMV)
        assert (n_p, n_s) == (8, 7), (n_p, n_s)
        with pytest.raises(mf.PcgError):
            mf.pcg_profile_enable(h, -1)
    finally:
        mf.pcg_destroy(h)


def test_whole_tile_kernels_match_generic(dev, monkeypatch):
    """On a grid of whole tiles the straight-line kernels run by default; with
    MFPCG_COL_FULL=0 / MFPCG_ST_FULL=0 (read at pcg_create) the guarded ones do.
    Both compute the same elimination and stencil: apply_A, precond and 5 CG
    steps of each variant agree to rounding."""
    import torch
    w = W.make_workload(4, scale_xy=(128, 6), nz=64)
    prob = w.problem
    x = W.uniform_field(prob.nx, prob.ny, prob.nz, 11)

    def run(full):
        monkeypatch.setenv("MFPCG_COL_FULL", "1" if full else "0")
        monkeypatch.setenv("MFPCG_ST_FULL", "1" if full else "0")
        h = mf.pcg_create(prob)
        try:
            xd = to_dev(x, dev)
            y, z = torch.empty_like(xd), torch.empty_like(xd)
            mf.pcg_apply_A(h, xd, y)
            mf.pcg_precond(h, xd, z)
            out = {"y": to_host(y), "z": to_host(z)}
            for name, fn in SOLVERS.items():
                bd = to_dev(w.rhs, dev)
                xs = torch.zeros_like(bd)
                res = fn(h, bd, xs, 0.0, 5)
                out[name] = (to_host(xs), res["hist"])
            torch.cuda.synchronize()
            return out
        finally:
            mf.pcg_destroy(h)

    a, b = run(True), run(False)
    assert np.abs(a["y"] - b["y"]).max() <= apply_tol(prob, x)
    assert np.abs(a["z"] - b["z"]).max() <= precond_tol(prob, b["z"])
    for name in SOLVERS:
        xa, ha = a[name]
        xb, hb = b[name]
        assert np.allclose(ha, hb, rtol=1e-12, atol=0), name
        assert np.linalg.norm(xa - xb) <= 1e-12 * np.linalg.norm(xb), name


# (label, problem, segment lengths compared): nz = 64 and 128 take 16-level
# segments over the 8-level table by default; 40 keeps 8 by default (whole
# segments) and is forced to 16 (a ragged last segment); 200 and 130 have
# 16-level tables and are forced to 32
SEGMENT_CASES = [
    ("cfg4-128x6x64", lambda: W.config_problem(4, scale_xy=(128, 6), nz=64), 8, 16),
    ("cfg4-64x4x128", lambda: W.config_problem(4, scale_xy=(64, 4), nz=128), 8, 16),
    ("cfg4-70x5x40", lambda: W.config_problem(4, scale_xy=(70, 5), nz=40), 8, 16),
    ("cfg4-64x3x200", lambda: W.config_problem(4, scale_xy=(64, 3), nz=200), 16, 32),
    ("cfg4-65x4x130", lambda: W.config_problem(4, scale_xy=(65, 4), nz=130), 16, 32),
]


@pytest.mark.parametrize("label,make,short,long_", SEGMENT_CASES, ids=[c[0] for c in SEGMENT_CASES])
def test_column_segment_lengths_agree(dev, monkeypatch, label, make, short, long_):
    """MFPCG_COL_LF (read at pcg_create) sets the segment length of the column
    passes that use no stored matrix; longer segments start at every
    (long/short)-th boundary of the multiplier table computed for the short
    ones.  Same elimination either way: precond matches the oracle and the
    first 5 steps of each solve agree to rounding."""
    import torch
    prob = make()
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 31)
    b = W.uniform_field(prob.nx, prob.ny, prob.nz, 32)
    ref = oracle.precond(prob, r)

    def run(lf):
        monkeypatch.setenv("MFPCG_COL_LF", str(lf))
        h = mf.pcg_create(prob)
        try:
            rd = to_dev(r, dev)
            zd = torch.full_like(rd, float("nan"))
            mf.pcg_precond(h, rd, zd)
            out = {"z": to_host(zd)}
            for name, fn in SOLVERS.items():
                bd = to_dev(b, dev)
                xs = torch.zeros_like(bd)
                res = fn(h, bd, xs, 0.0, 5)
                out[name] = (to_host(xs), res["hist"])
            torch.cuda.synchronize()
            return out
        finally:
            mf.pcg_destroy(h)

    a, c = run(short), run(long_)
    for o in (a, c):
        assert np.abs(o["z"] - ref).max() <= precond_tol(prob, ref), label
    for name in SOLVERS:
        xa, ha = a[name]
        xc, hc = c[name]
        assert np.allclose(ha, hc, rtol=1e-11, atol=0), (label, name)
        assert np.linalg.norm(xa - xc) <= 1e-11 * np.linalg.norm(xa), (label, name)



# (columns per column-pass workgroup, segment length): the generic column
# kernel at every shape its tuning variables allow on these grids
COLUMN_SHAPES = [(32, 8), (64, 4), (32, 4), (32, 16)]
COLUMN_SHAPE_GRIDS = [
    ("cfg4-70x45x40", lambda: W.config_problem(4, scale_xy=(70, 45), nz=40)),
    ("cfg4-128x24x64", lambda: W.config_problem(4, scale_xy=(128, 24), nz=64)),
    ("cfg4-33x5x7", lambda: W.config_problem(4, scale_xy=(33, 5), nz=7)),
]


@pytest.mark.parametrize("shape", COLUMN_SHAPES, ids=[f"C{c}-L{l}" for c, l in COLUMN_SHAPES])
@pytest.mark.parametrize("label,make", COLUMN_SHAPE_GRIDS, ids=[g[0] for g in COLUMN_SHAPE_GRIDS])
def test_column_tile_shapes(dev, monkeypatch, label, make, shape):
    """MFPCG_COL_C (32 or 64 columns per workgroup) and MFPCG_COL_L (4, 8,
    16 or 32 levels per segment), read at pcg_create, choose the generic
    column kernel's shape (every pass on 32-column tiles, and ragged ones,
    runs it): precond matches the oracle within the column-solve bound, and
    5 steps of each solve agree with the default shape's to rounding."""
    import torch
    cols, seg = shape
    prob = make()
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 41)
    b = W.uniform_field(prob.nx, prob.ny, prob.nz, 42)
    ref = oracle.precond(prob, r)

    def run(env):
        for k in ("MFPCG_COL_C", "MFPCG_COL_L", "MFPCG_COL_LF"):
            monkeypatch.delenv(k, raising=False)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        h = mf.pcg_create(prob)
        try:
            ov = mf.pcg_tuning_overrides(h)
            rd = to_dev(r, dev)
            zd = torch.full_like(rd, float("nan"))
            mf.pcg_precond(h, rd, zd)
            out = {"z": to_host(zd), "ov": ov}
            for name, fn in SOLVERS.items():
                bd = to_dev(b, dev)
                xs = torch.zeros_like(bd)
                res = fn(h, bd, xs, 0.0, 5)
                out[name] = (to_host(xs), res["hist"])
            torch.cuda.synchronize()
            return out
        finally:
            mf.pcg_destroy(h)
            for k in ("MFPCG_COL_C", "MFPCG_COL_L", "MFPCG_COL_LF"):
                monkeypatch.delenv(k, raising=False)

    d = run({})
    a = run({"MFPCG_COL_C": str(cols), "MFPCG_COL_L": str(seg), "MFPCG_COL_LF": str(seg)})
    assert d["ov"] == 0 and a["ov"] & 0x7 == 0x7, (d["ov"], a["ov"])
    err = np.abs(a["z"] - ref).max()
    print(f"{label} C={cols} L={seg}: precond max err {err:.2e} (bound {precond_tol(prob, ref):.2e})")
    assert err <= precond_tol(prob, ref), (label, shape, err)
    for name in SOLVERS:
        xa, ha = a[name]
        xd, hd = d[name]
        assert np.allclose(ha, hd, rtol=1e-11, atol=0), (label, shape, name)
        assert np.linalg.norm(xa - xd) <= 1e-11 * np.linalg.norm(xd), (label, shape, name)

# grids of whole tiles: ny a multiple of 8 (row tiles of 4 or 8 rows in every
# stencil pass), ny = 6 (in the operator-only passes only), a general operator
ROW_TILE_CASES = [
    ("cfg4-128x24x64", lambda: W.config_problem(4, scale_xy=(128, 24), nz=64)),
    ("cfg4-64x6x32", lambda: W.config_problem(4, scale_xy=(64, 6), nz=32)),
    ("general-64x8x48", lambda: W.general_problem(64, 8, 48, 6)),
]


@pytest.mark.parametrize("label,make", ROW_TILE_CASES, ids=[c[0] for c in ROW_TILE_CASES])
def test_row_tiles_match_one_row_tiles(dev, monkeypatch, label, make):
    """On whole tiles the stencil passes take tiles of several rows j whose
    waves pass z through LDS (default; MFPCG_ST_JT=4 or 8 rows for the fused
    passes, read at pcg_create); MFPCG_ST_JT=1 takes one-row tiles.  Same
    stencil: apply_A matches the oracle every way and the first 5 steps of
    every solve agree to rounding (the dot products' per-tile partial sums
    group differently)."""
    import torch
    prob = make()
    general = isinstance(prob, W.GeneralProblem)
    x = W.uniform_field(prob.nx, prob.ny, prob.nz, 41)
    b = W.uniform_field(prob.nx, prob.ny, prob.nz, 42)
    ref = oracle.apply_A_gen(prob, x) if general else oracle.apply_A(prob, x)

    def run(jt):
        monkeypatch.setenv("MFPCG_ST_JT", str(jt))
        h = mf.pcg_create(prob)
        try:
            xd = to_dev(x, dev)
            yd = torch.full_like(xd, float("nan"))
            mf.pcg_apply_A(h, xd, yd)
            out = {"y": to_host(yd)}
            for name, fn in SOLVERS.items():
                bd = to_dev(b, dev)
                xs = torch.zeros_like(bd)
                res = fn(h, bd, xs, 0.0, 5)
                out[name] = (to_host(xs), res["hist"])
            torch.cuda.synchronize()
            return out
        finally:
            mf.pcg_destroy(h)

    a, c, e = run(4), run(1), run(8)
    for o in (a, c, e):
        assert np.isfinite(o["y"]).all()
    if general:
        tol = 16 * np.finfo(float).eps * gen_scale(prob, x)
    else:
        tol = apply_tol(prob, x)
    for o in (a, c, e):
        assert np.abs(o["y"] - ref).max() <= tol, label
    for name in SOLVERS:
        xc, hc = c[name]
        for o in (a, e):
            xa, ha = o[name]
            assert np.allclose(ha, hc, rtol=1e-11, atol=0), (label, name)
            assert np.linalg.norm(xa - xc) <= 1e-11 * np.linalg.norm(xc), (label, name)


def _random_shapes(count=24, seed=20261202):
    """Seeded grid shapes that mix whole and ragged tiles in every direction:
    nx a multiple of 64 or not, ny a multiple of 8, 4, 2 or odd, nz a multiple
    of 16 or not (1..200)."""
    rng = np.random.default_rng(seed)
    shapes = []
    for n in range(count):
        nx = int(rng.choice([64, 128, 192])) if n % 2 == 0 else int(rng.integers(1, 150))
        ny = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        nz = int(rng.choice([16, 32, 48, 64, 128])) if n % 3 != 2 else int(rng.integers(1, 200))
        shapes.append((nx, ny, nz))
    return shapes


@pytest.mark.parametrize("nx,ny,nz", _random_shapes(), ids=lambda v: str(v))
def test_random_shapes_match_oracle(dev, nx, ny, nz):
    """apply_A, precond and the first 3 steps of the interleaved and the
    standard solve against the oracle on seeded grid shapes (the launch
    geometry the library picks for each: row tiles, 16-level segments, ragged
    tiles)."""
    import torch
    prob = W.config_problem(4, scale_xy=(nx, ny), nz=nz)
    x = W.uniform_field(nx, ny, nz, 51)
    r = W.gaussian_field(nx, ny, nz, 52)
    b = W.uniform_field(nx, ny, nz, 53)
    h = mf.pcg_create(prob)
    try:
        xd, rd = to_dev(x, dev), to_dev(r, dev)
        yd, zd = torch.full_like(xd, float("nan")), torch.full_like(xd, float("nan"))
        mf.pcg_apply_A(h, xd, yd)
        mf.pcg_precond(h, rd, zd)
        y, z = to_host(yd), to_host(zd)
        runs = {}
        for name in ("interleaved", "standard"):
            bd = to_dev(b, dev)
            xs = torch.zeros_like(bd)
            res = SOLVERS[name](h, bd, xs, 0.0, 3)
            runs[name] = (to_host(xs), res)
        torch.cuda.synchronize()
    finally:
        mf.pcg_destroy(h)
    assert np.abs(y - oracle.apply_A(prob, x)).max() <= apply_tol(prob, x)
    zo = oracle.precond(prob, r)
    assert np.abs(z - zo).max() <= precond_tol(prob, zo)
    ref = oracle.pcg(prob, b, tol=0.0, maxit=3)
    for name, (xg, res) in runs.items():
        assert res["iters"] == ref["iters"] == 3, name
        assert np.allclose(res["hist"], ref["hist"], rtol=1e-11, atol=0), name
        assert np.linalg.norm(xg - ref["x"]) <= 1e-11 * np.linalg.norm(ref["x"]), name
