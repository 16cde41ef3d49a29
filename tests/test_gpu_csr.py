"""GPU parity of the explicit comparison path (CSR matrix + stored column
matrices + standard PCG) against the CPU oracle.

The expected CSR structure is read off the oracle's dense operator (the
oracle stencil applied to unit vectors): row pointers and column indices must
match exactly, values to rounding."""
import numpy as np
import pytest

import matrix_free_pcg_amd as mf
import oracle
from gpu_helpers import EPS, apply_tol, precond_tol, require_gpu, to_dev, to_host
from matrix_free_pcg_amd import workloads as W
from oracle_pins import dense_from_apply, varying_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


SMALL = [(5, 4, 6), (1, 3, 4), (2, 2, 3), (3, 1, 1), (7, 2, 2), (4, 5, 1)]


@pytest.mark.parametrize("nx,ny,nz", SMALL)
def test_csr_structure_matches_dense_operator(dev, nx, ny, nz):
    import torch
    prob = varying_problem(nx, ny, nz, delta=0.07, seed=nx * 10 + ny, az_scale=30.0)
    A = dense_from_apply(oracle.default(), prob)
    h = mf.pcg_create(prob)
    try:
        C = mf.pcg_csr_assemble(h)
        torch.cuda.synchronize()
        rp, col, val = to_host(C.row_ptr), to_host(C.col), to_host(C.val)
    finally:
        mf.pcg_destroy(h)
    n = prob.n
    exp_rp = [0]
    exp_col, exp_val = [], []
    for l in range(n):
        nzc = np.nonzero(A[l])[0]
        exp_col.extend(nzc.tolist())
        exp_val.extend(A[l, nzc].tolist())
        exp_rp.append(len(exp_col))
    assert rp.dtype == np.int64 and col.dtype == np.int32
    assert np.array_equal(rp, np.array(exp_rp)), (rp, exp_rp)
    assert np.array_equal(col, np.array(exp_col, dtype=np.int32))
    scale = np.abs(A).max()
    assert np.abs(val - np.array(exp_val)).max() <= 8 * EPS * scale


CASES = [
    ("cfg1-32x32x16", lambda: W.config_problem(1)),
    ("cfg4-70x45x40", lambda: W.config_problem(4, scale_xy=(70, 45), nz=40)),
    ("cfg4-129x3x128", lambda: W.config_problem(4, scale_xy=(129, 3), nz=128)),
    ("cfg2-3x1x2", lambda: W.config_problem(2, scale_xy=(3, 1), nz=2)),
]


@pytest.mark.parametrize("label,make", CASES, ids=[c[0] for c in CASES])
def test_csr_spmv_and_stored_precond_match_oracle(dev, label, make):
    import torch
    prob = make()
    x = W.uniform_field(prob.nx, prob.ny, prob.nz, 303)
    r = W.gaussian_field(prob.nx, prob.ny, prob.nz, 304)
    h = mf.pcg_create(prob)
    try:
        C = mf.pcg_csr_assemble(h)
        tri = mf.pcg_tridiag_assemble(h)
        xd, rd = to_dev(x, dev), to_dev(r, dev)
        yd = torch.full_like(xd, float("nan"))
        zd = torch.full_like(xd, float("nan"))
        mf.pcg_csr_spmv(h, C, xd, yd)
        mf.pcg_tridiag_precond(h, tri, rd, zd)
        torch.cuda.synchronize()
        y, z = to_host(yd), to_host(zd)
    finally:
        mf.pcg_destroy(h)
    yref = oracle.apply_A(prob, x)
    zref = oracle.precond(prob, r)
    assert np.abs(y - yref).max() <= apply_tol(prob, x), label
    assert np.abs(z - zref).max() <= precond_tol(prob, zref), label


SOLVES = [
    ("cfg1", lambda: W.make_workload(1)),
    ("cfg4-70x45x40", lambda: W.make_workload(4, scale_xy=(70, 45), nz=40)),
]


@pytest.mark.parametrize("label,make", SOLVES, ids=[c[0] for c in SOLVES])
def test_solve_csr_matches_oracle(dev, label, make):
    import torch
    w = make()
    h = mf.pcg_create(w.problem)
    try:
        C = mf.pcg_csr_assemble(h)
        tri = mf.pcg_tridiag_assemble(h)
        bd = to_dev(w.rhs, dev)
        xd = torch.zeros_like(bd)
        res = mf.pcg_solve_csr(h, C, tri, bd, xd, w.tol, w.maxit)
        torch.cuda.synchronize()
        xg = to_host(xd)
    finally:
        mf.pcg_destroy(h)
    ref = oracle.pcg(w.problem, w.rhs, tol=w.tol, maxit=w.maxit)
    assert res["status"] == ref["status"] == 0
    assert abs(res["iters"] - ref["iters"]) <= 1
    rel = np.linalg.norm(xg - ref["x"]) / np.linalg.norm(ref["x"])
    print(f"{label} csr: iters gpu={res['iters']} oracle={ref['iters']} rel-L2={rel:.2e}")
    assert rel <= 1e-9


def test_csr_fixed_steps_match_oracle(dev):
    import torch
    w = W.make_workload(4, scale_xy=(70, 45), nz=40)
    h = mf.pcg_create(w.problem)
    try:
        C = mf.pcg_csr_assemble(h)
        tri = mf.pcg_tridiag_assemble(h)
        bd = to_dev(w.rhs, dev)
        xd = torch.zeros_like(bd)
        res = mf.pcg_solve_csr(h, C, tri, bd, xd, 0.0, 5)
        torch.cuda.synchronize()
        xg = to_host(xd)
    finally:
        mf.pcg_destroy(h)
    ref = oracle.pcg(w.problem, w.rhs, tol=0.0, maxit=5)
    assert res["iters"] == ref["iters"] == 5
    assert np.allclose(res["hist"], ref["hist"], rtol=1e-11, atol=0)
    assert np.linalg.norm(xg - ref["x"]) <= 1e-11 * np.linalg.norm(ref["x"])


def test_stored_matrices_keep_their_own_factors(dev):
    """The segment-boundary multipliers of stored column matrices live in
    the tri buffer itself: factoring a second, different set of matrices
    leaves the first one's solve unchanged, each solve satisfies its own
    matrices (backward error per row), and a buffer of only the three
    diagonals is refused before any work is queued."""
    import ctypes
    import torch
    from matrix_free_pcg_amd import _abi
    prob = W.config_problem(4, scale_xy=(8, 8), nz=40)
    n = prob.n
    r = W.uniform_field(prob.nx, prob.ny, prob.nz, 77)
    h = mf.pcg_create(prob)
    try:
        tri1 = mf.pcg_tridiag_assemble(h)
        tri2 = tri1.clone()
        tri2[n:2 * n] *= 2.0     # another diagonally dominant set of column matrices
        mf.pcg_tridiag_factor(h, tri2)
        rd = to_dev(r, dev)
        z1 = torch.empty_like(rd)
        z2 = torch.empty_like(rd)
        mf.pcg_tridiag_precond(h, tri1, rd, z1)
        mf.pcg_tridiag_precond(h, tri2, rd, z2)
        short = torch.zeros(3 * n, dtype=torch.float64, device=dev)
        rc = _abi.load().pcg_tridiag_precond(h.ptr, short.data_ptr(), ctypes.c_size_t(3 * n * 8),
                                             rd.data_ptr(), z1.data_ptr())
        assert rc == mf.PCG_ERR_INVALID and "tri_dev" in mf.pcg_last_error(h.ptr)
        torch.cuda.synchronize()
        z1h, z2h, t2 = to_host(z1), to_host(z2), to_host(tri2)
    finally:
        mf.pcg_destroy(h)
    zo = oracle.precond(prob, r)
    assert np.abs(z1h - zo).max() <= precond_tol(prob, zo)
    sub, dia, sup = (t2[m * n:(m + 1) * n].reshape(r.shape) for m in range(3))
    zm = np.zeros_like(z2h)
    zp = np.zeros_like(z2h)
    zm[:, 1:, :] = z2h[:, :-1, :]
    zp[:, :-1, :] = z2h[:, 1:, :]
    Mz = sub * zm + dia * z2h + sup * zp
    scale = np.abs(sub * zm) + np.abs(dia * z2h) + np.abs(sup * zp) + np.abs(r)
    assert np.all(np.abs(Mz - r) <= 64 * EPS * scale)
    assert np.abs(z2h - z1h).max() > 1e-3 * np.abs(z1h).max()   # the second matrices really differ
