"""The no-allocation solve (pcg_solve_static) through the C ABI: its result
equals that of pcg_solve (the same kernels on a caller workspace) bit for bit,
on two calls in a row, the second with a smaller grid, so the fixed scratch
array is reused with the previous call's contents in it; grids whose
workspace exceeds the array are refused on the host."""
import numpy as np
import pytest

import matrix_free_pcg_amd as mf
from gpu_helpers import require_gpu, to_dev, to_host
from matrix_free_pcg_amd import workloads as W

pytestmark = pytest.mark.gpu


def _both(dev, w):
    import torch
    h = mf.pcg_create(w.problem)
    try:
        print(f"[no-alloc] {w.name} {w.problem.nx}x{w.problem.ny}x{w.problem.nz} maxit {w.maxit}", flush=True)
        need = mf.pcg_solve_workspace_bytes(h, w.maxit)
        assert need <= mf.pcg_solve_static_max_bytes(), need
        bd = to_dev(w.rhs, dev)
        xs = torch.zeros_like(bd)
        rs = mf.pcg_solve_static(h, bd, xs, w.tol, w.maxit)
        xw = torch.zeros_like(bd)
        rw = mf.pcg_solve(h, bd, xw, w.tol, w.maxit)
        torch.cuda.synchronize()
        return rs, to_host(xs), rw, to_host(xw)
    finally:
        mf.pcg_destroy(h)


def test_static_solve_matches_workspace_solve_twice():
    dev = require_gpu()
    # first call: 128x128x64 (1 M points, 40 MiB of vectors in the array);
    # second: a smaller 32x32x16 grid over the first call's leftovers
    for w in (W.make_workload(2), W.make_workload(1)):
        rs, xs, rw, xw = _both(dev, w)
        assert rs["status"] == rw["status"] == mf.PCG_OK, (rs, rw)
        assert rs["iters"] == rw["iters"], (rs["iters"], rw["iters"])
        assert np.array_equal(rs["hist"], rw["hist"])
        assert np.array_equal(xs, xw)
        assert rs["final_rel_res"] == rw["final_rel_res"]
        print(f"[no-alloc] {w.name}: {rs['iters']} steps, bit-identical to pcg_solve", flush=True)


def test_static_solve_refuses_grids_beyond_the_array():
    import torch
    dev = require_gpu()
    prob = W.config_problem(2, (512, 512), 64)   # 16.8 M points: 7 vectors > 64 MiB
    h = mf.pcg_create(prob)
    try:
        b = torch.zeros(h.n, dtype=torch.float64, device=dev)
        x = torch.zeros_like(b)
        with pytest.raises(mf.PcgError) as e:
            mf.pcg_solve_static(h, b, x, 1e-8, 10)
        assert e.value.code == mf.PCG_ERR_INVALID
        assert "scratch" in str(e.value)
        with pytest.raises(mf.PcgError):   # a negative maxit, as in pcg_solve
            mf.pcg_solve_static(h, b, x, 1e-8, -1)
    finally:
        mf.pcg_destroy(h)
