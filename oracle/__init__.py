"""CPU oracle (plain C, float64, single-threaded) — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The HIP product path never calls it and shares
no code with it; ``oracle.c`` names the passage each function follows and the
readings taken where the source page is silent.

Functions take a :class:`matrix_free_pcg_amd.workloads.Problem` (inputs only)
and numpy float64 fields of shape (ny, nz, nx); the ``*_f32`` functions take
and return float32 fields (binary32 arithmetic, readings in ``oracle.c``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
import types

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_default = None

OK, NOT_CONVERGED, ERR_INVALID, ERR_BREAKDOWN = 0, 1, -1, -2

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def compile_source(src: str, out: str) -> str:
    """Compile an oracle source file with gcc into a shared library."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (always, when force)."""
    if force or not os.path.exists(_LIB):
        compile_source(SOURCE, _LIB)
    return _LIB


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _fptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        d = ctypes.c_double
        lib.orc_apply_A.argtypes = [i, i, i, d, dp, dp, dp, dp]
        lib.orc_apply_A.restype = None
        lib.orc_precond.argtypes = [i, i, i, d, dp, dp, dp, dp]
        lib.orc_precond.restype = i
        lib.orc_dot.argtypes = [ctypes.c_size_t, dp, dp]
        lib.orc_dot.restype = d
        lib.orc_alpha_T.argtypes = [i, i, dp, i, i]
        lib.orc_alpha_T.restype = d
        lib.orc_pcg.argtypes = [i, i, i, d, dp, dp, dp, dp, d, i, dp,
                                ctypes.POINTER(ctypes.c_int), i, dp, dp, dp]
        lib.orc_pcg.restype = i
        lib.orc_last_loop_seconds.argtypes = []
        lib.orc_last_loop_seconds.restype = d
        lib.orc_last_full_steps_seconds.argtypes = [ctypes.POINTER(ctypes.c_int)]
        lib.orc_last_full_steps_seconds.restype = d
        fp = ctypes.POINTER(ctypes.c_float)
        f = ctypes.c_float
        ip = ctypes.POINTER(ctypes.c_int)
        lib.orc_apply_A_f32.argtypes = [i, i, i, f, fp, fp, fp, fp]
        lib.orc_apply_A_f32.restype = None
        lib.orc_precond_f32.argtypes = [i, i, i, f, fp, fp, fp, fp]
        lib.orc_precond_f32.restype = i
        lib.orc_dot_f32.argtypes = [ctypes.c_size_t, fp, fp]
        lib.orc_dot_f32.restype = d
        lib.orc_pcg_f32.argtypes = [i, i, i, d, dp, dp, fp, fp, d, i, dp, ip]
        lib.orc_pcg_f32.restype = i
        lib.orc_pcg_mixed.argtypes = [i, i, i, d, dp, dp, dp, dp, d, i, dp, ip]
        lib.orc_pcg_mixed.restype = i
        gen = [i, i, i, dp, dp, dp, dp, dp, dp]
        lib.orc_apply_A_gen.argtypes = gen + [dp, dp]
        lib.orc_apply_A_gen.restype = None
        lib.orc_precond_gen.argtypes = gen + [dp, dp]
        lib.orc_precond_gen.restype = i
        lib.orc_pcg_gen.argtypes = gen + [dp, dp, d, i, dp, ip]
        lib.orc_pcg_gen.restype = i
        lib.orc_mg_coarsen.argtypes = [i, i, dp, dp, dp, ip, ip, dp, dp, dp]
        lib.orc_mg_coarsen.restype = i
        lib.orc_mg_num_levels.argtypes = [i, i, i]
        lib.orc_mg_num_levels.restype = i
        mg = [i, d, i, i, d]
        lib.orc_mg_vcycle.argtypes = gen + mg + [dp, dp]
        lib.orc_mg_vcycle.restype = i
        lib.orc_pcg_mg.argtypes = gen + mg + [dp, dp, d, i, dp, ip]
        lib.orc_pcg_mg.restype = i
        self.lib = lib
        self.path = path

    @staticmethod
    def _field(a, prob) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float64)
        if a.size != prob.n:
            raise ValueError(f"field has {a.size} entries, grid needs {prob.n}")
        return a.reshape(prob.ny, prob.nz, prob.nx)

    @staticmethod
    def _coeffs(prob):
        az = np.ascontiguousarray(prob.alpha_z_face, dtype=np.float64)
        if az.shape != (prob.nz + 1,):
            raise ValueError("alpha_z_face must have nz+1 entries")
        return az, prob.alpha_h_field()

    def apply_A(self, prob, x) -> np.ndarray:
        """y = A x (matrix-free 7-point stencil)."""
        x = self._field(x, prob)
        az, ah = self._coeffs(prob)
        y = np.empty_like(x)
        self.lib.orc_apply_A(prob.nx, prob.ny, prob.nz, prob.delta, _ptr(az), _ptr(ah), _ptr(x), _ptr(y))
        return y

    def precond(self, prob, r) -> np.ndarray:
        """z = M^{-1} r (Thomas algorithm, one tridiagonal system per column)."""
        r = self._field(r, prob)
        az, ah = self._coeffs(prob)
        z = np.empty_like(r)
        st = self.lib.orc_precond(prob.nx, prob.ny, prob.nz, prob.delta, _ptr(az), _ptr(ah), _ptr(r), _ptr(z))
        if st != OK:
            raise FloatingPointError("zero pivot in the column solve")
        return z

    @staticmethod
    def _field32(a, prob) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float32)
        if a.size != prob.n:
            raise ValueError(f"field has {a.size} entries, grid needs {prob.n}")
        return a.reshape(prob.ny, prob.nz, prob.nx)

    def _coeffs32(self, prob):
        az, ah = self._coeffs(prob)
        return np.float32(prob.delta), az.astype(np.float32), np.ascontiguousarray(ah, dtype=np.float32)

    def apply_A_f32(self, prob, x) -> np.ndarray:
        """y = A x in binary32 (coefficients rounded to binary32)."""
        x = self._field32(x, prob)
        d32, az, ah = self._coeffs32(prob)
        y = np.empty_like(x)
        self.lib.orc_apply_A_f32(prob.nx, prob.ny, prob.nz, float(d32), _fptr(az), _fptr(ah), _fptr(x), _fptr(y))
        return y

    def precond_f32(self, prob, r) -> np.ndarray:
        """z = M^{-1} r in binary32 (Thomas algorithm per column)."""
        r = self._field32(r, prob)
        d32, az, ah = self._coeffs32(prob)
        z = np.empty_like(r)
        st = self.lib.orc_precond_f32(prob.nx, prob.ny, prob.nz, float(d32), _fptr(az), _fptr(ah), _fptr(r), _fptr(z))
        if st != OK:
            raise FloatingPointError("zero pivot in the column solve")
        return z

    def dot_f32(self, a, b) -> float:
        a = np.ascontiguousarray(a, dtype=np.float32).ravel()
        b = np.ascontiguousarray(b, dtype=np.float32).ravel()
        return self.lib.orc_dot_f32(a.size, _fptr(a), _fptr(b))

    def pcg_f32(self, prob, b, x0=None, tol: float = 1e-5, maxit: int = 500):
        """PCG in binary32.  Returns dict(x (float32), iters, hist (float64), status)."""
        b = self._field32(b, prob)
        x = np.zeros_like(b) if x0 is None else self._field32(x0, prob).copy()
        az, ah = self._coeffs(prob)
        hist = np.zeros(max(1, maxit + 1))
        iters = ctypes.c_int(0)
        st = self.lib.orc_pcg_f32(prob.nx, prob.ny, prob.nz, prob.delta, _ptr(az), _ptr(ah), _fptr(b),
                                  _fptr(x), float(tol), int(maxit), _ptr(hist), ctypes.byref(iters))
        return dict(x=x, iters=iters.value, hist=hist[: iters.value + 1].copy(), status=st)

    def pcg_mixed(self, prob, b, x0=None, tol: float = 1e-10, maxit: int = 500):
        """Binary64 PCG with the preconditioner applied in binary32."""
        b = self._field(b, prob)
        x = np.zeros_like(b) if x0 is None else self._field(x0, prob).copy()
        az, ah = self._coeffs(prob)
        hist = np.zeros(max(1, maxit + 1))
        iters = ctypes.c_int(0)
        st = self.lib.orc_pcg_mixed(prob.nx, prob.ny, prob.nz, prob.delta, _ptr(az), _ptr(ah), _ptr(b),
                                    _ptr(x), float(tol), int(maxit), _ptr(hist), ctypes.byref(iters))
        return dict(x=x, iters=iters.value, hist=hist[: iters.value + 1].copy(), status=st)

    @staticmethod
    def _gen(gp):
        """Coefficient arrays of a GeneralProblem (float64, contiguous, checked)."""
        nz, ncol = gp.nz, gp.nx * gp.ny
        arrs = []
        for name, size in (("a", nz), ("d", nz), ("beta_face", nz + 1), ("area", ncol),
                           ("alpha_x", ncol), ("alpha_y", ncol)):
            v = np.ascontiguousarray(getattr(gp, name), dtype=np.float64).ravel()
            if v.size != size:
                raise ValueError(f"{name} has {v.size} entries, needs {size}")
            arrs.append(v)
        return arrs

    def _gen_args(self, gp):
        arrs = self._gen(gp)
        return (gp.nx, gp.ny, gp.nz, *[_ptr(v) for v in arrs]), arrs

    def apply_A_gen(self, gp, x) -> np.ndarray:
        """y = A x for general tensor-product coefficients (eqs. (5)-(8))."""
        x = self._field(x, gp)
        args, keep = self._gen_args(gp)
        y = np.empty_like(x)
        self.lib.orc_apply_A_gen(*args, _ptr(x), _ptr(y))
        return y

    def precond_gen(self, gp, r) -> np.ndarray:
        """z = M^{-1} r for general coefficients (Thomas per column)."""
        r = self._field(r, gp)
        args, keep = self._gen_args(gp)
        z = np.empty_like(r)
        if self.lib.orc_precond_gen(*args, _ptr(r), _ptr(z)) != OK:
            raise FloatingPointError("zero pivot in the column solve")
        return z

    def pcg_gen(self, gp, b, x0=None, tol: float = 1e-10, maxit: int = 500):
        """Textbook PCG with general coefficients.  Returns dict(x, iters, hist, status)."""
        b = self._field(b, gp)
        x = np.zeros_like(b) if x0 is None else self._field(x0, gp).copy()
        args, keep = self._gen_args(gp)
        hist = np.zeros(max(1, maxit + 1))
        iters = ctypes.c_int(0)
        st = self.lib.orc_pcg_gen(*args, _ptr(b), _ptr(x), float(tol), int(maxit), _ptr(hist),
                                  ctypes.byref(iters))
        return dict(x=x, iters=iters.value, hist=hist[: iters.value + 1].copy(), status=st)

    # ---- tensor-product multigrid (readings in oracle.c) --------------------
    def mg_coarsen(self, gp):
        """The Galerkin coarse operator of one coarsening step, as an object
        with the fields of a general problem; None if the level cannot be
        coarsened."""
        a, d, beta, area, ax, ay = self._gen(gp)
        ncol = gp.nx * gp.ny
        ca, cx, cy = np.zeros(ncol), np.zeros(ncol), np.zeros(ncol)
        ncx, ncy = ctypes.c_int(0), ctypes.c_int(0)
        if not self.lib.orc_mg_coarsen(gp.nx, gp.ny, _ptr(area), _ptr(ax), _ptr(ay), ctypes.byref(ncx),
                                       ctypes.byref(ncy), _ptr(ca), _ptr(cx), _ptr(cy)):
            return None
        m = ncx.value * ncy.value
        shape = (ncy.value, ncx.value)
        return types.SimpleNamespace(nx=ncx.value, ny=ncy.value, nz=gp.nz, n=m * gp.nz, a=a.copy(), d=d.copy(),
                                     beta_face=beta.copy(), area=ca[:m].reshape(shape).copy(),
                                     alpha_x=cx[:m].reshape(shape).copy(), alpha_y=cy[:m].reshape(shape).copy())

    def mg_num_levels(self, nx: int, ny: int, max_levels: int = 0) -> int:
        return self.lib.orc_mg_num_levels(int(nx), int(ny), int(max_levels))

    def mg_vcycle(self, gp, r, nu: int = 1, omega: float = 0.8, max_levels: int = 0,
                  coarse_sweeps: int = 2, coarse_lo: float = 0.0) -> np.ndarray:
        """z = B r: one V(nu, nu) cycle of the multigrid hierarchy (coarse_lo > 0:
        Chebyshev-accelerated coarsest sweeps on [coarse_lo, 2])."""
        r = self._field(r, gp)
        args, keep = self._gen_args(gp)
        z = np.empty_like(r)
        st = self.lib.orc_mg_vcycle(*args, int(nu), float(omega), int(max_levels), int(coarse_sweeps),
                                    float(coarse_lo), _ptr(r), _ptr(z))
        if st != OK:
            raise FloatingPointError(f"V-cycle failed ({st})")
        return z

    def pcg_mg(self, gp, b, x0=None, tol: float = 1e-10, maxit: int = 500, nu: int = 1,
               omega: float = 0.8, max_levels: int = 0, coarse_sweeps: int = 2, coarse_lo: float = 0.0):
        """Textbook PCG with one V-cycle per step.  Returns dict(x, iters, hist, status)."""
        b = self._field(b, gp)
        x = np.zeros_like(b) if x0 is None else self._field(x0, gp).copy()
        args, keep = self._gen_args(gp)
        hist = np.zeros(max(1, maxit + 1))
        iters = ctypes.c_int(0)
        st = self.lib.orc_pcg_mg(*args, int(nu), float(omega), int(max_levels), int(coarse_sweeps),
                                 float(coarse_lo), _ptr(b), _ptr(x), float(tol), int(maxit), _ptr(hist),
                                 ctypes.byref(iters))
        return dict(x=x, iters=iters.value, hist=hist[: iters.value + 1].copy(), status=st)

    def dot(self, a, b) -> float:
        a = np.ascontiguousarray(a, dtype=np.float64).ravel()
        b = np.ascontiguousarray(b, dtype=np.float64).ravel()
        return self.lib.orc_dot(a.size, _ptr(a), _ptr(b))

    def alpha_T(self, prob, i: int, j: int) -> float:
        ah = prob.alpha_h_field()
        return self.lib.orc_alpha_T(prob.nx, prob.ny, _ptr(ah), i, j)

    def pcg(self, prob, b, x0=None, tol: float = 1e-10, maxit: int = 500, ntrace: int = 0):
        """Textbook PCG.  Returns dict(x, iters, hist, status[, trace_r, trace_z, trace_p])."""
        b = self._field(b, prob)
        x = np.zeros_like(b) if x0 is None else self._field(x0, prob).copy()
        az, ah = self._coeffs(prob)
        hist = np.zeros(max(1, maxit + 1))
        iters = ctypes.c_int(0)
        ntr = max(0, min(ntrace, maxit + 1))
        tr = [np.zeros((ntr,) + b.shape) for _ in range(3)] if ntr > 0 else [np.zeros(1)] * 3
        st = self.lib.orc_pcg(prob.nx, prob.ny, prob.nz, prob.delta, _ptr(az), _ptr(ah), _ptr(b),
                              _ptr(x), float(tol), int(maxit), _ptr(hist), ctypes.byref(iters), ntr,
                              _ptr(tr[0]), _ptr(tr[1]), _ptr(tr[2]))
        nfull = ctypes.c_int(0)
        full_s = self.lib.orc_last_full_steps_seconds(ctypes.byref(nfull))
        out = dict(x=x, iters=iters.value, hist=hist[: iters.value + 1].copy(), status=st,
                   loop_seconds=self.lib.orc_last_loop_seconds(),
                   full_steps=nfull.value, full_steps_seconds=full_s)
        if ntr > 0:
            out.update(trace_r=tr[0], trace_z=tr[1], trace_p=tr[2])
        return out


def default() -> Oracle:
    """The oracle built from oracle.c (rebuilt when the source is newer)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
                build(force=True)
            _default = Oracle(_LIB)
        return _default


def apply_A(prob, x):
    return default().apply_A(prob, x)


def precond(prob, r):
    return default().precond(prob, r)


def dot(a, b):
    return default().dot(a, b)


def alpha_T(prob, i, j):
    return default().alpha_T(prob, i, j)


def pcg(prob, b, x0=None, tol=1e-10, maxit=500, ntrace=0):
    return default().pcg(prob, b, x0, tol, maxit, ntrace)


def apply_A_f32(prob, x):
    return default().apply_A_f32(prob, x)


def precond_f32(prob, r):
    return default().precond_f32(prob, r)


def dot_f32(a, b):
    return default().dot_f32(a, b)


def pcg_f32(prob, b, x0=None, tol=1e-5, maxit=500):
    return default().pcg_f32(prob, b, x0, tol, maxit)


def pcg_mixed(prob, b, x0=None, tol=1e-10, maxit=500):
    return default().pcg_mixed(prob, b, x0, tol, maxit)


def apply_A_gen(gp, x):
    return default().apply_A_gen(gp, x)


def precond_gen(gp, r):
    return default().precond_gen(gp, r)


def pcg_gen(gp, b, x0=None, tol=1e-10, maxit=500):
    return default().pcg_gen(gp, b, x0, tol, maxit)


def mg_coarsen(gp):
    return default().mg_coarsen(gp)


def mg_num_levels(nx, ny, max_levels=0):
    return default().mg_num_levels(nx, ny, max_levels)


def mg_vcycle(gp, r, nu=1, omega=0.8, max_levels=0, coarse_sweeps=2, coarse_lo=0.0):
    return default().mg_vcycle(gp, r, nu, omega, max_levels, coarse_sweeps, coarse_lo)


def pcg_mg(gp, b, x0=None, tol=1e-10, maxit=500, nu=1, omega=0.8, max_levels=0, coarse_sweeps=2, coarse_lo=0.0):
    return default().pcg_mg(gp, b, x0, tol, maxit, nu, omega, max_levels, coarse_sweeps, coarse_lo)
