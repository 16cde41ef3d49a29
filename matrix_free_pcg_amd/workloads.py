"""Seeded synthetic workloads for the anisotropic pressure-correction solve.

This module only *describes and generates inputs*: grid sizes, the vertical
face coefficients, the horizontal coefficient field and seeded right-hand
sides.  It holds none of the solver's arithmetic (no operator, no
preconditioner, no Krylov step), so both the CPU oracle and the HIP path can
take their inputs from here without sharing any of the method.

Field layout (shared by every consumer): a 3-D field is a float64 array of
shape ``(ny, nz, nx)``, i.e. linear index ``l = i + nx*(k + nz*j)``; the first
horizontal index runs fastest.  This is the GPU ordering of Müller et al.,
"Matrix-free GPU implementation of a preconditioned conjugate gradient solver
for anisotropic elliptic PDEs" (2013), section 6.1, eq. (22).

Random numbers come from a counter-based SplitMix64 generator (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
value for grid cell (i, j, k) uses the counter ``c = i + nx*(j + ny*k)``, so a
field does not depend on the memory order it is stored in.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_TWO_M53 = 2.0 ** -53


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on uint64 values (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_stream(seed: int, n: int) -> np.ndarray:
    """First ``n`` outputs of the sequential SplitMix64 generator from ``seed``.

    The sequential generator adds the golden gamma to its state before each
    output; output ``t`` (0-based) is therefore ``mix64(seed + (t+1)*gamma)``,
    which is exactly the counter form used by :func:`uniform01`.
    """
    t = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + t * GOLDEN_GAMMA)


def uniform01(seed: int, counters: np.ndarray) -> np.ndarray:
    """U[0,1) doubles (53-bit) for the given counters."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        bits = mix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (c + np.uint64(1)) * GOLDEN_GAMMA)
    return (bits >> np.uint64(11)).astype(np.float64) * _TWO_M53


def _cell_counters(nx: int, ny: int, nz: int, j0: int, j1: int) -> np.ndarray:
    """Canonical counters c = i + nx*(j + ny*k) for rows j0..j1-1, in (j, k, i) order."""
    j = np.arange(j0, j1, dtype=np.uint64)[:, None, None]
    k = np.arange(nz, dtype=np.uint64)[None, :, None]
    i = np.arange(nx, dtype=np.uint64)[None, None, :]
    return i + np.uint64(nx) * (j + np.uint64(ny) * k)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked_field(nx, ny, nz, fn, rows_per_chunk=None):
    """Fill a (ny, nz, nx) field block of rows by block of rows.  Each block
    depends only on its own counters, so the blocks are computed by a pool of
    threads (numpy releases the interpreter lock inside its loops) and the
    result does not depend on the number of threads."""
    out = np.empty((ny, nz, nx), dtype=np.float64)
    if rows_per_chunk is None:
        rows_per_chunk = max(1, (1 << 22) // max(1, nx * nz))
    blocks = [(j0, min(ny, j0 + rows_per_chunk)) for j0 in range(0, ny, rows_per_chunk)]

    def fill(blk):
        j0, j1 = blk
        out[j0:j1] = fn(_cell_counters(nx, ny, nz, j0, j1))

    nw = min(_workers(), len(blocks))
    if nw <= 1:
        for blk in blocks:
            fill(blk)
    else:
        with concurrent.futures.ThreadPoolExecutor(nw) as pool:
            list(pool.map(fill, blocks))
    return out


def uniform_field(nx: int, ny: int, nz: int, seed: int, lo=-1.0, hi=1.0) -> np.ndarray:
    """Seeded U[lo,hi) field of shape (ny, nz, nx)."""
    return _chunked_field(nx, ny, nz, lambda c: lo + (hi - lo) * uniform01(seed, c))


def gaussian_field(nx: int, ny: int, nz: int, seed: int) -> np.ndarray:
    """Seeded N(0,1) field (Box-Muller from counters 2c and 2c+1)."""
    def fn(c):
        u1 = uniform01(seed, c * np.uint64(2))
        u2 = uniform01(seed, c * np.uint64(2) + np.uint64(1))
        return np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)
    return _chunked_field(nx, ny, nz, fn)


@dataclasses.dataclass
class Problem:
    """Operator coefficients of one problem (no solver state).

    ``alpha_z_face`` has nz+1 entries; face f lies between cells f-1 and f, and
    faces 0 and nz carry no flux (zero).  ``alpha_h`` is the per-column
    horizontal coefficient field of shape (ny, nx), or a float for a constant.
    """
    nx: int
    ny: int
    nz: int
    delta: float
    alpha_z_face: np.ndarray
    alpha_h: object  # float or (ny, nx) float64 array

    @property
    def n(self) -> int:
        return self.nx * self.ny * self.nz

    def alpha_h_field(self) -> np.ndarray:
        if isinstance(self.alpha_h, np.ndarray):
            return np.ascontiguousarray(self.alpha_h, dtype=np.float64)
        return np.full((self.ny, self.nx), float(self.alpha_h), dtype=np.float64)

    def alpha_h_is_const(self) -> bool:
        return not isinstance(self.alpha_h, np.ndarray)


@dataclasses.dataclass
class GeneralProblem:
    """Operator coefficients in the general tensor-product form of section 3,
    eqs. (5)-(8), as inputs only (no solver arithmetic):

      ``a``, ``d``      per level (nz): the zero-order term and the factor of the
                        horizontal couplings;
      ``beta_face``     nz+1 vertical face coefficients (faces 0 and nz are 0);
      ``area``          (ny, nx): |T| of every column;
      ``alpha_x``       (ny, nx): the edge coefficient between (i, j) and
                        (i+1 mod nx, j);
      ``alpha_y``       (ny, nx): between (i, j) and (i, j+1 mod ny).
    """
    nx: int
    ny: int
    nz: int
    a: np.ndarray
    d: np.ndarray
    beta_face: np.ndarray
    area: np.ndarray
    alpha_x: np.ndarray
    alpha_y: np.ndarray

    @property
    def n(self) -> int:
        return self.nx * self.ny * self.nz


def general_problem(nx: int, ny: int, nz: int, seed: int) -> GeneralProblem:
    """Seeded general-coefficient operator: a synthetic stand-in for the thin
    spherical shell of the paper's model problem (its own parameters are not
    recoverable from the page).  Vertical faces r_f = 1 + 0.02 (f/nz)^2
    (finer near the ground); with cell thicknesses h_k, mean thickness hb and
    mid-points m_k: a_k = 1e-3 h_k / hb, d_k = h_k / hb, interior
    beta_f = 1e4 r_f^2 hb / (m_f - m_{f-1}).  The area is that of a gnomonic
    panel cell, (1 + x^2 + y^2)^(-3/2) at the cell centre (x, y) in [-1, 1]^2,
    times 1 + 0.1 sin(...); the edge coefficients are 1 + 0.25 * products of
    sinusoids; phases from the generator keyed ``seed ^ 0x5A``."""
    u = uniform01(seed ^ 0x5A, np.arange(6, dtype=np.uint64))
    ph = 2.0 * math.pi * u
    f = np.arange(nz + 1, dtype=np.float64)
    r = 1.0 + 0.02 * (f / nz) ** 2
    h = np.diff(r)
    hb = h.mean()
    m = 0.5 * (r[:-1] + r[1:])
    a = 1e-3 * h / hb
    d = h / hb
    beta = np.zeros(nz + 1)
    if nz > 1:
        beta[1:nz] = 1e4 * r[1:nz] ** 2 * hb / np.diff(m)
    i = np.arange(nx, dtype=np.float64)
    j = np.arange(ny, dtype=np.float64)
    x = -1.0 + (2.0 * i + 1.0) / nx
    y = -1.0 + (2.0 * j + 1.0) / ny
    area = (1.0 + x[None, :] ** 2 + y[:, None] ** 2) ** -1.5
    area = area * (1.0 + 0.1 * np.sin(2.0 * math.pi * j[:, None] / ny + ph[0]) * np.sin(2.0 * math.pi * i[None, :] / nx + ph[1]))
    ax = 1.0 + 0.25 * np.cos(2.0 * math.pi * (i[None, :] + 0.5) / nx + ph[2]) * np.sin(2.0 * math.pi * j[:, None] / ny + ph[3])
    ay = 1.0 + 0.25 * np.sin(2.0 * math.pi * i[None, :] / nx + ph[4]) * np.cos(2.0 * math.pi * (j[:, None] + 0.5) / ny + ph[5])
    return GeneralProblem(nx, ny, nz, a, d, beta, np.ascontiguousarray(area), np.ascontiguousarray(ax),
                          np.ascontiguousarray(ay))


@dataclasses.dataclass
class Workload:
    name: str
    problem: object                  # Problem, or GeneralProblem for the general workload
    rhs: Optional[np.ndarray]        # b, or None when b = A x_true (each side applies its own A)
    x_true: Optional[np.ndarray]     # manufactured solution, when there is one
    tol: float
    maxit: int
    fixed_iterations: bool = False   # run exactly maxit steps (tol = 0)


def constant_faces(nz: int, value: float) -> np.ndarray:
    f = np.zeros(nz + 1)
    f[1:nz] = value
    return f


def graded_faces(nz: int, scale: float, slope: float) -> np.ndarray:
    """alpha_z on face f = scale*(1 + slope*f/nz)^2 for interior faces f=1..nz-1."""
    f = np.zeros(nz + 1)
    ff = np.arange(1, nz, dtype=np.float64)
    f[1:nz] = scale * (1.0 + slope * ff / nz) ** 2
    return f


def separable_alpha_h(nx: int, ny: int, h0: float, h1: float) -> np.ndarray:
    """alpha_h(i,j) = h0 + h1*sin(2 pi i/nx)*cos(2 pi j/ny), shape (ny, nx)."""
    sx = np.sin(2.0 * math.pi * np.arange(nx) / nx)
    cy = np.cos(2.0 * math.pi * np.arange(ny) / ny)
    return h0 + h1 * (cy[:, None] * sx[None, :])


def smooth_field(nx: int, ny: int, nz: int, seed: int, modes: int = 8) -> np.ndarray:
    """Sum of `modes` random low-wavenumber separable sinusoids (manufactured x_true).

    Mode m uses amplitude a ~ U[-1,1], horizontal wavenumbers p, q in {0..4},
    a non-integer vertical wavenumber w ~ U[0.5, 3.5] and phases ~ U[0, 2 pi),
    all drawn from the generator keyed ``seed ^ 0xC3`` at counters 7m..7m+6.
    """
    key = seed ^ 0xC3
    u = uniform01(key, np.arange(7 * modes, dtype=np.uint64)).reshape(modes, 7)
    i = np.arange(nx, dtype=np.float64)
    j = np.arange(ny, dtype=np.float64)
    k = np.arange(nz, dtype=np.float64)
    out = np.zeros((ny, nz, nx))
    for m in range(modes):
        a = 2.0 * u[m, 0] - 1.0
        p = math.floor(5.0 * u[m, 1])
        q = math.floor(5.0 * u[m, 2])
        w = 0.5 + 3.0 * u[m, 3]
        th, ps, ch = (2.0 * math.pi * u[m, 4], 2.0 * math.pi * u[m, 5], 2.0 * math.pi * u[m, 6])
        fx = np.cos(2.0 * math.pi * p * i / nx + th)
        fy = np.cos(2.0 * math.pi * q * j / ny + ps)
        fz = np.cos(math.pi * w * (k + 0.5) / nz + ch)
        out += a * fy[:, None, None] * fz[None, :, None] * fx[None, None, :]
    return out


CONFIG_NAMES = {
    1: "tiny-32x32x16",
    2: "graded-128x128x64",
    3: "manufactured-512x512x128",
    4: "varying-1024x1024x128",
    5: "csr-vs-mf-2048x2048x128",
    6: "general-1024x1024x128",
}


def config_problem(cfg: int, scale_xy: Optional[tuple] = None, nz: Optional[int] = None):
    """Operator of workload `cfg` (1..6); `scale_xy`/`nz` override the grid (same recipe)."""
    dims = {1: (32, 32, 16), 2: (128, 128, 64), 3: (512, 512, 128),
            4: (1024, 1024, 128), 5: (2048, 2048, 128), 6: (1024, 1024, 128)}[cfg]
    nx, ny, z = dims
    if scale_xy is not None:
        nx, ny = scale_xy
    if nz is not None:
        z = nz
    if cfg == 6:
        return general_problem(nx, ny, z, 6)
    if cfg == 1:
        return Problem(nx, ny, z, 1e-2, constant_faces(z, 1e3), 1.0)
    if cfg == 2:
        return Problem(nx, ny, z, 1e-3, graded_faces(z, 1e3, 1.0), 1.0)
    if cfg == 3:
        return Problem(nx, ny, z, 1e-3, constant_faces(z, 1e4), 1.0)
    # configs 4 and 5 share the operator
    return Problem(nx, ny, z, 1e-3, graded_faces(z, 1e4, 2.0), separable_alpha_h(nx, ny, 1.0, 0.5))


def make_workload(cfg: int, scale_xy: Optional[tuple] = None, nz: Optional[int] = None) -> Workload:
    """Seeded workload `cfg` (1..6), optionally on a smaller grid with the same recipe."""
    prob = config_problem(cfg, scale_xy, nz)
    nx, ny, z = prob.nx, prob.ny, prob.nz
    name = CONFIG_NAMES[cfg] if scale_xy is None and nz is None else f"cfg{cfg}-{nx}x{ny}x{z}"
    if cfg == 1:
        return Workload(name, prob, uniform_field(nx, ny, z, 1), None, 1e-10, 500)
    if cfg == 2:
        b = gaussian_field(nx, ny, z, 2)
        b -= b.mean()
        return Workload(name, prob, b, None, 1e-10, 5000)
    if cfg == 3:
        return Workload(name, prob, None, smooth_field(nx, ny, z, 3), 1e-10, 5000)
    if cfg == 4:
        return Workload(name, prob, uniform_field(nx, ny, z, 4), None, 1e-10, 5000)
    if cfg == 6:
        return Workload(name, prob, uniform_field(nx, ny, z, 6), None, 1e-10, 5000)
    return Workload(name, prob, gaussian_field(nx, ny, z, 5), None, 0.0, 50, fixed_iterations=True)
