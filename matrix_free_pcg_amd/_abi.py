"""ctypes binding of the C ABI in include/mfpcg.h (argument marshalling only).

Every function here has the name of the C entry point it calls.  Device
vectors are torch float64 CUDA tensors of shape [ny, nz, nx] (or any
contiguous tensor with nx*ny*nz elements); the stream is torch's current
stream unless one is given.  Nothing here computes any part of the method:
if the HIP library is missing the calls raise, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from . import build as _build

PCG_OK = 0
PCG_NOT_CONVERGED = 1
PCG_ERR_INVALID = -1
PCG_ERR_BREAKDOWN = -2
PCG_ERR_HIP = -3
PCG_ERR_UNSUPPORTED = -4

PCG_AH_CONST = 0
PCG_AH_FIELD = 1

PCG_KID_FUSED_PREC = 0
PCG_KID_FUSED_SPMV = 1
PCG_KID_APPLY_A = 2
PCG_KID_PRECOND = 3
PCG_KID_VECTOR = 4
PCG_KID_CSR_SPMV = 5
PCG_KID_MG_VCYCLE = 6
PCG_KID_COUNT = 7

EXPORTED = sorted([
    "pcg_handle_bytes", "pcg_create", "pcg_destroy", "pcg_set_stream", "pcg_tuning_overrides",
    "pcg_apply_A", "pcg_precond",
    "pcg_solve_workspace_bytes", "pcg_solve", "pcg_solve_standard", "pcg_solve_no_q",
    "pcg_solve_static", "pcg_solve_static_max_bytes",
    "pcg_profile_enable",
    "pcg_profile_reset", "pcg_profile_read", "pcg_last_error", "pcg_version",
    "pcg_csr_nnz", "pcg_csr_assemble", "pcg_csr_spmv", "pcg_tridiag_bytes", "pcg_tridiag_assemble",
    "pcg_tridiag_factor", "pcg_tridiag_precond", "pcg_solve_csr",
    "pcg_apply_A_f32", "pcg_precond_f32", "pcg_solve_f32", "pcg_solve_mixed", "pcg_create_general",
    "pcg_mg_setup_bytes", "pcg_mg_setup", "pcg_mg_num_levels", "pcg_mg_level", "pcg_mg_workspace_bytes",
    "pcg_mg_vcycle", "pcg_solve_mg",
])

PCG_TUNE_NAMES = {
    0x001: "MFPCG_COL_C", 0x002: "MFPCG_COL_L", 0x004: "MFPCG_COL_LF", 0x008: "MFPCG_ST_L",
    0x010: "MFPCG_ST_W", 0x020: "MFPCG_COL_FULL", 0x040: "MFPCG_ST_FULL", 0x080: "MFPCG_ST_JT",
    0x100: "MFPCG_COL_STRIP", 0x200: "MFPCG_ST_STRIP", 0x400: "MFPCG_MG_COARSE_C",
}


class PcgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class pcg_grid(ctypes.Structure):
    _fields_ = [("nx", ctypes.c_int32), ("ny", ctypes.c_int32), ("nz", ctypes.c_int32)]


class pcg_coeffs_general(ctypes.Structure):
    _fields_ = [(name, ctypes.POINTER(ctypes.c_double))
                for name in ("a", "d", "beta_face", "area", "alpha_x", "alpha_y")]


class pcg_mg_params(ctypes.Structure):
    _fields_ = [("nu", ctypes.c_int32), ("omega", ctypes.c_double), ("max_levels", ctypes.c_int32),
                ("coarse_sweeps", ctypes.c_int32), ("coarse_lo", ctypes.c_double)]


class pcg_coeffs(ctypes.Structure):
    _fields_ = [
        ("delta", ctypes.c_double),
        ("alpha_z_face", ctypes.POINTER(ctypes.c_double)),
        ("alpha_h_kind", ctypes.c_int32),
        ("alpha_h_const", ctypes.c_double),
        ("alpha_h_field", ctypes.POINTER(ctypes.c_double)),
    ]


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _build.LIB


def load():
    """Load libmfpcg.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = _build.LIB
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library not built: {path} is missing (run __graft_entry__.build() "
                "or python -m matrix_free_pcg_amd.build)")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        dp = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int32)
        H = ctypes.c_void_p
        sz = ctypes.c_size_t
        lib.pcg_handle_bytes.argtypes = [ctypes.POINTER(pcg_grid)]
        lib.pcg_handle_bytes.restype = sz
        lib.pcg_create.argtypes = [ctypes.POINTER(pcg_grid), ctypes.POINTER(pcg_coeffs), vp, vp, sz,
                                   ctypes.POINTER(H)]
        lib.pcg_create.restype = ctypes.c_int
        lib.pcg_create_general.argtypes = [ctypes.POINTER(pcg_grid), ctypes.POINTER(pcg_coeffs_general), vp,
                                           vp, sz, ctypes.POINTER(H)]
        lib.pcg_create_general.restype = ctypes.c_int
        lib.pcg_tuning_overrides.argtypes = [H]
        lib.pcg_tuning_overrides.restype = ctypes.c_int32
        lib.pcg_solve_static.argtypes = [H, vp, vp, ctypes.c_double, ctypes.c_int32, i32p, dp, i32p, dp]
        lib.pcg_solve_static.restype = ctypes.c_int
        lib.pcg_solve_static_max_bytes.argtypes = []
        lib.pcg_solve_static_max_bytes.restype = sz
        lib.pcg_mg_setup_bytes.argtypes = [H, ctypes.POINTER(pcg_mg_params)]
        lib.pcg_mg_setup_bytes.restype = sz
        lib.pcg_tridiag_bytes.argtypes = [H]
        lib.pcg_tridiag_bytes.restype = sz
        lib.pcg_destroy.argtypes = [H]
        lib.pcg_destroy.restype = ctypes.c_int
        lib.pcg_set_stream.argtypes = [H, vp]
        lib.pcg_set_stream.restype = ctypes.c_int
        lib.pcg_apply_A.argtypes = [H, vp, vp]
        lib.pcg_apply_A.restype = ctypes.c_int
        lib.pcg_precond.argtypes = [H, vp, vp]
        lib.pcg_precond.restype = ctypes.c_int
        lib.pcg_solve_workspace_bytes.argtypes = [H, ctypes.c_int32]
        lib.pcg_solve_workspace_bytes.restype = ctypes.c_size_t
        lib.pcg_apply_A_f32.argtypes = [H, vp, vp]
        lib.pcg_apply_A_f32.restype = ctypes.c_int
        lib.pcg_precond_f32.argtypes = [H, vp, vp]
        lib.pcg_precond_f32.restype = ctypes.c_int
        lib.pcg_mg_setup.argtypes = [H, ctypes.POINTER(pcg_mg_params), vp, sz]
        lib.pcg_mg_setup.restype = ctypes.c_int
        lib.pcg_mg_num_levels.argtypes = [H, i32p]
        lib.pcg_mg_num_levels.restype = ctypes.c_int
        lib.pcg_mg_level.argtypes = [H, ctypes.c_int32, i32p, i32p, dp, dp, dp]
        lib.pcg_mg_level.restype = ctypes.c_int
        lib.pcg_mg_workspace_bytes.argtypes = [H, ctypes.c_int32]
        lib.pcg_mg_workspace_bytes.restype = ctypes.c_size_t
        lib.pcg_mg_vcycle.argtypes = [H, vp, vp, vp, ctypes.c_size_t]
        lib.pcg_mg_vcycle.restype = ctypes.c_int
        for name in ("pcg_solve", "pcg_solve_standard", "pcg_solve_no_q", "pcg_solve_f32",
                     "pcg_solve_mixed", "pcg_solve_mg"):
            f = getattr(lib, name)
            f.argtypes = [H, vp, vp, ctypes.c_double, ctypes.c_int32, vp, ctypes.c_size_t,
                          i32p, dp, i32p, dp]
            f.restype = ctypes.c_int
        lib.pcg_profile_enable.argtypes = [H, ctypes.c_int32]
        lib.pcg_profile_enable.restype = ctypes.c_int
        lib.pcg_profile_reset.argtypes = [H]
        lib.pcg_profile_reset.restype = ctypes.c_int
        lib.pcg_profile_read.argtypes = [H, ctypes.c_int32, dp, ctypes.POINTER(ctypes.c_int64)]
        lib.pcg_profile_read.restype = ctypes.c_int
        lib.pcg_last_error.argtypes = [H]
        lib.pcg_last_error.restype = ctypes.c_char_p
        lib.pcg_version.argtypes = []
        lib.pcg_version.restype = ctypes.c_char_p
        lib.pcg_csr_nnz.argtypes = [H, ctypes.POINTER(ctypes.c_int64)]
        lib.pcg_csr_nnz.restype = ctypes.c_int
        lib.pcg_csr_assemble.argtypes = [H, vp, vp, vp]
        lib.pcg_csr_assemble.restype = ctypes.c_int
        lib.pcg_csr_spmv.argtypes = [H, vp, vp, vp, vp, vp]
        lib.pcg_csr_spmv.restype = ctypes.c_int
        lib.pcg_tridiag_assemble.argtypes = [H, vp, sz]
        lib.pcg_tridiag_assemble.restype = ctypes.c_int
        lib.pcg_tridiag_factor.argtypes = [H, vp, sz]
        lib.pcg_tridiag_factor.restype = ctypes.c_int
        lib.pcg_tridiag_precond.argtypes = [H, vp, sz, vp, vp]
        lib.pcg_tridiag_precond.restype = ctypes.c_int
        lib.pcg_solve_csr.argtypes = [H, vp, vp, vp, vp, sz, vp, vp, ctypes.c_double, ctypes.c_int32,
                                      vp, ctypes.c_size_t, i32p, dp, i32p, dp]
        lib.pcg_solve_csr.restype = ctypes.c_int
        _lib = lib
        return lib


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(t, n: int, name: str, dtype_name: str = "float64") -> int:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != getattr(torch, dtype_name) or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype_name} CUDA tensor (got {t.dtype} on {t.device})")
    if not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be contiguous with {n} elements (got {tuple(t.shape)})")
    return t.data_ptr()


def pcg_last_error(h=None) -> str:
    return load().pcg_last_error(h).decode()


def pcg_version() -> str:
    return load().pcg_version().decode()


def _check(h, rc: int, allow=(PCG_OK,)) -> int:
    if rc in allow:
        return rc
    raise PcgError(rc, pcg_last_error(h))


class Handle:
    """An open pcg_handle plus the grid it was created for and the device
    buffers it reads (its tables, and the multigrid levels' tables), which
    the caller owns: they live as long as this object."""

    def __init__(self, ptr: int, nx: int, ny: int, nz: int, device, tables=None):
        self.ptr = ptr
        self.nx, self.ny, self.nz = nx, ny, nz
        self.n = nx * ny * nz
        self.device = device
        self.tables = tables
        self.mg_tables = None

    def __repr__(self):
        return f"Handle({self.nx}x{self.ny}x{self.nz})"


def pcg_handle_bytes(nx: int, ny: int, nz: int) -> int:
    """Device bytes of a handle's tables for this grid (0 for an invalid grid)."""
    g = pcg_grid(int(nx), int(ny), int(nz))
    return int(load().pcg_handle_bytes(ctypes.byref(g)))


def _tables(g: pcg_grid):
    """A caller-owned (torch) device buffer for a handle's tables."""
    import torch
    need = int(load().pcg_handle_bytes(ctypes.byref(g)))
    return torch.empty(max(need, 256), dtype=torch.uint8, device=torch.device("cuda", torch.cuda.current_device()))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _create_general(problem, stream) -> Handle:
    import torch
    lib = load()
    g = pcg_grid(problem.nx, problem.ny, problem.nz)
    ncol = problem.nx * problem.ny
    c = pcg_coeffs_general()
    keep = []
    for name, size in (("a", problem.nz), ("d", problem.nz), ("beta_face", problem.nz + 1),
                       ("area", ncol), ("alpha_x", ncol), ("alpha_y", ncol)):
        v = np.ascontiguousarray(getattr(problem, name), dtype=np.float64).ravel()
        if v.size != size:
            raise ValueError(f"{name} must have {size} entries (got {v.size})")
        keep.append(v)
        setattr(c, name, v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    out = ctypes.c_void_p()
    tables = _tables(g)
    rc = lib.pcg_create_general(ctypes.byref(g), ctypes.byref(c), ctypes.c_void_p(_stream_ptr(stream)),
                                tables.data_ptr(), _nbytes(tables), ctypes.byref(out))
    del keep
    if rc != PCG_OK:
        raise PcgError(rc, pcg_last_error(None))
    return Handle(out.value, problem.nx, problem.ny, problem.nz, torch.cuda.current_device(), tables)


def pcg_create(problem, stream=None) -> Handle:
    """Create a handle for a :class:`workloads.Problem` (pcg_create) or a
    :class:`workloads.GeneralProblem` (pcg_create_general) on the current
    CUDA device."""
    import torch
    from .workloads import GeneralProblem
    if isinstance(problem, GeneralProblem):
        return _create_general(problem, stream)
    lib = load()
    g = pcg_grid(problem.nx, problem.ny, problem.nz)
    az = np.ascontiguousarray(problem.alpha_z_face, dtype=np.float64)
    if az.shape != (problem.nz + 1,):
        raise ValueError("alpha_z_face must have nz+1 entries")
    c = pcg_coeffs()
    c.delta = float(problem.delta)
    c.alpha_z_face = az.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    keep = [az]
    if problem.alpha_h_is_const():
        c.alpha_h_kind = PCG_AH_CONST
        c.alpha_h_const = float(problem.alpha_h)
        c.alpha_h_field = ctypes.POINTER(ctypes.c_double)()
    else:
        ah = np.ascontiguousarray(problem.alpha_h_field(), dtype=np.float64)
        if ah.shape != (problem.ny, problem.nx):
            raise ValueError("alpha_h field must have shape (ny, nx)")
        keep.append(ah)
        c.alpha_h_kind = PCG_AH_FIELD
        c.alpha_h_const = 0.0
        c.alpha_h_field = ah.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    out = ctypes.c_void_p()
    tables = _tables(g)
    rc = lib.pcg_create(ctypes.byref(g), ctypes.byref(c), ctypes.c_void_p(_stream_ptr(stream)),
                        tables.data_ptr(), _nbytes(tables), ctypes.byref(out))
    del keep
    if rc != PCG_OK:
        raise PcgError(rc, pcg_last_error(None))
    return Handle(out.value, problem.nx, problem.ny, problem.nz, torch.cuda.current_device(), tables)


def pcg_destroy(h: Handle) -> None:
    if h is not None and h.ptr:
        load().pcg_destroy(h.ptr)
        h.ptr = None
        h.tables = h.mg_tables = None


def pcg_tuning_overrides(h: Handle) -> int:
    """PCG_TUNE_* bits of the tuning variables set when the handle was created."""
    return int(load().pcg_tuning_overrides(h.ptr))


def pcg_set_stream(h: Handle, stream) -> None:
    _check(h.ptr, load().pcg_set_stream(h.ptr, ctypes.c_void_p(_stream_ptr(stream))))


def pcg_apply_A(h: Handle, x, y) -> None:
    """y = A x (asynchronous on the handle's stream)."""
    rc = load().pcg_apply_A(h.ptr, _dev_ptr(x, h.n, "x"), _dev_ptr(y, h.n, "y"))
    _check(h.ptr, rc)


def pcg_precond(h: Handle, r, z) -> None:
    """z = M^{-1} r (asynchronous on the handle's stream)."""
    rc = load().pcg_precond(h.ptr, _dev_ptr(r, h.n, "r"), _dev_ptr(z, h.n, "z"))
    _check(h.ptr, rc)


def pcg_solve_workspace_bytes(h: Handle, maxit: int) -> int:
    return int(load().pcg_solve_workspace_bytes(h.ptr, int(maxit)))


def _solve(fn, h: Handle, b, x, tol: float, maxit: int, workspace=None, dtype_name="float64",
           need=None) -> dict:
    import torch
    if need is None:
        need = pcg_solve_workspace_bytes(h, maxit)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a CUDA tensor of >= {need} bytes")
    hist = np.zeros(max(1, maxit + 1), dtype=np.float64)
    iters = ctypes.c_int32(0)
    hlen = ctypes.c_int32(0)
    rel = ctypes.c_double(0.0)
    rc = fn(h.ptr, _dev_ptr(b, h.n, "b", dtype_name), _dev_ptr(x, h.n, "x", dtype_name), float(tol), int(maxit),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            ctypes.byref(iters), hist.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            ctypes.byref(hlen), ctypes.byref(rel))
    _check(h.ptr, rc, allow=(PCG_OK, PCG_NOT_CONVERGED, PCG_ERR_BREAKDOWN))
    return dict(status=rc, iters=iters.value, hist=hist[: hlen.value].copy(),
                final_rel_res=rel.value,
                error=pcg_last_error(h.ptr) if rc == PCG_ERR_BREAKDOWN else "")


def pcg_solve(h: Handle, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Interleaved PCG, Algorithms 1-3 (x in: x0, out: solution).
    Returns status, iters, hist, final_rel_res."""
    return _solve(load().pcg_solve, h, b, x, tol, maxit, workspace)


def pcg_solve_no_q(h: Handle, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Interleaved PCG without storing q (A p recomputed; 72 B per point per iteration)."""
    return _solve(load().pcg_solve_no_q, h, b, x, tol, maxit, workspace)


def pcg_solve_static_max_bytes() -> int:
    return int(load().pcg_solve_static_max_bytes())


def pcg_solve_static(h: Handle, b, x, tol: float, maxit: int) -> dict:
    """pcg_solve with its workspace in the library's fixed device array (no
    allocation in the library or here beyond the host history array)."""
    hist = np.zeros(max(1, maxit + 1), dtype=np.float64)
    iters = ctypes.c_int32(0)
    hlen = ctypes.c_int32(0)
    rel = ctypes.c_double(0.0)
    rc = load().pcg_solve_static(h.ptr, _dev_ptr(b, h.n, "b"), _dev_ptr(x, h.n, "x"), float(tol), int(maxit),
                                 ctypes.byref(iters), hist.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                 ctypes.byref(hlen), ctypes.byref(rel))
    _check(h.ptr, rc, allow=(PCG_OK, PCG_NOT_CONVERGED, PCG_ERR_BREAKDOWN))
    return dict(status=rc, iters=iters.value, hist=hist[: hlen.value].copy(),
                final_rel_res=rel.value,
                error=pcg_last_error(h.ptr) if rc == PCG_ERR_BREAKDOWN else "")


def pcg_solve_standard(h: Handle, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Standard (non-interleaved) PCG; same contract as pcg_solve."""
    return _solve(load().pcg_solve_standard, h, b, x, tol, maxit, workspace)


def pcg_apply_A_f32(h: Handle, x, y) -> None:
    """y = A x in binary32 (float32 tensors; asynchronous on the handle's stream)."""
    rc = load().pcg_apply_A_f32(h.ptr, _dev_ptr(x, h.n, "x", "float32"), _dev_ptr(y, h.n, "y", "float32"))
    _check(h.ptr, rc)


def pcg_precond_f32(h: Handle, r, z) -> None:
    """z = M^{-1} r in binary32 (float32 tensors; asynchronous)."""
    rc = load().pcg_precond_f32(h.ptr, _dev_ptr(r, h.n, "r", "float32"), _dev_ptr(z, h.n, "z", "float32"))
    _check(h.ptr, rc)


def pcg_solve_f32(h: Handle, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Interleaved PCG in binary32 (float32 b, x; binary64 dots and scalars)."""
    return _solve(load().pcg_solve_f32, h, b, x, tol, maxit, workspace, "float32")


def pcg_solve_mixed(h: Handle, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Interleaved binary64 PCG with the column preconditioner in binary32."""
    return _solve(load().pcg_solve_mixed, h, b, x, tol, maxit, workspace)


# ---- tensor-product multigrid preconditioner ----------------------------------

def pcg_mg_setup_bytes(h: Handle, nu: int = 1, omega: float = 0.8, max_levels: int = 0,
                       coarse_sweeps: int = 2, coarse_lo: float = 0.0) -> int:
    p = pcg_mg_params(int(nu), float(omega), int(max_levels), int(coarse_sweeps), float(coarse_lo))
    return int(load().pcg_mg_setup_bytes(h.ptr, ctypes.byref(p)))


def pcg_mg_setup(h: Handle, nu: int = 1, omega: float = 0.8, max_levels: int = 0,
                 coarse_sweeps: int = 2, coarse_lo: float = 0.0) -> None:
    """Build the level hierarchy; its tables go to a (torch) device buffer
    kept on the handle object.  coarse_lo > 0: Chebyshev-accelerated
    coarsest sweeps on [coarse_lo, 2]."""
    import torch
    p = pcg_mg_params(int(nu), float(omega), int(max_levels), int(coarse_sweeps), float(coarse_lo))
    need = int(load().pcg_mg_setup_bytes(h.ptr, ctypes.byref(p)))
    buf = torch.empty(max(need, 256), dtype=torch.uint8, device=torch.device("cuda", h.device))
    _check(h.ptr, load().pcg_mg_setup(h.ptr, ctypes.byref(p), buf.data_ptr(), _nbytes(buf)))
    h.mg_tables = buf


def pcg_mg_num_levels(h: Handle) -> int:
    n = ctypes.c_int32(0)
    _check(h.ptr, load().pcg_mg_num_levels(h.ptr, ctypes.byref(n)))
    return n.value


def pcg_mg_level(h: Handle, level: int):
    """(nx, ny, area, alpha_x, alpha_y) of a level, the arrays of shape (ny, nx)."""
    lib = load()
    nx, ny = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(h.ptr, lib.pcg_mg_level(h.ptr, int(level), ctypes.byref(nx), ctypes.byref(ny), None, None, None))
    arrs = [np.zeros((ny.value, nx.value)) for _ in range(3)]
    dp = ctypes.POINTER(ctypes.c_double)
    _check(h.ptr, lib.pcg_mg_level(h.ptr, int(level), None, None, *[a.ctypes.data_as(dp) for a in arrs]))
    return nx.value, ny.value, arrs[0], arrs[1], arrs[2]


def pcg_mg_workspace_bytes(h: Handle, maxit: int) -> int:
    return int(load().pcg_mg_workspace_bytes(h.ptr, int(maxit)))


def pcg_mg_vcycle(h: Handle, r, z, workspace=None) -> None:
    """z = B r, one V-cycle (asynchronous on the handle's stream)."""
    import torch
    need = pcg_mg_workspace_bytes(h, 0)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=z.device)
    if not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a CUDA tensor of >= {need} bytes")
    rc = load().pcg_mg_vcycle(h.ptr, _dev_ptr(r, h.n, "r"), _dev_ptr(z, h.n, "z"), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size())
    _check(h.ptr, rc)


def pcg_solve_mg(h: Handle, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Interleaved PCG with one multigrid V-cycle as the preconditioner."""
    return _solve(load().pcg_solve_mg, h, b, x, tol, maxit, workspace,
                  need=pcg_mg_workspace_bytes(h, maxit))


def pcg_profile_enable(h: Handle, enable=True) -> None:
    """False/0: off; True/1: every launch; an int P >= 2: the solve loops'
    passes at the steps k with k mod P < 2 only."""
    _check(h.ptr, load().pcg_profile_enable(h.ptr, int(enable)))


def pcg_profile_reset(h: Handle) -> None:
    _check(h.ptr, load().pcg_profile_reset(h.ptr))


def pcg_profile_read(h: Handle, kid: int):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(h.ptr, load().pcg_profile_read(h.ptr, int(kid), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---- explicit (CSR + stored tridiagonal) comparison path --------------------

def _dev_tensor(t, numel: int, dtype_name: str, name: str) -> int:
    import torch
    dt = getattr(torch, dtype_name)
    if not isinstance(t, torch.Tensor) or t.dtype != dt or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype_name} CUDA tensor")
    if not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be contiguous with {numel} elements (got {t.numel()})")
    return t.data_ptr()


def pcg_csr_nnz(h: Handle) -> int:
    nnz = ctypes.c_int64(0)
    _check(h.ptr, load().pcg_csr_nnz(h.ptr, ctypes.byref(nnz)))
    return nnz.value


class Csr:
    """Device CSR matrix of the operator: row_ptr (int64, N+1), col (int32), val (float64)."""

    def __init__(self, row_ptr, col, val):
        self.row_ptr, self.col, self.val = row_ptr, col, val


def pcg_csr_assemble(h: Handle, device=None) -> Csr:
    """Allocate (torch) and assemble the CSR matrix on the device."""
    import torch
    nnz = pcg_csr_nnz(h)
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    rp = torch.empty(h.n + 1, dtype=torch.int64, device=dev)
    col = torch.empty(nnz, dtype=torch.int32, device=dev)
    val = torch.empty(nnz, dtype=torch.float64, device=dev)
    _check(h.ptr, load().pcg_csr_assemble(h.ptr, rp.data_ptr(), col.data_ptr(), val.data_ptr()))
    return Csr(rp, col, val)


def _csr_ptrs(h: Handle, A: Csr):
    nnz = A.col.numel()
    return (_dev_tensor(A.row_ptr, h.n + 1, "int64", "row_ptr"),
            _dev_tensor(A.col, nnz, "int32", "col"),
            _dev_tensor(A.val, nnz, "float64", "val"))


def pcg_csr_spmv(h: Handle, A: Csr, x, y) -> None:
    """y = A x with the CSR matrix (asynchronous)."""
    rp, col, val = _csr_ptrs(h, A)
    _check(h.ptr, load().pcg_csr_spmv(h.ptr, rp, col, val, _dev_ptr(x, h.n, "x"), _dev_ptr(y, h.n, "y")))


def pcg_tridiag_bytes(h: Handle) -> int:
    return int(load().pcg_tridiag_bytes(h.ptr))


def _tri_ptr(h: Handle, tri):
    n = pcg_tridiag_bytes(h) // 8
    return _dev_tensor(tri, n, "float64", "tri"), n * 8


def pcg_tridiag_assemble(h: Handle, device=None):
    """Allocate (torch, pcg_tridiag_bytes: [sub | diag | sup | phi]) and
    assemble + factor M's column matrices."""
    import torch
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    tri = torch.empty(pcg_tridiag_bytes(h) // 8, dtype=torch.float64, device=dev)
    _check(h.ptr, load().pcg_tridiag_assemble(h.ptr, tri.data_ptr(), _nbytes(tri)))
    return tri


def pcg_tridiag_factor(h: Handle, tri) -> None:
    _check(h.ptr, load().pcg_tridiag_factor(h.ptr, *_tri_ptr(h, tri)))


def pcg_tridiag_precond(h: Handle, tri, r, z) -> None:
    """z = M^{-1} r with the stored column matrices (asynchronous)."""
    _check(h.ptr, load().pcg_tridiag_precond(h.ptr, *_tri_ptr(h, tri), _dev_ptr(r, h.n, "r"),
                                             _dev_ptr(z, h.n, "z")))


def pcg_solve_csr(h: Handle, A: Csr, tri, b, x, tol: float, maxit: int, workspace=None) -> dict:
    """Standard PCG with the CSR matrix and the stored column matrices."""
    lib = load()
    rp, col, val = _csr_ptrs(h, A)
    tp, tb = _tri_ptr(h, tri)

    def fn(hp, bp, xp, tol_, maxit_, wsp, wsb, it, hist, hlen, rel):
        return lib.pcg_solve_csr(hp, rp, col, val, tp, tb, bp, xp, tol_, maxit_, wsp, wsb, it, hist, hlen, rel)
    return _solve(fn, h, b, x, tol, maxit, workspace)
