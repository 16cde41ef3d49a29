"""Matrix-free PCG for the anisotropic pressure-correction equation on AMD MI355X.

The solver lives in a HIP shared library with a C ABI (include/mfpcg.h); the
functions exported here are its ctypes binding (same names) plus the seeded
synthetic workloads.  Importing this package does not load the library; the
first call does, and raises if it has not been built.
"""
from . import workloads  # noqa: F401
from ._abi import (PCG_ERR_BREAKDOWN, PCG_ERR_HIP, PCG_ERR_INVALID, PCG_ERR_UNSUPPORTED,  # noqa: F401
                   PCG_KID_APPLY_A, PCG_KID_FUSED_PREC, PCG_KID_FUSED_SPMV, PCG_KID_PRECOND,
                   PCG_KID_VECTOR, PCG_NOT_CONVERGED, PCG_OK, Handle, PcgError, pcg_apply_A,
                   pcg_create, pcg_destroy, pcg_last_error, pcg_precond, pcg_profile_enable,
                   pcg_profile_read, pcg_profile_reset, pcg_set_stream, pcg_solve,
                   pcg_solve_standard, pcg_solve_no_q, pcg_solve_workspace_bytes, pcg_version,
                   PCG_KID_CSR_SPMV, Csr, pcg_csr_nnz, pcg_csr_assemble, pcg_csr_spmv,
                   pcg_tridiag_assemble, pcg_tridiag_factor, pcg_tridiag_precond, pcg_solve_csr,
                   pcg_apply_A_f32, pcg_precond_f32, pcg_solve_f32, pcg_solve_mixed,
                   PCG_KID_MG_VCYCLE, pcg_mg_setup, pcg_mg_num_levels, pcg_mg_level,
                   pcg_mg_workspace_bytes, pcg_mg_vcycle, pcg_solve_mg, pcg_handle_bytes,
                   pcg_tuning_overrides, pcg_solve_static, pcg_solve_static_max_bytes,
                   pcg_mg_setup_bytes, pcg_tridiag_bytes)

__all__ = [
    "workloads", "Handle", "PcgError", "pcg_create", "pcg_destroy", "pcg_set_stream",
    "pcg_apply_A", "pcg_precond", "pcg_solve", "pcg_solve_standard", "pcg_solve_no_q",
    "pcg_solve_workspace_bytes", "pcg_profile_enable", "pcg_profile_reset",
    "pcg_profile_read", "pcg_last_error", "pcg_version", "Csr", "pcg_csr_nnz",
    "pcg_csr_assemble", "pcg_csr_spmv", "pcg_tridiag_assemble", "pcg_tridiag_factor",
    "pcg_tridiag_precond", "pcg_solve_csr", "pcg_apply_A_f32", "pcg_precond_f32", "pcg_solve_f32",
    "pcg_solve_mixed", "pcg_mg_setup", "pcg_mg_num_levels", "pcg_mg_level", "pcg_mg_workspace_bytes",
    "pcg_mg_vcycle", "pcg_solve_mg", "pcg_handle_bytes", "pcg_tuning_overrides", "pcg_solve_static",
    "pcg_solve_static_max_bytes", "pcg_mg_setup_bytes", "pcg_tridiag_bytes",
]
