/*
 * mfpcg.h - C ABI of the matrix-free preconditioned conjugate gradient
 * library for AMD Instinct MI355X (gfx950).
 *
 * The library solves A x = b for the 3-D anisotropic elliptic
 * pressure-correction operator of E. Mueller, X. Guo, R. Scheichl, S. Shi,
 * "Matrix-free GPU implementation of a preconditioned conjugate gradient
 * solver for anisotropic elliptic PDEs" (2013), on a flat nx*ny*nz grid:
 *
 *   (A u)_ijk = delta*u_ijk
 *             + sum over the 4 horizontal faces of c_face*(u_ijk - u_nb)
 *             + alpha_z[k+1]*(u_ijk - u_i,j,k+1) + alpha_z[k]*(u_ijk - u_i,j,k-1)
 *
 * (section 3, eqs. (5)-(8), and the stencil of section 4.2, eq. (18), with
 * |T| = d_k = 1), periodic in i and j, zero-flux at the bottom and top of
 * each column.  A horizontal face coefficient is the mean of the alpha_h
 * values of the two cells it separates.  The preconditioner M keeps the
 * column blocks A_T of A (tridiagonal, eq. (8)) and drops the couplings
 * between columns (section 4.2, eq. (19)); it is inverted column by column
 * with the Thomas algorithm.
 *
 * Field layout (all device vectors): float64, linear index
 *   l = i + nx*(k + nz*j)
 * i.e. the first horizontal index runs fastest (section 6.1, eq. (22)); a
 * torch tensor of shape [ny, nz, nx].
 *
 * Memory: every pointer named *_dev is device memory on the device that was
 * current when the handle was created; *_host pointers are host memory.  The
 * library allocates no device memory: the caller owns all vectors, the
 * handle's coefficient tables (pcg_handle_bytes), the multigrid levels'
 * tables (pcg_mg_setup_bytes), the stored column matrices
 * (pcg_tridiag_bytes) and every solve workspace, and each buffer must stay
 * allocated while the handle uses it (until pcg_destroy for the tables).
 * Device buffers passed as tables or workspace must be 256-byte aligned
 * (torch's allocations are).  Besides its host-side object the handle holds
 * one 32-byte word of pinned host memory, to which the device writes each
 * step's stop decision (hipHostMalloc at creation, freed at pcg_destroy),
 * and one HIP event.  pcg_solve_static uses a fixed device array that the
 * library's code object holds (see there).
 *
 * Streams: every call is ordered on the handle's HIP stream (the one passed
 * to pcg_create, or pcg_set_stream).  pcg_apply_A and pcg_precond are
 * asynchronous; the solves block the calling thread until the result is
 * known.
 *
 * Errors: functions return PCG_OK (0), PCG_NOT_CONVERGED (+1, solves only),
 * or a negative code; pcg_last_error() then describes the failure.  Invalid
 * arguments are detected on the host before any work is queued.
 *
 * Thread safety: one handle must not be used from two threads at once.
 */
#ifndef MFPCG_H
#define MFPCG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PCG_OK 0
#define PCG_NOT_CONVERGED 1
#define PCG_ERR_INVALID (-1)     /* bad argument, grid or coefficients       */
#define PCG_ERR_BREAKDOWN (-2)   /* sigma <= 0, kappa <= 0 or a non-finite scalar */
#define PCG_ERR_HIP (-3)         /* HIP runtime error (see pcg_last_error)   */
#define PCG_ERR_UNSUPPORTED (-4) /* grid outside the supported range          */

#define PCG_AH_CONST 0 /* alpha_h(i,j) = alpha_h_const                          */
#define PCG_AH_FIELD 1 /* alpha_h(i,j) = alpha_h_field[j*nx + i] (host array)   */

typedef struct pcg_handle pcg_handle;

/* Grid: nx, ny >= 1 (periodic), 1 <= nz <= 512. */
typedef struct {
    int32_t nx, ny, nz;
} pcg_grid;

/* Tuning variables.  pcg_create, pcg_create_general and pcg_handle_bytes
 * read these environment variables; each changes the launch geometry (and
 * with it the number of partial sums, so the last bits of dot products and
 * of iterates), never the operator.  Unset or empty means the default.  They
 * are measurement and test hooks: set them only to compare launch shapes.
 *   MFPCG_COL_C      columns per column-pass workgroup, 32 or 64 (64)
 *   MFPCG_COL_L      segment length of the column solve, 4/8/16/32 (the
 *                    smallest of 8, 16, 32 that fits 1024 threads)
 *   MFPCG_COL_LF     segment length of the column passes without a stored
 *                    matrix (except pcg_solve_no_q's, which keep
 *                    MFPCG_COL_L's), 1, 2 or 4 times MFPCG_COL_L, at most 32
 *   MFPCG_ST_L       levels per wave of the stencil passes, 1/2/4/8 (4)
 *   MFPCG_ST_W       waves per stencil workgroup, 1..16 (min(4, nz/4))
 *   MFPCG_COL_FULL   0: never use the straight-line whole-tile column kernel
 *   MFPCG_ST_FULL    0: never use the whole-tile stencil kernels
 *   MFPCG_ST_JT      rows per fused stencil tile, 1, 4 or 8
 *   MFPCG_COL_STRIP, MFPCG_ST_STRIP  i-tiles per strip of the tile order
 *                    (one strip per XCD)
 * and pcg_mg_setup reads
 *   MFPCG_MG_COARSE_C  columns per column-pass workgroup on the coarsest
 *                    level, 16, 32 or 64 (the widest of 64, 32, 16 that
 *                    gives at least 256 workgroups, else 16; 64 for a
 *                    single column or segments longer than 8 levels)
 * pcg_tuning_overrides reports which of them were set when a handle was
 * created (or its hierarchy set up), as a mask of these bits (0: every
 * default): */
#define PCG_TUNE_COL_C 0x001
#define PCG_TUNE_COL_L 0x002
#define PCG_TUNE_COL_LF 0x004
#define PCG_TUNE_ST_L 0x008
#define PCG_TUNE_ST_W 0x010
#define PCG_TUNE_COL_FULL 0x020
#define PCG_TUNE_ST_FULL 0x040
#define PCG_TUNE_ST_JT 0x080
#define PCG_TUNE_COL_STRIP 0x100
#define PCG_TUNE_ST_STRIP 0x200
#define PCG_TUNE_MG_COARSE_C 0x400

/* Operator coefficients (section 3, eqs. (5)-(8); section 4.2, eq. (17)).
 *   delta         zero-order term, > 0
 *   alpha_z_face  HOST, nz+1 entries; face f lies between cells f-1 and f;
 *                 every entry >= 0 and faces 0 and nz must be 0 (no flux)
 *   alpha_h_kind  PCG_AH_CONST or PCG_AH_FIELD
 *   alpha_h_const used when kind == PCG_AH_CONST, >= 0
 *   alpha_h_field HOST, ny*nx entries [j*nx + i], each >= 0, when kind ==
 *                 PCG_AH_FIELD
 * All values are copied at pcg_create; the caller may free them after. */
typedef struct {
    double delta;
    const double *alpha_z_face;
    int32_t alpha_h_kind;
    double alpha_h_const;
    const double *alpha_h_field;
} pcg_coeffs;

/* Bytes of device memory the handle's tables need for this grid: the nz+1
 * vertical faces, a and d per level, |T| and the two edge coefficients per
 * column, and the Thomas multipliers at the column segments' boundaries in
 * binary64 and binary32, O(nz + (3 + 1.5 (ceil(nz/L) - 1)) nx*ny) doubles
 * (L: the segment length, 8 up to nz = 128).  0 for an invalid grid. */
size_t pcg_handle_bytes(const pcg_grid *grid);

/* Create a handle for one grid and operator (section 6: the coefficient
 * vectors are copied to the device once).  The operator is the special case
 * of the general form below with |T| = 1, a_k = delta, d_k = 1, beta = alpha_z
 * and the edge coefficient between two cells the mean of their alpha_h.
 *   hip_stream   a hipStream_t, or NULL for the null stream
 *   tables_dev   caller-owned device memory of >= pcg_handle_bytes(grid)
 *                bytes, 256-byte aligned, on the current device; the handle
 *                writes its tables there and reads them until pcg_destroy
 * Blocks until the tables are written.  Returns PCG_ERR_INVALID for bad
 * arguments (also a missing, misaligned or short table buffer),
 * PCG_ERR_UNSUPPORTED for nz > 512, PCG_ERR_HIP on a runtime error.  *out is
 * NULL on failure. */
int pcg_create(const pcg_grid *grid, const pcg_coeffs *coeffs, void *hip_stream,
               void *tables_dev, size_t tables_bytes, pcg_handle **out);

/* The operator with general tensor-product coefficients (section 3,
 * eqs. (5)-(8), with the signs of a symmetric positive definite operator):
 *   (A u)_{T,k} = |T| a_k u_{T,k} + d_k sum_{T'} alpha_{T,T'} (u_{T,k} - u_{T',k})
 *               + |T| (beta_{k+1} (u_{T,k} - u_{T,k+1}) + beta_k (u_{T,k} - u_{T,k-1}))
 * and M = its column blocks A_T (the couplings between columns dropped).
 *   a          HOST, nz entries, each finite and > 0 (zero-order term)
 *   d          HOST, nz entries, each finite and >= 0 (factor of the
 *              horizontal couplings at level k)
 *   beta_face  HOST, nz+1 entries, each finite and >= 0; face f lies between
 *              levels f-1 and f; faces 0 and nz must be 0 (no flux)
 *   area       HOST, ny*nx entries [j*nx + i], each finite and > 0 (|T|)
 *   alpha_x    HOST, ny*nx entries: the edge between (i, j) and
 *              (i+1 mod nx, j), each finite and >= 0
 *   alpha_y    HOST, ny*nx entries: the edge between (i, j) and
 *              (i, j+1 mod ny), each finite and >= 0
 * All values are copied at creation; the caller may free them after. */
typedef struct {
    const double *a;
    const double *d;
    const double *beta_face;
    const double *area;
    const double *alpha_x;
    const double *alpha_y;
} pcg_coeffs_general;

/* As pcg_create, for general coefficients (tables_dev: pcg_handle_bytes(grid)
 * bytes as there).  Every other entry point works on the handle unchanged
 * (binary64, binary32, mixed, explicit path). */
int pcg_create_general(const pcg_grid *grid, const pcg_coeffs_general *coeffs, void *hip_stream,
                       void *tables_dev, size_t tables_bytes, pcg_handle **out);

/* Release the handle (waits for its stream).  The table buffers stay the
 * caller's, free to reuse after this returns.  NULL is a no-op. */
int pcg_destroy(pcg_handle *h);

/* The PCG_TUNE_* bits of the tuning variables that were set when the handle
 * was created (0: every launch-geometry default; 0 for NULL). */
int32_t pcg_tuning_overrides(const pcg_handle *h);

/* Change the stream later calls are ordered on. */
int pcg_set_stream(pcg_handle *h, void *hip_stream);

/* y = A x, the matrix-free stencil that recomputes its coefficients in every
 * cell (section 4.2, eq. (18)).  x_dev, y_dev: N = nx*ny*nz doubles each,
 * must not overlap.  Asynchronous. */
int pcg_apply_A(pcg_handle *h, const double *x_dev, double *y_dev);

/* z = M^{-1} r, one tridiagonal (Thomas) solve per vertical column
 * (section 4.2, eq. (19)).  r_dev, z_dev: N doubles each, must not overlap.
 * Asynchronous. */
int pcg_precond(pcg_handle *h, const double *r_dev, double *z_dev);

/* Bytes of device workspace a solve with this maxit needs (seven N-vectors,
 * per-workgroup partial sums, the scalar state and the residual history). */
size_t pcg_solve_workspace_bytes(const pcg_handle *h, int32_t maxit);

/* Solve A x = b by PCG with the interleaved loop of section 4.3
 * (Algorithm 1): per iteration one fused preconditioner pass (Appendix A,
 * Algorithm 3: r -= alpha q, z = M^{-1} r, <r,r>, <r,z>) and one fused
 * stencil pass (Algorithm 2: x += alpha p, p = z + beta p, q = A z + beta q,
 * <p,q>), each followed by a deterministic reduction.  The x updates of
 * three steps are deferred to the stencil pass of the fourth, which applies
 * the four terms one after the other (the same sums as four updates), so x
 * is read and written every fourth step; the four latest directions live in
 * four workspace vectors, and the updates still pending when the loop stops
 * are applied before the call returns.  82 bytes per point per step
 * (preconditioner pass: read r, q, write r, z; stencil pass: read z, p, q,
 * write p, q, and every fourth step also read x and the three older
 * directions, write x).
 *   b_dev          right-hand side, N doubles
 *   x_dev          in: initial guess x0; out: the last iterate.  Must not
 *                  alias b_dev or the workspace.
 *   tol            stop after the first step with ||r_k||/||r_0|| < tol
 *                  (2-norms of the unpreconditioned residual) or r_k = 0;
 *                  tol <= 0 runs exactly maxit steps
 *   maxit          >= 0, maximum number of CG steps (x updates)
 *   workspace_dev  >= pcg_solve_workspace_bytes(h, maxit) bytes, 256-byte
 *                  aligned; contents on entry are ignored
 *   iters_out      (may be NULL) number of CG steps taken
 *   hist_host      (may be NULL) ||r_k||_2 for k = 0..iters; needs maxit+1
 *                  entries
 *   hist_len_out   (may be NULL) iters + 1 (entries written)
 *   final_rel_res  (may be NULL) hist[iters]/hist[0] (0 when r_0 = 0)
 * Returns PCG_OK, PCG_NOT_CONVERGED (maxit reached; x is the last iterate),
 * PCG_ERR_BREAKDOWN (x holds the iterate before the failing step),
 * PCG_ERR_INVALID or PCG_ERR_HIP.  Blocks until done. */
int pcg_solve(pcg_handle *h, const double *b_dev, double *x_dev, double tol, int32_t maxit,
              void *workspace_dev, size_t workspace_bytes, int32_t *iters_out,
              double *hist_host, int32_t *hist_len_out, double *final_rel_res);

/* Same contract as pcg_solve, with q never stored: the preconditioner pass
 * recomputes A p from p and its neighbours, and the stencil pass forms
 * <p_new, A z + beta A p_old> (72 bytes per point per iteration; two stencils
 * of neighbour reads per iteration instead of one). */
int pcg_solve_no_q(pcg_handle *h, const double *b_dev, double *x_dev, double tol, int32_t maxit,
                   void *workspace_dev, size_t workspace_bytes, int32_t *iters_out,
                   double *hist_host, int32_t *hist_len_out, double *final_rel_res);

/* ---- Tensor-product multigrid preconditioner ---------------------------
 * Section 2 names geometric multigrid with the vertical line relaxation as
 * the faster CPU solver and section 8 plans it for the GPU; the pages give
 * no intergrid operators, so this one is read as follows.  Levels keep nz
 * and halve nx where it is even and > 1 and ny where it is even and > 1
 * (horizontal semi-coarsening), down to one column, to a level that cannot
 * be halved, or to max_levels levels.  Prolongation P is piecewise constant
 * (a fine column takes its coarse parent's values), restriction is P^T (the
 * sum over the children), and the coarse operator is P^T A P, which has the
 * general form of section 3 again: |T| summed over the children, the edge
 * between two coarse columns the sum of the fine edges crossing it (zero in
 * a dimension of size 1), a, d and beta unchanged.  The smoother is the
 * column solve of eq. (19) as damped block Jacobi, z <- z + omega M^{-1}
 * (f - A z); the cycle is V(nu, nu) from z = 0; the coarsest level is solved
 * exactly by the column solve when it is one column, else by coarse_sweeps
 * sweeps from z = 0.  With coarse_lo > 0 those sweeps are accelerated by
 * Chebyshev polynomials on [coarse_lo, 2] (the Chebyshev semi-iteration of
 * Golub and Varga; the eigenvalues of M^{-1} A lie in (0, 2) for these
 * operators): z_1 = M^{-1} f / theta, then z_{k+1} = z_k + rho_k rho_{k-1}
 * (z_k - z_{k-1}) + (2 rho_k / delta) M^{-1} (f - A z_k), theta and delta
 * the interval's centre and half-width, rho_0 = delta / theta and
 * rho_k = 1 / (2 theta / delta - rho_{k-1}).  B (one cycle) is symmetric
 * positive definite for 0 < omega <= 1 and any coarse_lo, so CG with B is
 * PCG. */
typedef struct {
    int32_t nu;            /* sweeps before and after the coarse correction, 1..16 */
    double omega;          /* damping of the smoother, 0 < omega <= 1 */
    int32_t max_levels;    /* 0: as many levels as the grid allows; else 1..64 */
    int32_t coarse_sweeps; /* sweeps on a coarsest level of several columns, 1..1024 */
    double coarse_lo;      /* 0: damped coarsest sweeps; in (0, 2): Chebyshev on [coarse_lo, 2] */
} pcg_mg_params;

/* Bytes of device memory the coarse levels' tables need for these
 * parameters (only max_levels matters; one pcg_handle_bytes-sized set of
 * tables per coarse level, about a third of the handle's in all).  0 when
 * the hierarchy has no coarse level, or for bad arguments. */
size_t pcg_mg_setup_bytes(const pcg_handle *h, const pcg_mg_params *params);

/* Build (or rebuild) the level hierarchy: the coarse levels' coefficient
 * tables are computed on the device from the handle's, in levels_dev
 * (caller-owned device memory, >= pcg_mg_setup_bytes(h, params) bytes,
 * 256-byte aligned; may be NULL when that is 0), which the handle reads until
 * pcg_destroy or the next pcg_mg_setup.  Blocks until done.  Returns
 * PCG_ERR_INVALID for bad parameters or a short buffer, PCG_ERR_UNSUPPORTED
 * when the column tiles are not 64 columns wide, PCG_ERR_HIP on a runtime
 * error. */
int pcg_mg_setup(pcg_handle *h, const pcg_mg_params *params, void *levels_dev, size_t levels_bytes);

/* Number of levels of the hierarchy built by pcg_mg_setup (1 = none coarser
 * than the grid).  PCG_ERR_INVALID before pcg_mg_setup. */
int pcg_mg_num_levels(const pcg_handle *h, int32_t *levels);

/* Size and coefficients of level `level` (0 = the grid): nx, ny (may be
 * NULL) and, when not NULL, the HOST arrays area, alpha_x, alpha_y of
 * nx*ny entries each (layout as in pcg_coeffs_general).  Blocks. */
int pcg_mg_level(pcg_handle *h, int32_t level, int32_t *nx, int32_t *ny, double *area_host,
                 double *alpha_x_host, double *alpha_y_host);

/* Bytes of device workspace of pcg_solve_mg with this maxit (those of
 * pcg_solve, two more N-vectors, and four vectors per coarse level: about
 * 8.3 N-vectors for a full hierarchy).  0 before pcg_mg_setup. */
size_t pcg_mg_workspace_bytes(const pcg_handle *h, int32_t maxit);

/* z = B r, one V-cycle.  r_dev, z_dev: N doubles each, must not overlap each
 * other or the workspace (>= pcg_mg_workspace_bytes(h, 0) bytes, 256-byte
 * aligned).  Asynchronous. */
int pcg_mg_vcycle(pcg_handle *h, const double *r_dev, double *z_dev, void *workspace_dev,
                  size_t workspace_bytes);

/* pcg_solve with one V-cycle as the preconditioner: the interleaved loop of
 * section 4.3 with its preconditioner pass replaced by the cycle, whose first
 * sweep applies r -= alpha q and whose last sweep forms <r,r> and <r,z>.
 * Same arguments, results and errors as pcg_solve; the workspace is
 * pcg_mg_workspace_bytes(h, maxit).  PCG_ERR_INVALID before pcg_mg_setup. */
int pcg_solve_mg(pcg_handle *h, const double *b_dev, double *x_dev, double tol, int32_t maxit,
                 void *workspace_dev, size_t workspace_bytes, int32_t *iters_out,
                 double *hist_host, int32_t *hist_len_out, double *final_rel_res);

/* ---- Single precision (section 7 runs the solver in single and in double
 * precision) -------------------------------------------------------------
 * The same operator and preconditioner with the coefficients (kept in
 * binary64 by the handle) rounded to binary32 where they are used.  In every
 * entry point below the dot products <r,r>, <r,z>, <p,q> accumulate in binary64
 * and the scalars alpha, beta and the stop test are binary64 (alpha and beta
 * are rounded to binary32 where they scale a binary32 vector). */

/* y = A x in binary32 (eq. (18)); x_dev, y_dev: N floats each, must not
 * overlap.  Asynchronous. */
int pcg_apply_A_f32(pcg_handle *h, const float *x_dev, float *y_dev);

/* z = M^{-1} r in binary32 (eq. (19)), one Thomas solve per column with
 * binary32 pivots; r_dev, z_dev: N floats each, must not overlap.
 * Asynchronous. */
int pcg_precond_f32(pcg_handle *h, const float *r_dev, float *z_dev);

/* The interleaved solve of pcg_solve with every vector (b, x and the
 * workspace's r, z, p, q) in binary32: 42 bytes per point per step.  b_dev,
 * x_dev: N floats.  The workspace is the one pcg_solve_workspace_bytes sizes
 * (binary32 vectors use the front of each slot); tol below the binary32
 * rounding level of the residual (about 1e-6 relative) is not reached.
 * Returns as pcg_solve. */
int pcg_solve_f32(pcg_handle *h, const float *b_dev, float *x_dev, double tol, int32_t maxit,
                  void *workspace_dev, size_t workspace_bytes, int32_t *iters_out,
                  double *hist_host, int32_t *hist_len_out, double *final_rel_res);

/* pcg_solve with the preconditioner applied in binary32: the preconditioner
 * pass rounds the (binary64) residual to binary32, solves the column systems
 * in binary32 and stores z in binary32; the stencil pass widens z exactly.
 * Everything else is binary64: 76 bytes per point per step.  Same contract
 * and arguments as pcg_solve. */
int pcg_solve_mixed(pcg_handle *h, const double *b_dev, double *x_dev, double tol, int32_t maxit,
                    void *workspace_dev, size_t workspace_bytes, int32_t *iters_out,
                    double *hist_host, int32_t *hist_len_out, double *final_rel_res);

/* ---- The no-allocation solve --------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture set-up, tight serving loops, harnesses that forbid
 * allocation.  pcg_solve with its workspace in a fixed array that the
 * library's device code object holds (pcg_solve_static_max_bytes bytes, 64
 * MiB: each device the library runs on keeps one until the process ends).
 * The call allocates nothing (no hipMalloc, no event, no allocating library
 * routine); the caller still passes b, x and the host results.  The grid and
 * maxit must fit the array: pcg_solve_workspace_bytes(h, maxit) <= the
 * maximum (about 1.2 million points), else PCG_ERR_INVALID with the sizes in
 * pcg_last_error.  Every call on one device shares that device's array, and
 * each call leaves its state there: calls that overlap in time on one device
 * (two host threads, or two handles' streams) race and give wrong results.
 * Per-kernel timing (pcg_profile_enable) is not recorded during the call.
 * Arguments, results and errors otherwise as pcg_solve; the same kernels,
 * so the results equal pcg_solve's bit for bit. */
size_t pcg_solve_static_max_bytes(void);
int pcg_solve_static(pcg_handle *h, const double *b_dev, double *x_dev, double tol, int32_t maxit,
                     int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
                     double *final_rel_res);

/* Same contract as pcg_solve, computed by the standard (non-interleaved)
 * PCG of section 4.1: separate stencil, preconditioner and vector-update
 * passes, each vector update fused with its dot product (section 6: the
 * stand-alone kernels plus level-1 BLAS operations). */
int pcg_solve_standard(pcg_handle *h, const double *b_dev, double *x_dev, double tol,
                       int32_t maxit, void *workspace_dev, size_t workspace_bytes,
                       int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
                       double *final_rel_res);

/* ---- Explicit (matrix-stored) comparison path, section 6.2 ----------------
 * The same operator assembled as a CSR matrix and the preconditioner's column
 * matrices stored as three vectors, solved with the standard PCG loop.  Rows
 * and vectors follow the field layout; a row holds the diagonal, its distinct
 * horizontal neighbours and the vertical neighbours that exist, columns
 * ascending.  Requires N < 2^31 (int32 column indices), else
 * PCG_ERR_UNSUPPORTED.  All arrays are caller-owned device memory. */

/* Number of stored entries of the CSR matrix (host computation). */
int pcg_csr_nnz(const pcg_handle *h, int64_t *nnz);

/* Assemble the CSR matrix on the device: row_ptr_dev (N+1 int64), col_dev
 * (nnz int32), val_dev (nnz doubles).  Asynchronous. */
int pcg_csr_assemble(pcg_handle *h, int64_t *row_ptr_dev, int32_t *col_dev, double *val_dev);

/* y = A x with the assembled CSR matrix (one row per thread).  Asynchronous. */
int pcg_csr_spmv(pcg_handle *h, const int64_t *row_ptr_dev, const int32_t *col_dev,
                 const double *val_dev, const double *x_dev, double *y_dev);

/* Bytes of a stored set of column matrices: tri_dev = [sub | diag | sup |
 * phi], the three diagonals (N doubles each, field layout; sub is 0 at k = 0
 * and sup at k = nz-1) followed by their Thomas multipliers at the column
 * segments' boundaries ((ceil(nz/L) - 1) * nx*ny doubles, at least nx*ny). */
size_t pcg_tridiag_bytes(const pcg_handle *h);

/* Assemble M's column matrices into tri_dev (>= pcg_tridiag_bytes(h) bytes,
 * 256-byte aligned) and factor them (pcg_tridiag_factor).  Asynchronous. */
int pcg_tridiag_assemble(pcg_handle *h, double *tri_dev, size_t tri_bytes);

/* Compute the segment-boundary multipliers of the column matrices in
 * tri_dev's diagonals into its phi part; call again after changing the
 * diagonals.  Asynchronous. */
int pcg_tridiag_factor(pcg_handle *h, double *tri_dev, size_t tri_bytes);

/* z = M^{-1} r with the stored (factored) column matrices.  Asynchronous. */
int pcg_tridiag_precond(pcg_handle *h, const double *tri_dev, size_t tri_bytes, const double *r_dev,
                        double *z_dev);

/* Standard PCG (section 4.1) with the CSR matrix and the stored (factored)
 * column matrices (tri_dev, tri_bytes as above); arguments and results as
 * pcg_solve.  The matrix must have the
 * layout pcg_csr_assemble writes (every row stores its diagonal entry; the
 * values may differ): sigma = <p, A p> takes p at each row's point from the
 * diagonal entry's column. */
int pcg_solve_csr(pcg_handle *h, const int64_t *row_ptr_dev, const int32_t *col_dev,
                  const double *val_dev, const double *tri_dev, size_t tri_bytes,
                  const double *b_dev, double *x_dev, double tol, int32_t maxit,
                  void *workspace_dev, size_t workspace_bytes, int32_t *iters_out,
                  double *hist_host, int32_t *hist_len_out, double *final_rel_res);

/* Per-kernel timing with HIP events on the handle's stream (off by default).
 * While enabled, launches of the kernels below are bracketed by events;
 * pcg_profile_read returns the accumulated milliseconds and launch count of
 * one kernel id since the last pcg_profile_reset.  enable = 0 turns timing
 * off, 1 times every launch, P >= 2 times the solve loops' passes
 * (PCG_KID_FUSED_PREC, PCG_KID_FUSED_SPMV, PCG_KID_MG_VCYCLE) only at the
 * steps k with k mod P < 4 (four consecutive steps in every P: the stencil
 * pass's forms as often as in a whole solve; each recorded event delays the
 * next kernel by a few microseconds) and every other launch as with 1.
 * Negative: PCG_ERR_INVALID. */
#define PCG_KID_FUSED_PREC 0   /* interleaved preconditioner pass          */
#define PCG_KID_FUSED_SPMV 1   /* interleaved stencil pass                 */
#define PCG_KID_APPLY_A 2      /* stand-alone y = A x (and standard q = A p) */
#define PCG_KID_PRECOND 3      /* stand-alone z = M^{-1} r (and standard)    */
#define PCG_KID_VECTOR 4       /* standard-PCG vector updates               */
#define PCG_KID_CSR_SPMV 5     /* stand-alone CSR y = A x                    */
#define PCG_KID_MG_VCYCLE 6    /* one multigrid V-cycle (all its kernels)    */
#define PCG_KID_COUNT 7
int pcg_profile_enable(pcg_handle *h, int32_t enable);
int pcg_profile_reset(pcg_handle *h);
int pcg_profile_read(const pcg_handle *h, int32_t kernel_id, double *ms_total,
                     int64_t *launches);

/* Human-readable description of the last error on this handle (or, when h
 * is NULL, of the last failed pcg_create / pcg_create_general on the calling
 * thread).  Never NULL; valid until the next call that fails on the same
 * handle (or thread). */
const char *pcg_last_error(const pcg_handle *h);

/* Library version string. */
const char *pcg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MFPCG_H */
