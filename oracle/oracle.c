/*
 * CPU oracle for the matrix-free PCG solve of the anisotropic
 * pressure-correction equation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP
 * library.
 *
 * Source: E. Mueller, X. Guo, R. Scheichl, S. Shi, "Matrix-free GPU
 * implementation of a preconditioned conjugate gradient solver for
 * anisotropic elliptic PDEs" (2013).  Each function names the passage it
 * follows.  Deliberately plain: single thread, float64, no blocking, no
 * fusion, compiled with -O2 -ffp-contract=off.
 *
 * Readings taken where the page is silent or garbled (each is also listed in
 * the design notes):
 *  - operator signs: the symmetric positive definite 7-point operator
 *      (A u) = delta*u + sum over the 6 faces of coeff_face*(u - u_neighbour)
 *    (section 3 eqs. (5)-(8) and eq. (18) with |T|=d_k=1, a'_k=delta and the
 *    off-diagonal couplings negative);
 *  - boundaries: periodic in i and j; zero-flux faces at the bottom and the
 *    top of every column (face 0 and face nz carry no coupling);
 *  - a horizontal face coefficient is the arithmetic mean of the two cells'
 *    alpha_h values, so A is symmetric;
 *  - the preconditioner M keeps A's column blocks A_T (tridiagonal, with the
 *    full horizontal diagonal alpha_T on its diagonal) and drops only the
 *    couplings between columns (section 4.2, before eq. (19));
 *  - PCG is the textbook loop (section 4.1); it stops after the first CG step
 *    with ||r_k||/||r_0|| < tol (strict) or r_k == 0 (section 4.3, Algorithm 1
 *    with tau disabled); a step count is a count of x-updates;
 *  - dot products use Neumaier-compensated sequential summation in memory
 *    order.
 *
 * Field layout: l = i + nx*(k + nz*j) (section 6.1, eq. (22)); the horizontal
 * coefficient field is indexed [j*nx + i].  The algorithm is indifferent to
 * the order; this order is used so that no conversion is needed.
 */
#define _POSIX_C_SOURCE 199309L
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ORC_OK 0
#define ORC_NOT_CONVERGED 1
#define ORC_ERR_INVALID (-1)
#define ORC_ERR_BREAKDOWN (-2)

static size_t at(int nx, int nz, int i, int j, int k)
{
    return (size_t)i + (size_t)nx * ((size_t)k + (size_t)nz * (size_t)j);
}

/* Horizontal face coefficients of cell (i,j): mean of the two cells sharing
 * the face (section 3, eqs. (6)-(7): alpha_{T,T'} is one symmetric value per
 * edge; here its value is the mean of the two cells' alpha_h). */
static double face_xp(int nx, const double *ah, int i, int j)
{
    int ip = (i + 1) % nx;
    return 0.5 * (ah[(size_t)j * nx + i] + ah[(size_t)j * nx + ip]);
}
static double face_xm(int nx, const double *ah, int i, int j)
{
    int im = (i + nx - 1) % nx;
    return 0.5 * (ah[(size_t)j * nx + i] + ah[(size_t)j * nx + im]);
}
static double face_yp(int nx, int ny, const double *ah, int i, int j)
{
    int jp = (j + 1) % ny;
    return 0.5 * (ah[(size_t)j * nx + i] + ah[(size_t)jp * nx + i]);
}
static double face_ym(int nx, int ny, const double *ah, int i, int j)
{
    int jm = (j + ny - 1) % ny;
    return 0.5 * (ah[(size_t)j * nx + i] + ah[(size_t)jm * nx + i]);
}

/* alpha_T: sum of the horizontal couplings of one column (section 3, eq. (7)). */
double orc_alpha_T(int nx, int ny, const double *ah, int i, int j)
{
    return face_xp(nx, ah, i, j) + face_xm(nx, ah, i, j)
         + face_yp(nx, ny, ah, i, j) + face_ym(nx, ny, ah, i, j);
}

/* y = A x: the matrix-free 7-point stencil, recomputing every coefficient
 * (section 4.2, eq. (18), read with the signs above). */
void orc_apply_A(int nx, int ny, int nz, double delta, const double *az,
                 const double *ah, const double *x, double *y)
{
    for (int j = 0; j < ny; ++j)
        for (int k = 0; k < nz; ++k)
            for (int i = 0; i < nx; ++i) {
                int ip = (i + 1) % nx, im = (i + nx - 1) % nx;
                int jp = (j + 1) % ny, jm = (j + ny - 1) % ny;
                double u = x[at(nx, nz, i, j, k)];
                double acc = delta * u;
                acc += face_xp(nx, ah, i, j) * (u - x[at(nx, nz, ip, j, k)]);
                acc += face_xm(nx, ah, i, j) * (u - x[at(nx, nz, im, j, k)]);
                acc += face_yp(nx, ny, ah, i, j) * (u - x[at(nx, nz, i, jp, k)]);
                acc += face_ym(nx, ny, ah, i, j) * (u - x[at(nx, nz, i, jm, k)]);
                if (k < nz - 1)
                    acc += az[k + 1] * (u - x[at(nx, nz, i, j, k + 1)]);
                if (k > 0)
                    acc += az[k] * (u - x[at(nx, nz, i, j, k - 1)]);
                y[at(nx, nz, i, j, k)] = acc;
            }
}

/* z = M^{-1} r with M = blockdiag over columns of A_T (section 4.2, eq. (19)):
 * one independent tridiagonal solve per column by the Thomas algorithm
 * (forward elimination with an auxiliary vector, then back substitution, as
 * in the cited Numerical Recipes routine).  No pivoting: every column matrix
 * is strictly diagonally dominant when delta > 0.  Returns ORC_ERR_BREAKDOWN
 * if a pivot is zero. */
int orc_precond(int nx, int ny, int nz, double delta, const double *az,
                const double *ah, const double *r, double *z)
{
    double *gam = (double *)malloc(sizeof(double) * (size_t)(nz > 0 ? nz : 1));
    if (!gam)
        return ORC_ERR_INVALID;
    int status = ORC_OK;
    for (int j = 0; j < ny; ++j)
        for (int i = 0; i < nx; ++i) {
            double aT = orc_alpha_T(nx, ny, ah, i, j);
            /* row k: sub*z[k-1] + diag*z[k] + sup*z[k+1] = r[k] */
            double diag0 = delta + aT + (nz > 1 ? az[1] : 0.0);
            double bet = diag0;
            if (bet == 0.0) { status = ORC_ERR_BREAKDOWN; }
            z[at(nx, nz, i, j, 0)] = r[at(nx, nz, i, j, 0)] / bet;
            for (int k = 1; k < nz; ++k) {
                double sub = -az[k];
                double sup_prev = -az[k];           /* super-diagonal of row k-1 */
                double up = (k < nz - 1) ? az[k + 1] : 0.0;
                double diag = delta + aT + az[k] + up;
                gam[k] = sup_prev / bet;
                bet = diag - sub * gam[k];
                if (bet == 0.0) { status = ORC_ERR_BREAKDOWN; }
                z[at(nx, nz, i, j, k)] =
                    (r[at(nx, nz, i, j, k)] - sub * z[at(nx, nz, i, j, k - 1)]) / bet;
            }
            for (int k = nz - 2; k >= 0; --k)
                z[at(nx, nz, i, j, k)] -= gam[k + 1] * z[at(nx, nz, i, j, k + 1)];
        }
    free(gam);
    return status;
}

/* Wall time of the CG-step loop of the last orc_pcg call (timing only; used
 * to report the oracle's seconds per step without its set-up pass). */
static double g_loop_seconds = 0.0;
double orc_last_loop_seconds(void) { return g_loop_seconds; }

/* Wall time of the complete CG steps of the last orc_pcg call (each with its
 * preconditioner application: the last step of a call skips it) and their
 * number; timing only. */
static double g_full_seconds = 0.0;
static int g_full_steps = 0;
double orc_last_full_steps_seconds(int *steps)
{
    if (steps) *steps = g_full_steps;
    return g_full_seconds;
}

static double now_seconds(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* Neumaier-compensated dot product in memory order. */
double orc_dot(size_t n, const double *a, const double *b)
{
    double s = 0.0, c = 0.0;
    for (size_t l = 0; l < n; ++l) {
        double t = a[l] * b[l];
        double u = s + t;
        if (fabs(s) >= fabs(t))
            c += (s - u) + t;
        else
            c += (t - u) + s;
        s = u;
    }
    return s + c;
}

/* Preconditioned conjugate gradients, textbook form (section 4.1: Krylov
 * space of r_0, A-orthogonal search directions, left preconditioning with M).
 * Same iterates, in exact arithmetic, as the interleaved loop of section 4.3
 * (Algorithm 1), which only reorders the same updates into two grid passes.
 *
 *   x      in: x0, out: last iterate
 *   hist   out: ||r_k||_2 for k = 0..iters (length >= maxit+1)
 *   trace  optional (may be NULL): the first ntrace iterates of r, z and p are
 *          copied to trace_r/z/p[t*n ...] (t = 0..ntrace-1) for invariant checks
 * Returns ORC_OK, ORC_NOT_CONVERGED or ORC_ERR_BREAKDOWN.
 */
int orc_pcg(int nx, int ny, int nz, double delta, const double *az, const double *ah,
            const double *b, double *x, double tol, int maxit,
            double *hist, int *iters_out,
            int ntrace, double *trace_r, double *trace_z, double *trace_p)
{
    size_t n = (size_t)nx * ny * nz;
    double *r = (double *)malloc(sizeof(double) * n);
    double *z = (double *)malloc(sizeof(double) * n);
    double *p = (double *)malloc(sizeof(double) * n);
    double *q = (double *)malloc(sizeof(double) * n);
    int status = ORC_NOT_CONVERGED;
    int it = 0;
    double t_loop = 0.0;
    if (!r || !z || !p || !q) {
        status = ORC_ERR_INVALID;
        goto done;
    }
    /* r0 = b - A x0 */
    orc_apply_A(nx, ny, nz, delta, az, ah, x, q);
    for (size_t l = 0; l < n; ++l)
        r[l] = b[l] - q[l];
    double R0 = sqrt(orc_dot(n, r, r));
    hist[0] = R0;
    if (!isfinite(R0)) { status = ORC_ERR_BREAKDOWN; goto done; }
    if (R0 == 0.0) { status = ORC_OK; goto done; }

    if (orc_precond(nx, ny, nz, delta, az, ah, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
    memcpy(p, z, sizeof(double) * n);
    double rho = orc_dot(n, r, z);
    if (!(rho > 0.0) || !isfinite(rho)) { status = ORC_ERR_BREAKDOWN; goto done; }
    if (ntrace > 0) {
        memcpy(trace_r, r, sizeof(double) * n);
        memcpy(trace_z, z, sizeof(double) * n);
        memcpy(trace_p, p, sizeof(double) * n);
    }

    t_loop = now_seconds();
    g_loop_seconds = 0.0;
    g_full_seconds = 0.0;
    g_full_steps = 0;
    for (int k = 1; k <= maxit; ++k) {
        g_loop_seconds = now_seconds() - t_loop;
        g_full_seconds = g_loop_seconds;
        g_full_steps = k - 1;
        orc_apply_A(nx, ny, nz, delta, az, ah, p, q);
        double sigma = orc_dot(n, p, q);
        if (!(sigma > 0.0) || !isfinite(sigma)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double alpha = rho / sigma;
        for (size_t l = 0; l < n; ++l) x[l] += alpha * p[l];
        for (size_t l = 0; l < n; ++l) r[l] -= alpha * q[l];
        double R = sqrt(orc_dot(n, r, r));
        hist[k] = R;
        it = k;
        if (!isfinite(R)) { status = ORC_ERR_BREAKDOWN; goto done; }
        if (R == 0.0 || R / R0 < tol) { status = ORC_OK; goto done; }
        if (k == maxit) break;
        if (orc_precond(nx, ny, nz, delta, az, ah, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
        double rho_new = orc_dot(n, r, z);
        if (!(rho_new > 0.0) || !isfinite(rho_new)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double beta = rho_new / rho;
        rho = rho_new;
        for (size_t l = 0; l < n; ++l) p[l] = z[l] + beta * p[l];
        if (k < ntrace) {
            memcpy(trace_r + (size_t)k * n, r, sizeof(double) * n);
            memcpy(trace_z + (size_t)k * n, z, sizeof(double) * n);
            memcpy(trace_p + (size_t)k * n, p, sizeof(double) * n);
        }
    }
    status = ORC_NOT_CONVERGED;
done:
    if (it > 0) g_loop_seconds = now_seconds() - t_loop;
    if (iters_out) *iters_out = it;
    free(r); free(z); free(p); free(q);
    return status;
}

/* ======================================================================
 * Single precision (section 7 measures the solver in single and in double
 * precision).  Readings (also in the design notes):
 *  - fp32 PCG: every vector (x, r, z, p, q), the stencil, the Thomas solve
 *    and the vector updates in binary32, with the coefficients delta, alpha_z,
 *    alpha_h rounded to binary32 and the face means and alpha_T formed in
 *    binary32; the dot products <r,r>, <r,z>, <p,q> are sums of the exact
 *    products of the binary32 values, accumulated in binary64; the scalars
 *    alpha = rho/sigma, beta = rho'/rho and the stop test are binary64, and
 *    alpha, beta are rounded to binary32 where they scale a vector;
 *  - mixed: the binary64 PCG above whose preconditioner rounds r to binary32,
 *    solves the column systems in binary32 (as in fp32 PCG) and widens z
 *    exactly back to binary64.
 * Compiled with -ffp-contract=off: every float operation is rounded once. */

static float face_f32(const float *ah, size_t a, size_t b)
{
    return 0.5f * (ah[a] + ah[b]);
}

/* alpha_T in binary32 (section 3, eq. (7)), faces as in face_xp .. face_ym. */
static float alpha_T_f32(int nx, int ny, const float *ah, int i, int j)
{
    size_t c = (size_t)j * nx + i;
    float xp = face_f32(ah, c, (size_t)j * nx + (i + 1) % nx);
    float xm = face_f32(ah, c, (size_t)j * nx + (i + nx - 1) % nx);
    float yp = face_f32(ah, c, (size_t)((j + 1) % ny) * nx + i);
    float ym = face_f32(ah, c, (size_t)((j + ny - 1) % ny) * nx + i);
    return xp + xm + yp + ym;
}

/* y = A x in binary32 (section 4.2, eq. (18)); same terms and order as
 * orc_apply_A. */
void orc_apply_A_f32(int nx, int ny, int nz, float delta, const float *az,
                     const float *ah, const float *x, float *y)
{
    for (int j = 0; j < ny; ++j)
        for (int k = 0; k < nz; ++k)
            for (int i = 0; i < nx; ++i) {
                int ip = (i + 1) % nx, im = (i + nx - 1) % nx;
                int jp = (j + 1) % ny, jm = (j + ny - 1) % ny;
                size_t c = (size_t)j * nx + i;
                float u = x[at(nx, nz, i, j, k)];
                float acc = delta * u;
                acc += face_f32(ah, c, (size_t)j * nx + ip) * (u - x[at(nx, nz, ip, j, k)]);
                acc += face_f32(ah, c, (size_t)j * nx + im) * (u - x[at(nx, nz, im, j, k)]);
                acc += face_f32(ah, c, (size_t)jp * nx + i) * (u - x[at(nx, nz, i, jp, k)]);
                acc += face_f32(ah, c, (size_t)jm * nx + i) * (u - x[at(nx, nz, i, jm, k)]);
                if (k < nz - 1)
                    acc += az[k + 1] * (u - x[at(nx, nz, i, j, k + 1)]);
                if (k > 0)
                    acc += az[k] * (u - x[at(nx, nz, i, j, k - 1)]);
                y[at(nx, nz, i, j, k)] = acc;
            }
}

/* z = M^{-1} r in binary32 (section 4.2, eq. (19)): the Thomas algorithm of
 * orc_precond with every operation in binary32. */
int orc_precond_f32(int nx, int ny, int nz, float delta, const float *az,
                    const float *ah, const float *r, float *z)
{
    float *gam = (float *)malloc(sizeof(float) * (size_t)(nz > 0 ? nz : 1));
    if (!gam)
        return ORC_ERR_INVALID;
    int status = ORC_OK;
    for (int j = 0; j < ny; ++j)
        for (int i = 0; i < nx; ++i) {
            float aT = alpha_T_f32(nx, ny, ah, i, j);
            float bet = delta + aT + (nz > 1 ? az[1] : 0.0f);
            if (bet == 0.0f) { status = ORC_ERR_BREAKDOWN; }
            z[at(nx, nz, i, j, 0)] = r[at(nx, nz, i, j, 0)] / bet;
            for (int k = 1; k < nz; ++k) {
                float sub = -az[k];
                float sup_prev = -az[k];
                float up = (k < nz - 1) ? az[k + 1] : 0.0f;
                float diag = delta + aT + az[k] + up;
                gam[k] = sup_prev / bet;
                bet = diag - sub * gam[k];
                if (bet == 0.0f) { status = ORC_ERR_BREAKDOWN; }
                z[at(nx, nz, i, j, k)] =
                    (r[at(nx, nz, i, j, k)] - sub * z[at(nx, nz, i, j, k - 1)]) / bet;
            }
            for (int k = nz - 2; k >= 0; --k)
                z[at(nx, nz, i, j, k)] -= gam[k + 1] * z[at(nx, nz, i, j, k + 1)];
        }
    free(gam);
    return status;
}

/* <a,b> of binary32 vectors: exact products, Neumaier-compensated binary64 sum. */
double orc_dot_f32(size_t n, const float *a, const float *b)
{
    double s = 0.0, c = 0.0;
    for (size_t l = 0; l < n; ++l) {
        double t = (double)a[l] * (double)b[l];
        double u = s + t;
        if (fabs(s) >= fabs(t))
            c += (s - u) + t;
        else
            c += (t - u) + s;
        s = u;
    }
    return s + c;
}

/* Coefficients rounded to binary32 (az: nz+1 faces, ah: nx*ny). */
static int round_coeffs(int nx, int ny, int nz, const double *az, const double *ah,
                        float **az32, float **ah32)
{
    size_t ncol = (size_t)nx * ny;
    *az32 = (float *)malloc(sizeof(float) * (size_t)(nz + 1));
    *ah32 = (float *)malloc(sizeof(float) * ncol);
    if (!*az32 || !*ah32)
        return ORC_ERR_INVALID;
    for (int f = 0; f <= nz; ++f) (*az32)[f] = (float)az[f];
    for (size_t c = 0; c < ncol; ++c) (*ah32)[c] = (float)ah[c];
    return ORC_OK;
}

/* PCG in binary32 (the textbook loop of orc_pcg with the readings above). */
int orc_pcg_f32(int nx, int ny, int nz, double delta, const double *az, const double *ah,
                const float *b, float *x, double tol, int maxit, double *hist, int *iters_out)
{
    size_t n = (size_t)nx * ny * nz;
    float *r = (float *)malloc(sizeof(float) * n);
    float *z = (float *)malloc(sizeof(float) * n);
    float *p = (float *)malloc(sizeof(float) * n);
    float *q = (float *)malloc(sizeof(float) * n);
    float *az32 = NULL, *ah32 = NULL;
    int status = ORC_NOT_CONVERGED, it = 0;
    const float d32 = (float)delta;
    if (!r || !z || !p || !q || round_coeffs(nx, ny, nz, az, ah, &az32, &ah32) != ORC_OK) {
        status = ORC_ERR_INVALID;
        goto done;
    }
    orc_apply_A_f32(nx, ny, nz, d32, az32, ah32, x, q);
    for (size_t l = 0; l < n; ++l)
        r[l] = b[l] - q[l];
    double R0 = sqrt(orc_dot_f32(n, r, r));
    hist[0] = R0;
    if (!isfinite(R0)) { status = ORC_ERR_BREAKDOWN; goto done; }
    if (R0 == 0.0) { status = ORC_OK; goto done; }
    if (orc_precond_f32(nx, ny, nz, d32, az32, ah32, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
    memcpy(p, z, sizeof(float) * n);
    double rho = orc_dot_f32(n, r, z);
    if (!(rho > 0.0) || !isfinite(rho)) { status = ORC_ERR_BREAKDOWN; goto done; }
    for (int k = 1; k <= maxit; ++k) {
        orc_apply_A_f32(nx, ny, nz, d32, az32, ah32, p, q);
        double sigma = orc_dot_f32(n, p, q);
        if (!(sigma > 0.0) || !isfinite(sigma)) { status = ORC_ERR_BREAKDOWN; goto done; }
        const float alpha = (float)(rho / sigma);
        for (size_t l = 0; l < n; ++l) x[l] += alpha * p[l];
        for (size_t l = 0; l < n; ++l) r[l] -= alpha * q[l];
        double R = sqrt(orc_dot_f32(n, r, r));
        hist[k] = R;
        it = k;
        if (!isfinite(R)) { status = ORC_ERR_BREAKDOWN; goto done; }
        if (R == 0.0 || R / R0 < tol) { status = ORC_OK; goto done; }
        if (k == maxit) break;
        if (orc_precond_f32(nx, ny, nz, d32, az32, ah32, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
        double rho_new = orc_dot_f32(n, r, z);
        if (!(rho_new > 0.0) || !isfinite(rho_new)) { status = ORC_ERR_BREAKDOWN; goto done; }
        const float beta = (float)(rho_new / rho);
        rho = rho_new;
        for (size_t l = 0; l < n; ++l) p[l] = z[l] + beta * p[l];
    }
    status = ORC_NOT_CONVERGED;
done:
    if (iters_out) *iters_out = it;
    free(r); free(z); free(p); free(q); free(az32); free(ah32);
    return status;
}

/* PCG in binary64 with the preconditioner applied in binary32 (readings
 * above): the loop of orc_pcg, z = widen(M32^{-1} round32(r)). */
int orc_pcg_mixed(int nx, int ny, int nz, double delta, const double *az, const double *ah,
                  const double *b, double *x, double tol, int maxit, double *hist, int *iters_out)
{
    size_t n = (size_t)nx * ny * nz;
    double *r = (double *)malloc(sizeof(double) * n);
    double *z = (double *)malloc(sizeof(double) * n);
    double *p = (double *)malloc(sizeof(double) * n);
    double *q = (double *)malloc(sizeof(double) * n);
    float *r32 = (float *)malloc(sizeof(float) * n);
    float *z32 = (float *)malloc(sizeof(float) * n);
    float *az32 = NULL, *ah32 = NULL;
    int status = ORC_NOT_CONVERGED, it = 0;
    const float d32 = (float)delta;
    if (!r || !z || !p || !q || !r32 || !z32 || round_coeffs(nx, ny, nz, az, ah, &az32, &ah32) != ORC_OK) {
        status = ORC_ERR_INVALID;
        goto done;
    }
    orc_apply_A(nx, ny, nz, delta, az, ah, x, q);
    for (size_t l = 0; l < n; ++l)
        r[l] = b[l] - q[l];
    double R0 = sqrt(orc_dot(n, r, r));
    hist[0] = R0;
    if (!isfinite(R0)) { status = ORC_ERR_BREAKDOWN; goto done; }
    if (R0 == 0.0) { status = ORC_OK; goto done; }
    for (size_t l = 0; l < n; ++l) r32[l] = (float)r[l];
    if (orc_precond_f32(nx, ny, nz, d32, az32, ah32, r32, z32) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
    for (size_t l = 0; l < n; ++l) z[l] = (double)z32[l];
    memcpy(p, z, sizeof(double) * n);
    double rho = orc_dot(n, r, z);
    if (!(rho > 0.0) || !isfinite(rho)) { status = ORC_ERR_BREAKDOWN; goto done; }
    for (int k = 1; k <= maxit; ++k) {
        orc_apply_A(nx, ny, nz, delta, az, ah, p, q);
        double sigma = orc_dot(n, p, q);
        if (!(sigma > 0.0) || !isfinite(sigma)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double alpha = rho / sigma;
        for (size_t l = 0; l < n; ++l) x[l] += alpha * p[l];
        for (size_t l = 0; l < n; ++l) r[l] -= alpha * q[l];
        double R = sqrt(orc_dot(n, r, r));
        hist[k] = R;
        it = k;
        if (!isfinite(R)) { status = ORC_ERR_BREAKDOWN; goto done; }
        if (R == 0.0 || R / R0 < tol) { status = ORC_OK; goto done; }
        if (k == maxit) break;
        for (size_t l = 0; l < n; ++l) r32[l] = (float)r[l];
        if (orc_precond_f32(nx, ny, nz, d32, az32, ah32, r32, z32) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
        for (size_t l = 0; l < n; ++l) z[l] = (double)z32[l];
        double rho_new = orc_dot(n, r, z);
        if (!(rho_new > 0.0) || !isfinite(rho_new)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double beta = rho_new / rho;
        rho = rho_new;
        for (size_t l = 0; l < n; ++l) p[l] = z[l] + beta * p[l];
    }
    status = ORC_NOT_CONVERGED;
done:
    if (iters_out) *iters_out = it;
    free(r); free(z); free(p); free(q); free(r32); free(z32); free(az32); free(ah32);
    return status;
}

/* ======================================================================
 * General tensor-product coefficients (section 3, eqs. (5)-(8)), read with
 * the signs of the symmetric positive definite operator as above:
 *   (A u)_{T,k} = |T| a_k u_{T,k}
 *               + d_k sum_{T' in N(T)} alpha_{T,T'} (u_{T,k} - u_{T',k})
 *               + |T| ( beta_{k+1} (u_{T,k} - u_{T,k+1}) + beta_k (u_{T,k} - u_{T,k-1}) )
 * with the tridiagonal column block A_T = |T| diag(a) + alpha_T diag(d) +
 * |T| (vertical second difference with face coefficients beta), eq. (8), the
 * diagonal horizontal blocks A_{T,T'} = -alpha_{T,T'} diag(d), eq. (6), and
 * alpha_T = sum of alpha_{T,T'}, eq. (7).  Faces 0 and nz carry no flux
 * (beta_0 = beta_nz = 0).  On the logically rectangular periodic grid the
 * edge coefficients are two fields: ax[j*nx + i] between (i, j) and
 * (i+1 mod nx, j), ay[j*nx + i] between (i, j) and (i, j+1 mod ny).  The
 * preconditioner keeps A_T and drops the A_{T,T'} (section 4.2). */

static double gen_alpha_T(int nx, int ny, const double *ax, const double *ay, int i, int j)
{
    int im = (i + nx - 1) % nx, jm = (j + ny - 1) % ny;
    return ax[(size_t)j * nx + i] + ax[(size_t)j * nx + im]
         + ay[(size_t)j * nx + i] + ay[(size_t)jm * nx + i];
}

/* y = A x for the general coefficients (eqs. (5)-(8)). */
void orc_apply_A_gen(int nx, int ny, int nz, const double *a, const double *d, const double *beta,
                     const double *area, const double *ax, const double *ay,
                     const double *x, double *y)
{
    for (int j = 0; j < ny; ++j)
        for (int k = 0; k < nz; ++k)
            for (int i = 0; i < nx; ++i) {
                int ip = (i + 1) % nx, im = (i + nx - 1) % nx;
                int jp = (j + 1) % ny, jm = (j + ny - 1) % ny;
                double T = area[(size_t)j * nx + i];
                double u = x[at(nx, nz, i, j, k)];
                double acc = T * a[k] * u;
                double hor = ax[(size_t)j * nx + i] * (u - x[at(nx, nz, ip, j, k)]);
                hor += ax[(size_t)j * nx + im] * (u - x[at(nx, nz, im, j, k)]);
                hor += ay[(size_t)j * nx + i] * (u - x[at(nx, nz, i, jp, k)]);
                hor += ay[(size_t)jm * nx + i] * (u - x[at(nx, nz, i, jm, k)]);
                acc += d[k] * hor;
                if (k < nz - 1)
                    acc += T * beta[k + 1] * (u - x[at(nx, nz, i, j, k + 1)]);
                if (k > 0)
                    acc += T * beta[k] * (u - x[at(nx, nz, i, j, k - 1)]);
                y[at(nx, nz, i, j, k)] = acc;
            }
}

/* z = M^{-1} r, M = blockdiag(A_T) for the general coefficients: one Thomas
 * solve per column (eq. (19)); diagonal |T| a_k + alpha_T d_k + |T| (beta_k +
 * beta_{k+1}), off-diagonals -|T| beta. */
int orc_precond_gen(int nx, int ny, int nz, const double *a, const double *d, const double *beta,
                    const double *area, const double *ax, const double *ay,
                    const double *r, double *z)
{
    double *gam = (double *)malloc(sizeof(double) * (size_t)(nz > 0 ? nz : 1));
    if (!gam)
        return ORC_ERR_INVALID;
    int status = ORC_OK;
    for (int j = 0; j < ny; ++j)
        for (int i = 0; i < nx; ++i) {
            double aT = gen_alpha_T(nx, ny, ax, ay, i, j);
            double T = area[(size_t)j * nx + i];
            double up0 = (nz > 1) ? T * beta[1] : 0.0;
            double bet = T * a[0] + aT * d[0] + up0;
            if (bet == 0.0) { status = ORC_ERR_BREAKDOWN; }
            z[at(nx, nz, i, j, 0)] = r[at(nx, nz, i, j, 0)] / bet;
            for (int k = 1; k < nz; ++k) {
                double sub = -T * beta[k];
                double sup_prev = -T * beta[k];
                double up = (k < nz - 1) ? T * beta[k + 1] : 0.0;
                double diag = T * a[k] + aT * d[k] + T * beta[k] + up;
                gam[k] = sup_prev / bet;
                bet = diag - sub * gam[k];
                if (bet == 0.0) { status = ORC_ERR_BREAKDOWN; }
                z[at(nx, nz, i, j, k)] =
                    (r[at(nx, nz, i, j, k)] - sub * z[at(nx, nz, i, j, k - 1)]) / bet;
            }
            for (int k = nz - 2; k >= 0; --k)
                z[at(nx, nz, i, j, k)] -= gam[k + 1] * z[at(nx, nz, i, j, k + 1)];
        }
    free(gam);
    return status;
}

/* Textbook PCG (as orc_pcg) with the general operator and preconditioner. */
int orc_pcg_gen(int nx, int ny, int nz, const double *a, const double *d, const double *beta,
                const double *area, const double *ax, const double *ay,
                const double *b, double *x, double tol, int maxit, double *hist, int *iters_out)
{
    size_t n = (size_t)nx * ny * nz;
    double *r = (double *)malloc(sizeof(double) * n);
    double *z = (double *)malloc(sizeof(double) * n);
    double *p = (double *)malloc(sizeof(double) * n);
    double *q = (double *)malloc(sizeof(double) * n);
    int status = ORC_NOT_CONVERGED, it = 0;
    if (!r || !z || !p || !q) {
        status = ORC_ERR_INVALID;
        goto done;
    }
    orc_apply_A_gen(nx, ny, nz, a, d, beta, area, ax, ay, x, q);
    for (size_t l = 0; l < n; ++l)
        r[l] = b[l] - q[l];
    double R0 = sqrt(orc_dot(n, r, r));
    hist[0] = R0;
    if (!isfinite(R0)) { status = ORC_ERR_BREAKDOWN; goto done; }
    if (R0 == 0.0) { status = ORC_OK; goto done; }
    if (orc_precond_gen(nx, ny, nz, a, d, beta, area, ax, ay, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
    memcpy(p, z, sizeof(double) * n);
    double rho = orc_dot(n, r, z);
    if (!(rho > 0.0) || !isfinite(rho)) { status = ORC_ERR_BREAKDOWN; goto done; }
    for (int k = 1; k <= maxit; ++k) {
        orc_apply_A_gen(nx, ny, nz, a, d, beta, area, ax, ay, p, q);
        double sigma = orc_dot(n, p, q);
        if (!(sigma > 0.0) || !isfinite(sigma)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double alpha = rho / sigma;
        for (size_t l = 0; l < n; ++l) x[l] += alpha * p[l];
        for (size_t l = 0; l < n; ++l) r[l] -= alpha * q[l];
        double R = sqrt(orc_dot(n, r, r));
        hist[k] = R;
        it = k;
        if (!isfinite(R)) { status = ORC_ERR_BREAKDOWN; goto done; }
        if (R == 0.0 || R / R0 < tol) { status = ORC_OK; goto done; }
        if (k == maxit) break;
        if (orc_precond_gen(nx, ny, nz, a, d, beta, area, ax, ay, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
        double rho_new = orc_dot(n, r, z);
        if (!(rho_new > 0.0) || !isfinite(rho_new)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double beta_cg = rho_new / rho;
        rho = rho_new;
        for (size_t l = 0; l < n; ++l) p[l] = z[l] + beta_cg * p[l];
    }
    status = ORC_NOT_CONVERGED;
done:
    if (iters_out) *iters_out = it;
    free(r); free(z); free(p); free(q);
    return status;
}

/* ======================================================================
 * Tensor-product multigrid as the preconditioner of CG (section 2 names
 * geometric multigrid with the vertical line relaxation as the faster CPU
 * solver, and section 8 plans it on the GPU; the pages give no intergrid
 * operators).  Readings (also in the design notes):
 *  - levels: level 0 is the grid; the next level halves nx where nx is even
 *    and > 1 and ny where ny is even and > 1, and keeps nz (horizontal
 *    semi-coarsening: the strong vertical coupling is left to the smoother);
 *    the hierarchy ends at a single column, at a level where neither
 *    dimension can be halved, or after max_levels levels (0 = no limit);
 *  - transfers: piecewise-constant prolongation P (a fine column takes its
 *    coarse parent's value at the same level) and restriction P^T (the sum
 *    over the children);
 *  - coarse operator: the Galerkin product P^T A P.  It has the general
 *    form again: a coarse column's |T| is the sum of its children's, its
 *    edge to a coarse neighbour is the sum of the fine edges crossing that
 *    coarse edge, a, d and beta are unchanged, and the edges of a dimension
 *    of size 1 are zero (they would couple a column with itself, which
 *    cancels in P^T A P);
 *  - smoother: damped block Jacobi with the column blocks (the line
 *    relaxation; M of the PCG preconditioner on that level):
 *    z <- z + omega M^{-1} (f - A z);
 *  - cycle: V(nu, nu): nu sweeps from z = 0, the coarse correction, nu
 *    sweeps; on the coarsest level z = M^{-1} f when it is one column (exact,
 *    its edges being zero), else coarse_sweeps sweeps from z = 0;
 *  - coarsest sweeps: with coarse_lo = 0 the damped sweeps above; with
 *    coarse_lo > 0 the same sweeps accelerated by Chebyshev polynomials on
 *    the interval [coarse_lo, 2] (Chebyshev semi-iteration, Golub and Varga
 *    1961; Saad, Iterative Methods for Sparse Linear Systems, 2nd ed., 12.3).
 *    The eigenvalues of M^{-1} A lie in (0, 2) here (M + N is diagonally
 *    dominant when A = M - N, N >= 0 holding the couplings between
 *    columns), so with the upper end 2 the result is q(M^{-1} A) M^{-1} f
 *    for a polynomial q that is positive on the whole spectrum, whatever
 *    coarse_lo: a symmetric positive definite coarse solve.
 * ====================================================================== */

/* Coarsening factors of an nx x ny level (1 or 2 each); 0 if neither
 * dimension can be halved. */
static int mg_factors(int nx, int ny, int *fx, int *fy)
{
    *fx = (nx > 1 && nx % 2 == 0) ? 2 : 1;
    *fy = (ny > 1 && ny % 2 == 0) ? 2 : 1;
    return (*fx > 1 || *fy > 1);
}

/* One Galerkin coarsening step (readings above).  The coarse arrays hold
 * (nx/fx)*(ny/fy) entries.  Sums run over the children in the order
 * (row b outer, column a inner).  Returns 1 and the coarse sizes, or 0 when
 * the level cannot be coarsened. */
int orc_mg_coarsen(int nx, int ny, const double *area, const double *ax, const double *ay,
                   int *ncx_out, int *ncy_out, double *carea, double *cax, double *cay)
{
    int fx, fy;
    if (!mg_factors(nx, ny, &fx, &fy))
        return 0;
    int ncx = nx / fx, ncy = ny / fy;
    for (int J = 0; J < ncy; ++J)
        for (int I = 0; I < ncx; ++I) {
            double sa = 0.0, sx = 0.0, sy = 0.0;
            for (int b = 0; b < fy; ++b)
                for (int a = 0; a < fx; ++a)
                    sa += area[(size_t)(fy * J + b) * nx + (fx * I + a)];
            /* fine x-edges between columns fx*I+fx-1 and fx*I+fx (mod nx) of
             * the children rows cross the coarse edge between I and I+1 */
            for (int b = 0; b < fy; ++b)
                sx += ax[(size_t)(fy * J + b) * nx + (fx * I + fx - 1)];
            /* fine y-edges between rows fy*J+fy-1 and fy*J+fy (mod ny) */
            for (int a = 0; a < fx; ++a)
                sy += ay[(size_t)(fy * J + fy - 1) * nx + (fx * I + a)];
            carea[(size_t)J * ncx + I] = sa;
            cax[(size_t)J * ncx + I] = (ncx == 1) ? 0.0 : sx;
            cay[(size_t)J * ncx + I] = (ncy == 1) ? 0.0 : sy;
        }
    *ncx_out = ncx;
    *ncy_out = ncy;
    return 1;
}

typedef struct {
    int nx, ny;
    double *area, *ax, *ay;    /* the level's coefficients (level 0: the caller's) */
    double *f, *z;             /* right-hand side and correction (levels >= 1) */
    double *t, *y;             /* residual and M^{-1} residual */
    int owns;
} mg_level;

static void mg_free(mg_level *lv, int nlev)
{
    if (!lv)
        return;
    for (int l = 0; l < nlev; ++l) {
        if (lv[l].owns) {
            free(lv[l].area); free(lv[l].ax); free(lv[l].ay);
        }
        free(lv[l].f); free(lv[l].z); free(lv[l].t); free(lv[l].y);
    }
    free(lv);
}

/* Number of levels for an nx x ny grid (readings above). */
int orc_mg_num_levels(int nx, int ny, int max_levels)
{
    int n = 1, fx, fy;
    while ((max_levels <= 0 || n < max_levels) && nx * ny > 1 && mg_factors(nx, ny, &fx, &fy)) {
        nx /= fx;
        ny /= fy;
        ++n;
    }
    return n;
}

static mg_level *mg_build(int nx, int ny, int nz, const double *area, const double *ax,
                          const double *ay, int max_levels, int *nlev_out)
{
    int nlev = orc_mg_num_levels(nx, ny, max_levels);
    mg_level *lv = (mg_level *)calloc((size_t)nlev, sizeof(mg_level));
    if (!lv)
        return NULL;
    lv[0].nx = nx;
    lv[0].ny = ny;
    lv[0].area = (double *)area;
    lv[0].ax = (double *)ax;
    lv[0].ay = (double *)ay;
    for (int l = 0; l < nlev; ++l) {
        size_t ncol = (size_t)lv[l].nx * lv[l].ny, n = ncol * nz;
        lv[l].t = (double *)malloc(sizeof(double) * n);
        lv[l].y = (double *)malloc(sizeof(double) * n);
        if (l > 0) {
            lv[l].f = (double *)malloc(sizeof(double) * n);
            lv[l].z = (double *)malloc(sizeof(double) * n);
        }
        if (!lv[l].t || !lv[l].y || (l > 0 && (!lv[l].f || !lv[l].z))) {
            mg_free(lv, nlev);
            return NULL;
        }
        if (l + 1 < nlev) {
            mg_level *c = &lv[l + 1];
            c->owns = 1;
            c->area = (double *)malloc(sizeof(double) * ncol);
            c->ax = (double *)malloc(sizeof(double) * ncol);
            c->ay = (double *)malloc(sizeof(double) * ncol);
            if (!c->area || !c->ax || !c->ay) {
                mg_free(lv, nlev);
                return NULL;
            }
            orc_mg_coarsen(lv[l].nx, lv[l].ny, lv[l].area, lv[l].ax, lv[l].ay, &c->nx, &c->ny,
                           c->area, c->ax, c->ay);
        }
    }
    *nlev_out = nlev;
    return lv;
}

/* One smoothing sweep on level L: z <- z + omega M^{-1} (f - A z). */
static int mg_smooth(const mg_level *L, int nz, const double *a, const double *d, const double *beta,
                     double omega, const double *f, double *z)
{
    size_t n = (size_t)L->nx * L->ny * nz;
    orc_apply_A_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, z, L->t);
    for (size_t l = 0; l < n; ++l)
        L->t[l] = f[l] - L->t[l];
    if (orc_precond_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, L->t, L->y) != ORC_OK)
        return ORC_ERR_BREAKDOWN;
    for (size_t l = 0; l < n; ++l)
        z[l] += omega * L->y[l];
    return ORC_OK;
}

/* The coarsest level with coarse_lo > 0: m = coarse_sweeps steps of the
 * Chebyshev semi-iteration for M^{-1} A z = M^{-1} f from z_0 = 0 on the
 * interval [lo, hi] = [coarse_lo, 2] (readings above).  With
 * theta = (hi + lo) / 2, delta = (hi - lo) / 2, s = theta / delta:
 *   z_1 = M^{-1} f / theta,  rho_0 = 1 / s,
 *   rho_k = 1 / (2 s - rho_{k-1}),
 *   z_{k+1} = z_k + rho_k rho_{k-1} (z_k - z_{k-1})
 *             + (2 rho_k / delta) M^{-1} (f - A z_k),   k = 1 .. m-1.
 * The residual f - A z_k is formed afresh at every step. */
static int mg_chebyshev(const mg_level *L, int nz, const double *a, const double *d, const double *beta,
                        int m, double lo, const double *f, double *z)
{
    const size_t n = (size_t)L->nx * L->ny * nz;
    const double hi = 2.0;
    const double theta = 0.5 * (hi + lo), delta = 0.5 * (hi - lo), s = theta / delta;
    if (orc_precond_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, f, L->y) != ORC_OK)
        return ORC_ERR_BREAKDOWN;
    for (size_t l = 0; l < n; ++l)
        z[l] = L->y[l] / theta;
    if (m < 2)
        return ORC_OK;
    double *zold = (double *)calloc(n, sizeof(double));   /* z_{k-1}; z_0 = 0 */
    double *znew = (double *)malloc(n * sizeof(double));
    if (!zold || !znew) { free(zold); free(znew); return ORC_ERR_INVALID; }
    int st = ORC_OK;
    double rho_prev = 1.0 / s;
    for (int k = 1; k < m; ++k) {
        const double rho = 1.0 / (2.0 * s - rho_prev);
        orc_apply_A_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, z, L->t);
        for (size_t l = 0; l < n; ++l)
            L->t[l] = f[l] - L->t[l];
        if (orc_precond_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, L->t, L->y) != ORC_OK) {
            st = ORC_ERR_BREAKDOWN;
            break;
        }
        for (size_t l = 0; l < n; ++l)
            znew[l] = (z[l] + (rho * rho_prev) * (z[l] - zold[l])) + (2.0 * rho / delta) * L->y[l];
        memcpy(zold, z, n * sizeof(double));
        memcpy(z, znew, n * sizeof(double));
        rho_prev = rho;
    }
    free(zold);
    free(znew);
    return st;
}

/* z = B_l f: one V(nu, nu) cycle from level l down (readings above). */
static int mg_vcycle(const mg_level *lv, int nlev, int l, int nz, const double *a, const double *d,
                     const double *beta, int nu, double omega, int coarse_sweeps, double coarse_lo,
                     const double *f, double *z)
{
    const mg_level *L = &lv[l];
    int nx = L->nx, ny = L->ny;
    size_t n = (size_t)nx * ny * nz;
    memset(z, 0, sizeof(double) * n);
    if (l == nlev - 1) {
        if (nx * ny == 1)
            return orc_precond_gen(nx, ny, nz, a, d, beta, L->area, L->ax, L->ay, f, z);
        if (coarse_lo > 0.0)
            return mg_chebyshev(L, nz, a, d, beta, coarse_sweeps, coarse_lo, f, z);
        for (int s = 0; s < coarse_sweeps; ++s)
            if (mg_smooth(L, nz, a, d, beta, omega, f, z) != ORC_OK)
                return ORC_ERR_BREAKDOWN;
        return ORC_OK;
    }
    for (int s = 0; s < nu; ++s)
        if (mg_smooth(L, nz, a, d, beta, omega, f, z) != ORC_OK)
            return ORC_ERR_BREAKDOWN;
    /* coarse right-hand side P^T (f - A z) */
    const mg_level *C = &lv[l + 1];
    int fx = nx / C->nx, fy = ny / C->ny;
    orc_apply_A_gen(nx, ny, nz, a, d, beta, L->area, L->ax, L->ay, z, L->t);
    for (size_t q = 0; q < n; ++q)
        L->t[q] = f[q] - L->t[q];
    memset(C->f, 0, sizeof(double) * (size_t)C->nx * C->ny * nz);
    for (int j = 0; j < ny; ++j)
        for (int k = 0; k < nz; ++k)
            for (int i = 0; i < nx; ++i)
                C->f[at(C->nx, nz, i / fx, j / fy, k)] += L->t[at(nx, nz, i, j, k)];
    if (mg_vcycle(lv, nlev, l + 1, nz, a, d, beta, nu, omega, coarse_sweeps, coarse_lo, C->f, C->z) != ORC_OK)
        return ORC_ERR_BREAKDOWN;
    /* z += P z_c */
    for (int j = 0; j < ny; ++j)
        for (int k = 0; k < nz; ++k)
            for (int i = 0; i < nx; ++i)
                z[at(nx, nz, i, j, k)] += C->z[at(C->nx, nz, i / fx, j / fy, k)];
    for (int s = 0; s < nu; ++s)
        if (mg_smooth(L, nz, a, d, beta, omega, f, z) != ORC_OK)
            return ORC_ERR_BREAKDOWN;
    return ORC_OK;
}

/* z = B r, one V-cycle of the hierarchy of the general operator. */
int orc_mg_vcycle(int nx, int ny, int nz, const double *a, const double *d, const double *beta,
                  const double *area, const double *ax, const double *ay, int nu, double omega,
                  int max_levels, int coarse_sweeps, double coarse_lo, const double *r, double *z)
{
    int nlev = 0;
    mg_level *lv = mg_build(nx, ny, nz, area, ax, ay, max_levels, &nlev);
    if (!lv)
        return ORC_ERR_INVALID;
    int st = mg_vcycle(lv, nlev, 0, nz, a, d, beta, nu, omega, coarse_sweeps, coarse_lo, r, z);
    mg_free(lv, nlev);
    return st;
}

/* Textbook PCG (as orc_pcg_gen) with one V-cycle as the preconditioner. */
int orc_pcg_mg(int nx, int ny, int nz, const double *a, const double *d, const double *beta,
               const double *area, const double *ax, const double *ay, int nu, double omega,
               int max_levels, int coarse_sweeps, double coarse_lo, const double *b, double *x, double tol, int maxit,
               double *hist, int *iters_out)
{
    size_t n = (size_t)nx * ny * nz;
    int nlev = 0;
    mg_level *lv = mg_build(nx, ny, nz, area, ax, ay, max_levels, &nlev);
    double *r = (double *)malloc(sizeof(double) * n);
    double *z = (double *)malloc(sizeof(double) * n);
    double *p = (double *)malloc(sizeof(double) * n);
    double *q = (double *)malloc(sizeof(double) * n);
    int status = ORC_NOT_CONVERGED, it = 0;
    double t0 = now_seconds();
    if (!lv || !r || !z || !p || !q) {
        status = ORC_ERR_INVALID;
        goto done;
    }
    orc_apply_A_gen(nx, ny, nz, a, d, beta, area, ax, ay, x, q);
    for (size_t l = 0; l < n; ++l)
        r[l] = b[l] - q[l];
    double R0 = sqrt(orc_dot(n, r, r));
    hist[0] = R0;
    if (!isfinite(R0)) { status = ORC_ERR_BREAKDOWN; goto done; }
    if (R0 == 0.0) { status = ORC_OK; goto done; }
    if (mg_vcycle(lv, nlev, 0, nz, a, d, beta, nu, omega, coarse_sweeps, coarse_lo, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
    memcpy(p, z, sizeof(double) * n);
    double rho = orc_dot(n, r, z);
    if (!(rho > 0.0) || !isfinite(rho)) { status = ORC_ERR_BREAKDOWN; goto done; }
    for (int k = 1; k <= maxit; ++k) {
        orc_apply_A_gen(nx, ny, nz, a, d, beta, area, ax, ay, p, q);
        double sigma = orc_dot(n, p, q);
        if (!(sigma > 0.0) || !isfinite(sigma)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double alpha = rho / sigma;
        for (size_t l = 0; l < n; ++l) x[l] += alpha * p[l];
        for (size_t l = 0; l < n; ++l) r[l] -= alpha * q[l];
        double R = sqrt(orc_dot(n, r, r));
        hist[k] = R;
        it = k;
        if (!isfinite(R)) { status = ORC_ERR_BREAKDOWN; goto done; }
        if (R == 0.0 || R / R0 < tol) { status = ORC_OK; goto done; }
        if (k == maxit) break;
        if (mg_vcycle(lv, nlev, 0, nz, a, d, beta, nu, omega, coarse_sweeps, coarse_lo, r, z) != ORC_OK) { status = ORC_ERR_BREAKDOWN; goto done; }
        double rho_new = orc_dot(n, r, z);
        if (!(rho_new > 0.0) || !isfinite(rho_new)) { status = ORC_ERR_BREAKDOWN; goto done; }
        double beta_cg = rho_new / rho;
        rho = rho_new;
        for (size_t l = 0; l < n; ++l) p[l] = z[l] + beta_cg * p[l];
    }
    status = ORC_NOT_CONVERGED;
done:
    g_loop_seconds = now_seconds() - t0;
    if (iters_out) *iters_out = it;
    mg_free(lv, nlev);
    free(r); free(z); free(p); free(q);
    return status;
}
