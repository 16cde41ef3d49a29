// Device kernels of the matrix-free PCG solver for gfx950 (MI355X).
//
// Method: E. Mueller, X. Guo, R. Scheichl, S. Shi, "Matrix-free GPU
// implementation of a preconditioned conjugate gradient solver for
// anisotropic elliptic PDEs" (2013).
//
// Field layout l = i + nx*(k + nz*j) (section 6.1, eq. (22)): a wave-wide
// access to consecutive i at fixed (j, k) is contiguous.
//
// Two work decompositions:
//  * column passes (the Thomas solve): a workgroup owns C consecutive columns
//    of one row j and all their levels; thread (c, s) owns column c and the
//    vertical segment k in [s*L, min(nz, (s+1)*L)).
//  * sweep passes (stencil and vector updates): a workgroup owns 64
//    consecutive columns of one row j over Ws*Ls consecutive levels; each
//    wave sweeps Ls levels with one column per lane, so per-column work (the
//    face coefficients) is done once per Ls points.
// Hardware workgroup ids are renumbered so that each of the 8 XCDs (which
// receive workgroups round-robin) walks one contiguous run of tiles, and tiles
// are numbered so that the neighbours a tile reads are read by workgroups of
// the same XCD at about the same time (served by its L2):
//  * column passes: the i-tiles are grouped in strips of csg tiles (one strip
//    per XCD); within a strip the i-tile is faster than j;
//  * sweep passes: the i-tiles are grouped in strips of sg tiles (one strip
//    per XCD); within a strip the k-tile is fastest, then the i-tile, then j.
//    The j-1 / j+1, k-1 / k+1 and (inside the strip) i-1 / i+1 neighbours of
//    a tile are read within a few tiles of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mfpcg {

constexpr int kWave = 64;
constexpr int kMaxThreads = 1024;
constexpr int kXcds = 8;
constexpr int kCus = 256;   // compute units (32 per XCD)

// Operator and launch geometry, passed by value to every kernel.
struct Op {
    int nx, ny, nz;
    int L, P, C, ntc;      // column passes: segment length, segments, columns per tile, tiles along i
    int Ls, Ws, nkt;       // sweep passes: levels per wave, waves per tile, tiles along k
    int ntx, sg;           // sweep passes: 64-column tiles along i, tiles per i-strip
    int csg;               // column passes: tiles per i-strip
    // The operator in the general tensor-product form of section 3, eqs.
    // (5)-(8) (symmetric positive definite signs):
    //   (A u)_{T,k} = |T| a_k u + d_k sum_{T'} alpha_{T,T'} (u - u_{T'})
    //               + |T| (beta_{k+1} (u - u_{k+1}) + beta_k (u - u_{k-1}))
    const double *az;      // nz+1 vertical face coefficients beta (faces 0, nz are 0)
    const double *lev_a;   // nz: zero-order coefficient a_k
    const double *lev_d;   // nz: factor d_k of the horizontal couplings
    const double *area;    // ny*nx: |T| per column
    const double *ex;      // ny*nx: edge coefficient between (i, j) and (i+1 mod nx, j)
    const double *ey;      // ny*nx: edge coefficient between (i, j) and (i, j+1 mod ny)
    const double *phib;    // Thomas multiplier phi at the boundaries of a table's segments
    int jt;                // sweep passes: rows per tile (1: the waves split the levels; > 1:
                           //   wave w takes row j0 + w, Ws = jt, nkt = nz / Ls)
    int pst;               // segments of the multiplier table per column segment: segment s
                           //   starts at table boundary s*pst (a table of shorter segments
                           //   holds every boundary of a longer segmentation too)
};

// Scalar state of one solve, in device memory (one writer: the reduce kernels).
// alpha is the newest step length, alpha_prev .. alpha_prev3 the three before
// it (the deferred x updates need them); x holds x_0 + sum of alpha_i p_i over
// i < x_steps.
struct SolveState {
    double alpha, beta, kappa_old, R0, R, sigma, kappa;
    double alpha_prev, alpha_prev2, alpha_prev3;
    int32_t k, done, x_steps, status, iters, pad1, pad2, pad3;
};

// Copy of the stop decision that the reduce kernel writes to pinned host memory.
struct HostStatus {
    int32_t k, done, status, iters;
    double R, pad;
};

enum : int32_t { ST_OK = 0, ST_NOT_CONVERGED = 1, ST_BREAKDOWN = -2 };

__device__ __forceinline__ int tile_of_block(int block, int nblocks)
{
    // Blocks 8q + x run on XCD x; give XCD x the contiguous tile range
    // [start(x), start(x) + count(x)).
    const int per = nblocks / kXcds, rem = nblocks % kXcds;
    const int x = block % kXcds, q = block / kXcds;
    return x * per + (x < rem ? x : rem) + q;
}

// Column-pass tile -> (i-tile, j): strips of csg i-tiles, the i-tile faster
// than j inside a strip (csg = 1: j fastest).
struct ColTile {
    int it, j;
};
__device__ __forceinline__ ColTile col_tile(const Op &o, int tile)
{
    const int per_strip = o.csg * o.ny;
    const int g = tile / per_strip;
    const int rem = tile - g * per_strip;
    const int gw = min(o.csg, o.ntc - g * o.csg);
    ColTile ct;
    ct.j = rem / gw;
    ct.it = g * o.csg + (rem - ct.j * gw);
    return ct;
}

__device__ __forceinline__ size_t lin(const Op &o, int i, int j, int k)
{
    return (size_t)i + (size_t)o.nx * ((size_t)k + (size_t)o.nz * (size_t)j);
}

// Precision.  Every kernel is written for two element types: TV, the type of
// the solver's vectors r, q, x, p, b and of their arithmetic, and TZ (or TI
// for a stencil's operand), the type of z and of the column solve.  binary64
// throughout is <double, double>; the single-precision runs of section 7 are
// <float, float>; binary64 PCG with a binary32 preconditioner is
// <double, float>.  The coefficients are kept in binary64 and rounded to the
// arithmetic type where they are used; dot products always accumulate in
// binary64.

// Horizontal edge coefficients alpha_{T,T'} of column (i, j) (section 3,
// eqs. (6)-(7)) and its area |T|, in T.  sum() is alpha_T.
template <typename T>
struct FacesT {
    T xp, xm, yp, ym;
    T area;
    __device__ __forceinline__ T sum() const { return (xp + xm) + (yp + ym); }
};
using Faces = FacesT<double>;

template <typename T>
__device__ __forceinline__ FacesT<T> column_faces_t(const Op &o, int i, int j)
{
    const int im = (i == 0) ? o.nx - 1 : i - 1;
    const int jm = (j == 0) ? o.ny - 1 : j - 1;
    const size_t c = (size_t)j * o.nx + i;
    FacesT<T> f;
    f.xp = (T)o.ex[c];
    f.xm = (T)o.ex[(size_t)j * o.nx + im];
    f.yp = (T)o.ey[c];
    f.ym = (T)o.ey[(size_t)jm * o.nx + i];
    f.area = (T)o.area[c];
    return f;
}

__device__ __forceinline__ Faces column_faces(const Op &o, int i, int j)
{
    return column_faces_t<double>(o, i, j);
}

// The parts of the column matrix A_T (eq. (8)) at level k of a column with
// edges f: the diagonal's zero-order and horizontal part |T| a_k + d_k alpha_T,
// and the vertical couplings lo = |T| beta_k (to k-1), up = |T| beta_{k+1}.
template <typename T>
__device__ __forceinline__ T diag_base_of(const FacesT<T> &f, T aT, double a_k, double d_k)
{
    return f.area * (T)a_k + (T)d_k * aT;
}
template <typename T>
__device__ __forceinline__ T diag_base(const Op &o, const FacesT<T> &f, T aT, int k)
{
    return diag_base_of(f, aT, o.lev_a[k], o.lev_d[k]);
}

// Thomas pivot of level k (section 4.2, eq. (19); Appendix A, Algorithm 3):
// D_k = diag_k - sub_k * phi_{k-1} with diag_k = base + lo + up,
// sub_k = -lo, phi_{k-1} = super_{k-1} / D_{k-1}.  The diagonal is summed in
// the order of its terms, (base + lo) + up: in binary32, adding the two
// large couplings first and the small base after them (lo + up rounded on
// its own) gave pivots whose rounding shifted the solve systematically (a
// forward error of 5.9e-4 instead of 3.8e-4 at 1024 x 1024 x 128 and a
// PCG trajectory apart from binary64's from the first step).
template <typename T>
__device__ __forceinline__ T thomas_pivot(T base, T lo, T up, T phi_prev)
{
    return ((base + lo) + up) + lo * phi_prev;
}

// One row of the stencil (eq. (18) in the general form): c the cell, its
// i-1 / i+1, j-1 / j+1 and k-1 / k+1 neighbours; za = |T| a_k, dk = d_k,
// lo / up the area-scaled vertical couplings.
template <typename T>
__device__ __forceinline__ T stencil_row(const FacesT<T> &f, T za, T dk, T lo, T up, T c, T xm, T xp,
                                         T ym, T yp, T km, T kp)
{
    T hor = f.xp * (c - xp);
    hor += f.xm * (c - xm);
    hor += f.yp * (c - yp);
    hor += f.ym * (c - ym);
    T acc = za * c;
    acc += dk * hor;
    acc += up * (c - kp);
    acc += lo * (c - km);
    return acc;
}

// (offset, slope) of a segment's affine map, exchanged through LDS
template <typename T>
struct __align__(2 * sizeof(T)) Pair {
    T a, b;
};

// Streams that a pass reads or writes exactly once per element go through
// non-temporal loads and stores, so that they do not displace the lines that
// are reused (the stencil halo of z, the coefficient tables) from the caches;
// on this chip that alone raised both fused passes' bandwidth by 6-11 %.
// The value lane `l` holds, in every lane (a wave-uniform copy).
__device__ __forceinline__ double lane_value(double v, int l)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(unsigned)(b & 0xffffffffll), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ float lane_value(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <typename T>
__device__ __forceinline__ T ld_s(const T *p)
{
    return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_s(T *p, T v)
{
    __builtin_nontemporal_store(v, p);
}

// ---------------------------------------------------------------------------
// Deterministic reductions: fixed shuffle tree in a wave, fixed order over the
// waves of a workgroup.
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

// Sum NV per-thread values over the workgroup; thread 0 gets the totals.
template <int NV>
__device__ __forceinline__ void block_sum(double (&v)[NV], double (*sh)[NV], double (&out)[NV])
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
#pragma unroll
    for (int a = 0; a < NV; ++a)
        v[a] = wave_sum(v[a]);
    if (lane == 0) {
#pragma unroll
        for (int a = 0; a < NV; ++a)
            sh[w][a] = v[a];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int a = 0; a < NV; ++a) {
            double t = 0.0;
            for (int q = 0; q < nw; ++q)
                t += sh[q][a];
            out[a] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// Column solve z = M^{-1} r, one tridiagonal system per column (section 4.2,
// eq. (19)), optionally fused with the residual update and the two dot
// products of the interleaved preconditioner kernel (Appendix A,
// Algorithm 3): r <- r - alpha q, <r,r>, <r,z>.
//
// The serial Thomas recurrence of a column is split over the P segment
// threads that own it.  It stays the same elimination:
//  * the pivots D_k and multipliers phi_k do not depend on the data; segment
//    s restarts their recurrence from phi_{s*L-1}, precomputed once per
//    column at set-up (Op::phib), so it reproduces the serial pivots;
//  * the forward-eliminated right-hand side z'_k is affine in the value z'
//    entering the segment: z'_e = z''_e + mu_e * z'_in (z'' and mu computed
//    locally); a scan over the segments through LDS gives every segment its
//    true inflow, after which it recomputes its z'_k exactly;
//  * back substitution z_k = z'_k - phi_k z_{k+1} is affine in the value
//    above the segment: z_k = zh_k + H_k * z_top; a second scan, top down,
//    gives every segment its z_top.
// Per thread only three length-L arrays live in registers (r, 1/D, z').
// Block: C * P threads rounded up to a multiple of 64 (extra threads idle).
//
// STORED: the explicit variant of section 6.2 -- the column matrices are read
// from three stored vectors tri = [sub | diag | sup] (N each, field layout)
// instead of being recomputed, and the boundary multipliers come from a
// table computed from those vectors (phib_tab).
//
// UPD selects the residual update done while loading r:
//   UPD_NONE  none (stand-alone preconditioner, standard loop),
//   UPD_Q     r -= alpha q, q stored by the previous stencil pass (Algorithm 3),
//   UPD_AP    r -= alpha (A p), the product recomputed from p and its
//             neighbours, so that q never has to be stored.
enum : int { UPD_NONE = 0, UPD_Q = 1, UPD_AP = 2 };

// Multigrid forms of the column solve (tensor-product multigrid: horizontal
// semi-coarsening, the column solve as damped block-Jacobi smoother), with
// y = M^{-1} rr:
//   MG_FIRST  rr from the UPD mode, z = omega y    (first sweep from z = 0)
//   MG_CORR   rr = rin, a residual f - A q computed by a stencil pass;
//             z = q + omega y                      (further sweeps)
//   MG_POST   rr = rin - A (P zc), rin the residual t = f - A q kept by the
//             restriction; z = (q + P zc) + omega y: the sweep after the
//             coarse correction, with the residual of q + P zc formed from t
//             and the coarse correction alone (no neighbour reads of q)
//   MG_SWEEP  with UPD_AP: rr = rin - A q with q's neighbours read here (the
//             recomputed-product path with alpha = 1), z = q + omega y: one
//             whole sweep in one pass; no dot products
//   MG_CHEB   MG_SWEEP with the Chebyshev three-term update of a coarsest
//             level: z holds z_{k-1} on entry (read at the thread's own
//             points only, before they are written) and receives
//             (q + c1 (q - z_{k-1})) + c2 y; mg.cheb == 1: z_{k-1} = 0 (the
//             buffer is not used)
// P zc is the value of the coarse parent.  Binary64 only.  The dot products
// of MG_CORR and MG_POST are <f, f> and <f, z> (f: the level's right-hand
// side); in every MG form they are skipped when partials is null.  MG_CORR
// with mg.cheb != 0 takes MG_CHEB's update (z_{k-1} read from z at each
// point before it is written).
enum : int { MG_NONE = 0, MG_FIRST = 1, MG_CORR = 2, MG_POST = 3, MG_SWEEP = 4, MG_CHEB = 5 };

// The one-pass sweep forms (the residual formed from q and its neighbours).
template <int MG>
constexpr bool kSweepForm = MG == MG_SWEEP || MG == MG_CHEB;

struct MgArgs {
    const double *zc;   // coarse correction (coarse layout), or null
    const double *f;    // the level's right-hand side (dot products of MG_CORR, MG_POST)
    double omega;       // damping of the smoother
    int ncx, fx, fy;    // coarse row length, coarsening factors in i and j
    double c1, c2;      // Chebyshev step: z_{k+1} = (z_k + c1 (z_k - z_{k-1})) + c2 M^{-1} (f - A z_k)
    int cheb;           // 0: the damped update; 1: Chebyshev, z_{k-1} = 0; 2: Chebyshev
};

// The Chebyshev three-term update of MG_CHEB and MG_CORR with mg.cheb != 0.
__device__ __forceinline__ double cheb_update(const MgArgs &mg, double zk, double zold, double y)
{
    const double zo = mg.cheb == 2 ? zold : 0.0;
    return (zk + mg.c1 * (zk - zo)) + mg.c2 * y;
}

// Where a column pass reads its residual.  The pointer arguments of the
// column kernels are restrict-qualified, so no two of them may name the same
// vector: in the solve's in-place update r -= alpha q the residual is read
// and written through rout (each thread reads its own elements before it
// writes them) and rin is null; every other form reads rin, a vector none of
// the other arguments names.
template <int UPD, int MG, typename TV, typename TZ>
__device__ __forceinline__ const TV *residual_source(const TV *rin, TV *rout, TZ *)
{
    if constexpr (!kSweepForm<MG> && UPD != UPD_NONE)
        return rout;
    else
        return rin;
}

// Index of the coarse parent of fine cell (i, j, k): (i / fx, j / fy, k).
__device__ __forceinline__ size_t mg_parent(const MgArgs &m, int nz, int i, int j, int k)
{
    return (size_t)(i / m.fx) + (size_t)m.ncx * ((size_t)k + (size_t)nz * (size_t)(j / m.fy));
}

// Threads per workgroup a column-solve instantiation is compiled for: the
// multigrid forms on narrow tiles (a coarsest level) have at most 16
// segments per column, the rest up to 1024 threads.
template <int C, int MG>
constexpr int col_bound() { return (MG != MG_NONE && C < kWave) ? 16 * C : kMaxThreads; }

template <int L, int C, int UPD, bool DOTS, bool STORED, typename TV = double, typename TZ = double,
          int MG = MG_NONE>
__global__ __launch_bounds__((col_bound<C, MG>())) void k_column_solve(
    const TV *__restrict__ rin, const TV *__restrict__ q, TV *__restrict__ rout,
    TZ *__restrict__ z, Op o, const SolveState *__restrict__ st, int first,
    double *__restrict__ partials, const double *__restrict__ tri,
    const TZ *__restrict__ phib_tab, MgArgs mg)
{
    const TV *rsrc = residual_source<UPD, MG>(rin, rout, z);
    static_assert((UPD != UPD_AP && !STORED) ||
                      (std::is_same<TV, double>::value && std::is_same<TZ, double>::value),
                  "the stored-matrix and recomputed-Ap forms are binary64 only");
    static_assert(MG == MG_NONE || ((UPD != UPD_AP || kSweepForm<MG>) && !STORED &&
                                    std::is_same<TV, double>::value && std::is_same<TZ, double>::value),
                  "the multigrid forms are binary64 only");
    static_assert(!kSweepForm<MG> || UPD == UPD_AP, "MG_SWEEP forms its residual on the recomputed-product path");
    static_assert(MG != MG_POST || UPD == UPD_NONE, "MG_POST reads its residual as it is");
    __shared__ TZ sh_a[kMaxThreads];
    __shared__ TZ sh_b[kMaxThreads];
    __shared__ double sh_red[kMaxThreads / kWave][2];

    if (st != nullptr && st->done)
        return;
    const int tid = threadIdx.x;
    const int c = tid % C;
    // with 64 columns a wave owns one segment: keep s in a scalar register
    const int s = (C == kWave) ? __builtin_amdgcn_readfirstlane(tid / C) : tid / C;
    const int P = o.P;
    const bool active = s < P;
    const int tile = tile_of_block(blockIdx.x, gridDim.x);
    const ColTile ct = col_tile(o, tile);
    const int it = ct.it, j = ct.j;
    const int i = it * C + c;
    const bool ok = active && i < o.nx;
    const int ic = i < o.nx ? i : o.nx - 1;
    const FacesT<TZ> fc = column_faces_t<TZ>(o, ic, j);
    const TZ aT = fc.sum();
    const int k0 = s * L;
    const int len = active ? min(L, o.nz - k0) : 0;
    const size_t base = lin(o, ic, j, 0);
    const size_t ks = (size_t)o.nx;
    const TV alpha = kSweepForm<MG> ? (TV)1 : ((UPD != UPD_NONE && !first) ? (TV)st->alpha : (TV)0);
    // the Thomas multiplier at the segment's lower boundary (set-up table),
    // requested before the segment's other loads
    const TZ phi_in = (s > 0 && active)
                          ? ld_s(phib_tab + (size_t)(s * o.pst - 1) * ((size_t)o.nx * o.ny) + (size_t)j * o.nx + ic)
                          : (TZ)0;

    // The segment's vertical face coefficients: face(t) couples levels
    // k0+t-1 and k0+t (face(0) below the segment, face(len) above it).  With
    // 64 columns the segment is wave-uniform and the loads are scalar; with
    // 32 a wave holds two segments and a register copy avoids reloading them.
    TZ fz[L + 1];
    if constexpr (C != kWave) {
#pragma unroll
        for (int t = 0; t <= L; ++t)
        {
            const TZ fv = (TZ)o.az[min(k0 + t, o.nz)];   // faces 0..nz
            fz[t] = (t <= len) ? fv : (TZ)0;
        }
    }
    // area-scaled vertical coupling across face(t)
    auto face = [&](int t) -> TZ {
        if constexpr (C == kWave)
            return fc.area * (TZ)o.az[k0 + t];
        else
            return fc.area * fz[t];
    };
    // stored coefficients of the segment's levels: lo = -sub, up = -sup, diag
    TZ slo[STORED ? L : 1], sup_[STORED ? L : 1], sdg[STORED ? L : 1];
    if constexpr (STORED) {
        const size_t n = (size_t)o.nx * o.ny * o.nz;
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const size_t l = base + (size_t)(k0 + t) * ks;
            const bool in = t < len;
            slo[t] = in ? -ld_s(tri + l) : 0.0;
            sdg[t] = in ? ld_s(tri + n + l) : 1.0;
            sup_[t] = in ? -ld_s(tri + 2 * n + l) : 0.0;
        }
    }
    auto lo_at = [&](int t) -> TZ {
        if constexpr (STORED) return slo[t]; else return face(t);
    };
    auto up_at = [&](int t) -> TZ {
        if constexpr (STORED) return sup_[t]; else return face(t + 1);
    };

    TV rr[L];
    TZ iD[L], zp[L];
    double r2 = 0.0;
    // Segments of up to 8 levels request a_k, d_k and r of all their levels
    // (clamped: in bounds for every thread) with the first loads, so no load
    // is left inside the per-level loops below, whose branches would wait
    // for each one in turn (one memory round trip per level); longer
    // segments load them where they are used, to keep their registers.
    constexpr bool kPre = L <= 8 && !STORED;
    double la[kPre ? L : 1], ldv[kPre ? L : 1];
    if constexpr (kPre) {
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const int kk = min(k0 + t, o.nz - 1);
            la[t] = o.lev_a[kk];
            ldv[t] = o.lev_d[kk];
        }
    }
    auto a_at = [&](int t) -> double {
        if constexpr (kPre) return la[t]; else return o.lev_a[k0 + t];
    };
    auto d_at = [&](int t) -> double {
        if constexpr (kPre) return ldv[t]; else return o.lev_d[k0 + t];
    };
    double zsw[kSweepForm<MG> ? L : 1];   // MG_SWEEP, MG_CHEB: the iterate at the column's levels
    double zo[MG == MG_CHEB ? L : 1];     // MG_CHEB: z_{k-1} at the column's levels
    if constexpr (kSweepForm<MG>) {
#pragma unroll
        for (int t = 0; t < L; ++t)
            zsw[t] = 0.0;
    }
    if constexpr (UPD == UPD_AP) {
        // q = p; (A p) at the segment's levels.  Load phase first (r, p at
        // levels k0-1..k0+L clamped to the grid, p at j-1 and j+1; with 64
        // columns per wave p at i-1 / i+1 comes from the adjacent lanes except
        // at the tile edges and the periodic wrap), then the products.
        const bool do_ap = !first && len > 0;
        const int lane = tid & (kWave - 1);
        const int ip = (ic + 1 == o.nx) ? 0 : ic + 1;
        const int im = (ic == 0) ? o.nx - 1 : ic - 1;
        const int jp = (j + 1 == o.ny) ? 0 : j + 1;
        const int jm = (j == 0) ? o.ny - 1 : j - 1;
        const size_t bxp = lin(o, ip, j, 0), bxm = lin(o, im, j, 0);
        const size_t byp = lin(o, ic, jp, 0), bym = lin(o, ic, jm, 0);
        constexpr bool kShfl = C == kWave;
        const bool needL = !kShfl || lane == 0;
        const bool needR = !kShfl || lane == kWave - 1 || ic + 1 >= o.nx;
        auto lev = [&](int k) { return (size_t)min(max(k, 0), o.nz - 1) * ks; };
        double pv[L + 2], pyp[L], pym[L], pxl[L], pxr[L];
        double ra[kPre ? L : 1];   // r at the segment's levels (kPre: with the operands)
        if constexpr (kPre) {
#pragma unroll
            for (int t = 0; t < L; ++t)
                ra[t] = ld_s(rsrc + base + (size_t)min(k0 + t, o.nz - 1) * ks);
        }
        if constexpr (MG == MG_CHEB) {   // z_{k-1}, with the operands (used only when mg.cheb == 2)
#pragma unroll
            for (int t = 0; t < L; ++t)
                zo[t] = ld_s(z + base + (size_t)min(k0 + t, o.nz - 1) * ks);
        }
        if (do_ap) {
#pragma unroll
            for (int t = 0; t < L + 2; ++t)
                pv[t] = q[base + lev(k0 - 1 + t)];
#pragma unroll
            for (int t = 0; t < L; ++t) {
                const size_t off = lev(k0 + t);
                pyp[t] = q[byp + off];
                pym[t] = q[bym + off];
                pxl[t] = needL ? q[bxm + off] : 0.0;
                pxr[t] = needR ? q[bxp + off] : 0.0;
            }
        }
#pragma unroll
        for (int t = 0; t < L; ++t) {
            double v = 0.0;
            if constexpr (kPre)
                v = (t < len && ok) ? ra[t] : 0.0;
            else if (t < len && ok)
                v = ld_s(rsrc + base + (size_t)(k0 + t) * ks);
            if (do_ap && t < len) {
                const double pc = pv[t + 1];
                double pl = pxl[t], pr = pxr[t];
                if constexpr (kShfl) {
                    const double pl_s = __shfl_up(pc, 1, kWave);
                    const double pr_s = __shfl_down(pc, 1, kWave);
                    pl = needL ? pl : pl_s;
                    pr = needR ? pr : pr_s;
                }
                const double lo = face(t), up = face(t + 1);
                const double Ap = stencil_row<double>(fc, fc.area * a_at(t), d_at(t), lo, up, pc, pl, pr,
                                                      pym[t], pyp[t], pv[t], pv[t + 2]);
                if (ok)
                    v = v - alpha * Ap;
                if constexpr (kSweepForm<MG>)
                    zsw[t] = pc;
            }
            rr[t] = v;
            r2 += v * v;
        }
    } else if constexpr (MG == MG_POST) {
        // rr = t - A (P zc): the coarse parents of the column (levels k0-1 ..
        // k0+L, clamped), of the j-1 and j+1 columns, and of the i-1 / i+1
        // columns (from the adjacent lanes, except where a lane loads its own).
        const bool do_it = len > 0;
        const int lane = tid & (kWave - 1);
        const int ip = (ic + 1 == o.nx) ? 0 : ic + 1;
        const int im = (ic == 0) ? o.nx - 1 : ic - 1;
        const int jp = (j + 1 == o.ny) ? 0 : j + 1;
        const int jm = (j == 0) ? o.ny - 1 : j - 1;
        const size_t pc = mg_parent(mg, o.nz, ic, j, 0);
        const size_t pxp = mg_parent(mg, o.nz, ip, j, 0), pxm = mg_parent(mg, o.nz, im, j, 0);
        const size_t pyp = mg_parent(mg, o.nz, ic, jp, 0), pym = mg_parent(mg, o.nz, ic, jm, 0);
        constexpr bool kShfl = C == kWave;
        const bool needL = !kShfl || lane == 0;
        const bool needR = !kShfl || lane == kWave - 1 || ic + 1 >= o.nx;
        const size_t ksc = (size_t)mg.ncx;
        auto lev = [&](int k) { return (size_t)min(max(k, 0), o.nz - 1) * ksc; };
        double cv[L + 2], cyp[L], cym[L], cxl[L], cxr[L];
        if (do_it) {
#pragma unroll
            for (int t = 0; t < L + 2; ++t)
                cv[t] = mg.zc[pc + lev(k0 - 1 + t)];
#pragma unroll
            for (int t = 0; t < L; ++t) {
                const size_t off = lev(k0 + t);
                cyp[t] = mg.zc[pyp + off];
                cym[t] = mg.zc[pym + off];
                cxl[t] = needL ? mg.zc[pxm + off] : 0.0;
                cxr[t] = needR ? mg.zc[pxp + off] : 0.0;
            }
        }
        double ra[kPre ? L : 1];   // as in the UPD_AP form
        if constexpr (kPre) {
#pragma unroll
            for (int t = 0; t < L; ++t)
                ra[t] = ld_s(rsrc + base + (size_t)min(k0 + t, o.nz - 1) * ks);
        }
#pragma unroll
        for (int t = 0; t < L; ++t) {
            double v = 0.0;
            if constexpr (kPre)
                v = (t < len && ok) ? ra[t] : 0.0;
            else if (t < len && ok)
                v = ld_s(rsrc + base + (size_t)(k0 + t) * ks);
            if (do_it && t < len) {
                const double c = cv[t + 1];
                double xl = cxl[t], xr = cxr[t];
                if constexpr (kShfl) {
                    const double l_s = __shfl_up(c, 1, kWave);
                    const double r_s = __shfl_down(c, 1, kWave);
                    xl = needL ? xl : l_s;
                    xr = needR ? xr : r_s;
                }
                const double APz = stencil_row<double>(fc, fc.area * a_at(t), d_at(t), face(t), face(t + 1),
                                                       c, xl, xr, cym[t], cyp[t], cv[t], cv[t + 2]);
                v = v - APz;
            }
            rr[t] = v;
        }
    } else {
        // kPre: all of the segment's loads first (clamped levels), then the selects
        TV ra[kPre ? L : 1], qa[kPre ? L : 1];
        if constexpr (kPre) {
#pragma unroll
            for (int t = 0; t < L; ++t)
                ra[t] = ld_s(rsrc + base + (size_t)min(k0 + t, o.nz - 1) * ks);
            if constexpr (UPD == UPD_Q) {   // on the first step too (not used then): no branch
#pragma unroll
                for (int t = 0; t < L; ++t)
                    qa[t] = ld_s(q + base + (size_t)min(k0 + t, o.nz - 1) * ks);
            }
        }
#pragma unroll
        for (int t = 0; t < L; ++t) {
            TV v = (TV)0;
            if (t < len && ok) {
                if constexpr (kPre) {
                    v = ra[t];
                    if (UPD == UPD_Q && !first)
                        v = v - alpha * qa[t];
                } else {
                    const size_t l = base + (size_t)(k0 + t) * ks;
                    v = ld_s(rsrc + l);
                    if (UPD == UPD_Q && !first)
                        v = v - alpha * ld_s(q + l);
                }
            }
            rr[t] = v;
            r2 += (double)v * (double)v;
        }
    }
    if (!kSweepForm<MG> && UPD != UPD_NONE && !first && ok) {
#pragma unroll
        for (int t = 0; t < L; ++t)
            if (t < len)
                st_s(rout + base + (size_t)(k0 + t) * ks, rr[t]);
    }

    // Local forward sweep: pivots from the true incoming phi, z'' with zero
    // inflow; the right-hand side rounded to TZ.
    TZ phi = phi_in;
    TZ zpp = 0, mu = 1;
#pragma unroll
    for (int t = 0; t < L; ++t) {
        if (t < len) {
            const TZ lo = lo_at(t), up = up_at(t);
            TZ D;
            if constexpr (STORED)
                D = sdg[t] + lo * phi;
            else
                D = thomas_pivot(diag_base_of(fc, aT, a_at(t), d_at(t)), lo, up, phi);
            const TZ inv = (TZ)1 / D;
            iD[t] = inv;
            phi = -up * inv;
            zpp = ((TZ)rr[t] + lo * zpp) * inv;
            mu = (lo * inv) * mu;
        } else {
            iD[t] = 0;
        }
    }
    if (active) {
        sh_a[s * C + c] = zpp;
        sh_b[s * C + c] = mu;
    }
    __syncthreads();
    // Both scans run over the largest segment count of the instantiation with
    // a select, so their LDS reads do not wait behind the recurrence.
    constexpr int kSegMax = col_bound<C, MG>() / C;
    TZ zin = 0;
#pragma unroll
    for (int w = 0; w < kSegMax - 1; ++w) {
        const TZ nz_ = sh_a[w * C + c] + sh_b[w * C + c] * zin;
        zin = w < s ? nz_ : zin;
    }

    // Forward sweep again with the true inflow: z'_k of the serial algorithm.
    TZ prev = zin;
#pragma unroll
    for (int t = 0; t < L; ++t) {
        if (t < len) {
            const TZ lo = lo_at(t);
            prev = ((TZ)rr[t] + lo * prev) * iD[t];
            zp[t] = prev;
        }
    }
    // Local back substitution with zero value above the segment.
    TZ znext = 0, H = 1;
#pragma unroll
    for (int t = L - 1; t >= 0; --t) {
        if (t < len) {
            const TZ up = up_at(t);
            const TZ ph = -up * iD[t];
            znext = zp[t] - ph * znext;
            H = -ph * H;
            zp[t] = znext;
        }
    }
    __syncthreads();   // every thread has finished reading the first scan
    if (active) {
        sh_a[s * C + c] = znext;   // zh at the segment's first level
        sh_b[s * C + c] = H;       // response of that level to the value above
    }
    __syncthreads();
    TZ ztop = 0;
#pragma unroll
    for (int w = kSegMax - 1; w > 0; --w) {
        const TZ nt = sh_a[w * C + c] + sh_b[w * C + c] * ztop;
        ztop = (w > s && w < P) ? nt : ztop;
    }

    double kap = 0.0, r2mg = 0.0;
    H = 1;
#pragma unroll
    for (int t = L - 1; t >= 0; --t) {
        if (t < len) {
            const TZ up = up_at(t);
            H = (up * iD[t]) * H;
            TZ zv = zp[t] + ztop * H;
            if constexpr (MG == MG_FIRST)
                zv = (TZ)mg.omega * zv;
            if constexpr (MG == MG_SWEEP)
                zv = zsw[t] + mg.omega * zv;
            if constexpr (MG == MG_CHEB)
                zv = cheb_update(mg, zsw[t], zo[t], zv);
            if constexpr (MG == MG_CORR || MG == MG_POST) {
                // the iterate (plus the coarse correction) and f, loaded here,
                // after the solve, to keep the registers of the sweep low
                const size_t l = base + (size_t)(k0 + t) * ks;
                double zq = ok ? ld_s(q + l) : 0.0;
                if constexpr (MG == MG_POST)
                    zq = zq + mg.zc[mg_parent(mg, o.nz, ic, j, k0 + t)];
                if (MG == MG_CORR && mg.cheb != 0)
                    zv = cheb_update(mg, zq, (ok && mg.cheb == 2) ? ld_s(z + l) : 0.0, zv);
                else
                    zv = zq + mg.omega * zv;
                const double fv = (ok && partials) ? ld_s(mg.f + l) : 0.0;
                kap += fv * zv;
                r2mg += fv * fv;
            } else {
                kap += (double)rr[t] * (double)zv;
            }
            if (ok)
                st_s(z + base + (size_t)(k0 + t) * ks, zv);
        }
    }
    if (DOTS && (MG == MG_NONE || partials != nullptr)) {
        double v[2] = {(MG == MG_CORR || MG == MG_POST) ? r2mg : r2, kap};
        double out[2];
        block_sum<2>(v, sh_red, out);
        if (tid == 0) {
            partials[2 * (size_t)tile + 0] = out[0];
            partials[2 * (size_t)tile + 1] = out[1];
        }
    }
}

// Loads and stores at a wave-uniform base plus a 32-bit per-lane byte offset:
// the base stays in scalar registers and the address needs no 64-bit vector
// arithmetic.
template <typename T>
__device__ __forceinline__ T ld_at(const T *base, unsigned boff)
{
    return ld_s((const T *)((const char *)base + boff));
}
// The same with an ordinary (cached) load, for lines other workgroups read
// again (the coarse correction of the multigrid sweeps).
template <typename T>
__device__ __forceinline__ T ldc_at(const T *base, unsigned boff)
{
    return *(const T *)((const char *)base + boff);
}
template <typename T>
__device__ __forceinline__ void st_at(T *base, unsigned boff, T v)
{
    st_s((T *)((char *)base + boff), v);
}

// The column solve of k_column_solve (same elimination, same segment scans)
// for grids whose tiles are all whole: nx a multiple of 64 and nz a multiple
// of L, so every thread owns L levels of an existing column and the code is
// straight-line.  Thread (lane, wave s): column it*64 + lane, segment s.
// The segment inflow / outflow scans read the other segments' affine maps as
// (offset, slope) pairs from LDS without branches, so the reads are not
// serialised behind the recurrence.
template <int L, int UPD, bool DOTS, typename TV = double, typename TZ = double, int MG = MG_NONE>
__global__ __launch_bounds__(kMaxThreads) void k_column_full(
    const TV *__restrict__ rin, const TV *__restrict__ q, TV *__restrict__ rout,
    TZ *__restrict__ z, Op o, const SolveState *__restrict__ st, int first,
    double *__restrict__ partials, const TZ *__restrict__ phib, MgArgs mg)
{
    const TV *rsrc = residual_source<UPD, MG>(rin, rout, z);
    static_assert(UPD != UPD_AP || (std::is_same<TV, double>::value && std::is_same<TZ, double>::value),
                  "the recomputed-Ap form is binary64 only");
    static_assert(MG == MG_NONE || ((UPD != UPD_AP || kSweepForm<MG>) && std::is_same<TV, double>::value &&
                                    std::is_same<TZ, double>::value),
                  "the multigrid forms are binary64 only");
    static_assert(!kSweepForm<MG> || UPD == UPD_AP, "MG_SWEEP forms its residual on the recomputed-product path");
    static_assert(MG != MG_POST || UPD == UPD_NONE, "MG_POST reads its residual as it is");
    constexpr int kSeg = kMaxThreads / kWave;
    __shared__ Pair<TZ> sh_ab[kMaxThreads];
    __shared__ double sh_red[kSeg][2];

    if (st != nullptr && st->done)
        return;
    const int lane = threadIdx.x & (kWave - 1);
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int P = o.P;
    const int nx = o.nx;
    const int tile = tile_of_block(blockIdx.x, gridDim.x);
    const ColTile ct = col_tile(o, tile);
    const int it = ct.it, j = ct.j;
    const int i = it * kWave + lane;
    const FacesT<TZ> fz = column_faces_t<TZ>(o, i, j);
    const TZ aT = fz.sum();
    const int k0 = s * L;
    const unsigned cv = (unsigned)i * (unsigned)sizeof(TV);   // lane's byte offset in a TV row
    const unsigned cz = (unsigned)i * (unsigned)sizeof(TZ);   // ... in a TZ row
    const size_t row0 = ((size_t)j * o.nz + k0) * nx;   // level k0 of row j (uniform)
    const TV alpha = kSweepForm<MG> ? (TV)1 : ((UPD != UPD_NONE && !first) ? (TV)st->alpha : (TV)0);
    const double *az = o.az + k0;                       // az[t]: face below level k0+t
    // area-scaled vertical couplings: vz(t) couples levels k0+t-1 and k0+t
    auto vz = [&](int t) -> TZ { return fz.area * (TZ)az[t]; };

    TV rr[L];
    double r2 = 0.0;
    double zsw[kSweepForm<MG> ? L : 1];   // MG_SWEEP, MG_CHEB: the iterate at the column's levels
    double zo[MG == MG_CHEB ? L : 1];     // MG_CHEB: z_{k-1} at the column's levels
    if constexpr (UPD == UPD_Q && L == 16) {
        // q is requested on the first step too (its buffer exists; the
        // values are not used then): a branch on `first` here would split
        // the load phase, and the compiler then waits for all of r before
        // requesting q.  (16-level segments: at 8 levels the extra
        // registers would cost a second workgroup per CU.)
        TV qv[L];
#pragma unroll
        for (int t = 0; t < L; ++t) {
            rr[t] = ld_at(rsrc + row0 + (size_t)t * nx, cv);
            qv[t] = ld_at(q + row0 + (size_t)t * nx, cv);
        }
#pragma unroll
        for (int t = 0; t < L; ++t)
            rr[t] = first ? rr[t] : rr[t] - alpha * qv[t];
    } else if (UPD == UPD_Q && !first) {
        TV qv[L];
#pragma unroll
        for (int t = 0; t < L; ++t) {
            rr[t] = ld_at(rsrc + row0 + (size_t)t * nx, cv);
            qv[t] = ld_at(q + row0 + (size_t)t * nx, cv);
        }
#pragma unroll
        for (int t = 0; t < L; ++t)
            rr[t] = rr[t] - alpha * qv[t];
    } else if (UPD == UPD_AP && !first) {
        // r -= alpha (A p): p at levels k0-1 .. k0+L (clamped to the grid),
        // at j-1 and j+1, and at i-1 / i+1 from the adjacent lanes (lanes 0
        // and 63 load theirs: one load with two active lanes per level).
        const Faces fc = column_faces(o, i, j);
        const int jp = (j + 1 == o.ny) ? 0 : j + 1;
        const int jm = (j == 0) ? o.ny - 1 : j - 1;
        const size_t rowp = ((size_t)jp * o.nz + k0) * nx, rowm = ((size_t)jm * o.nz + k0) * nx;
        const int ie = lane == 0 ? (i == 0 ? nx - 1 : i - 1) : (i + 1 == nx ? 0 : i + 1);
        const unsigned e8 = (unsigned)ie * 8u;
        const bool edge = lane == 0 || lane == kWave - 1;
        const int kb = k0 > 0 ? -1 : 0;                      // level below, clamped
        const int ka = k0 + L < o.nz ? L : L - 1;            // level above, clamped
        double pv[L + 2], pyp[L], pym[L], pe[L];
        pv[0] = ld_at(q + row0 + (ptrdiff_t)kb * nx, cv);
        pv[L + 1] = ld_at(q + row0 + (size_t)ka * nx, cv);
#pragma unroll
        for (int t = 0; t < L; ++t) {
            if constexpr (MG == MG_CHEB)   // z_{k-1} (used only when mg.cheb == 2)
                zo[t] = ld_at(z + row0 + (size_t)t * nx, cz);
            rr[t] = ld_at(rsrc + row0 + (size_t)t * nx, cv);
            pv[t + 1] = ld_at(q + row0 + (size_t)t * nx, cv);
            pyp[t] = ld_at(q + rowp + (size_t)t * nx, cv);
            pym[t] = ld_at(q + rowm + (size_t)t * nx, cv);
            pe[t] = edge ? ld_at(q + row0 + (size_t)t * nx, e8) : 0.0;
        }
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const double pc = pv[t + 1];
            const double pl_s = __shfl_up(pc, 1, kWave);
            const double pr_s = __shfl_down(pc, 1, kWave);
            const double pl = lane == 0 ? pe[t] : pl_s;
            const double pr = lane == kWave - 1 ? pe[t] : pr_s;
            const double Ap = stencil_row<double>(fc, fc.area * o.lev_a[k0 + t], o.lev_d[k0 + t],
                                                  fc.area * az[t], fc.area * az[t + 1], pc, pl, pr, pym[t],
                                                  pyp[t], pv[t], pv[t + 2]);
            rr[t] = rr[t] - alpha * Ap;
            if constexpr (kSweepForm<MG>)
                zsw[t] = pc;
        }
    } else if constexpr (MG == MG_POST) {
        // rr = t - A (P zc): the coarse parents of the column (levels k0-1 ..
        // k0+L, clamped), of the i-1 / i+1 columns from the adjacent lanes
        // (lanes 0 and 63 load theirs), and of the j-1 / j+1 columns: with
        // fy = 2 one of those is the column's own parent, so one row is loaded.
        // Parent rows are wave-uniform; a lane adds the byte offset of its parent.
        const int jp = (j + 1 == o.ny) ? 0 : j + 1;
        const int jm = (j == 0) ? o.ny - 1 : j - 1;
        const size_t ksc = (size_t)mg.ncx;
        const unsigned pl = (unsigned)(i / mg.fx) * 8u;
        const int J = j / mg.fy;
        const bool om = jm / mg.fy != J, op = jp / mg.fy != J;   // neighbour rows with another parent
        auto prow = [&](int jj) { return mg.zc + ksc * ((size_t)o.nz * (size_t)(jj / mg.fy) + (size_t)k0); };
        const double *zcc = prow(j);
        const double *zyo = om ? prow(jm) : prow(jp);
        const double *zy2 = prow(jp);
        const int kb = k0 > 0 ? -1 : 0;                      // level below, clamped
        const int ka = k0 + L < o.nz ? L : L - 1;            // level above, clamped
        double cc[L + 2], cy[L];
        cc[0] = ldc_at(zcc + (ptrdiff_t)kb * (ptrdiff_t)ksc, pl);
        cc[L + 1] = ldc_at(zcc + (size_t)ka * ksc, pl);
        // the parents of the tile's two outside columns at the segment's
        // levels in one load: lane e < L takes the left one's at level k0 + e,
        // lane L + e the right one's (handed to lanes 0 and 63 by readlane)
        double ev = 0.0;
        {
            static_assert(2 * L <= kWave, "edge parents in one load");
            const int t0 = i - lane;
            const int io = lane < L ? (t0 == 0 ? nx - 1 : t0 - 1) : (t0 + kWave == nx ? 0 : t0 + kWave);
            const int e = lane < L ? lane : lane - L;
            if (lane < 2 * L)
                ev = ldc_at(zcc + (size_t)e * ksc, (unsigned)(io / mg.fx) * 8u);
        }
#pragma unroll
        for (int t = 0; t < L; ++t) {
            rr[t] = ld_at(rsrc + row0 + (size_t)t * nx, cv);
            cc[t + 1] = ldc_at(zcc + (size_t)t * ksc, pl);
            cy[t] = (om || op) ? ldc_at(zyo + (size_t)t * ksc, pl) : 0.0;
        }
        const Faces fc = column_faces(o, i, j);
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const double c = cc[t + 1];
            const double l_s = __shfl_up(c, 1, kWave);
            const double r_s = __shfl_down(c, 1, kWave);
            const double xl = lane == 0 ? lane_value(ev, t) : l_s;
            const double xr = lane == kWave - 1 ? lane_value(ev, L + t) : r_s;
            const double ym = om ? cy[t] : c;
            double yp = c;
            if (op)   // wave-uniform; both rows differ only when fy = 1
                yp = om ? ldc_at(zy2 + (size_t)t * ksc, pl) : cy[t];
            const double APz = stencil_row<double>(fc, fc.area * o.lev_a[k0 + t], o.lev_d[k0 + t], fc.area * az[t],
                                                   fc.area * az[t + 1], c, xl, xr, ym, yp, cc[t], cc[t + 2]);
            rr[t] = rr[t] - APz;
        }
    } else {
#pragma unroll
        for (int t = 0; t < L; ++t)
            rr[t] = ld_at(rsrc + row0 + (size_t)t * nx, cv);
    }
#pragma unroll
    for (int t = 0; t < L; ++t)
        r2 += (double)rr[t] * (double)rr[t];
    if (!kSweepForm<MG> && UPD != UPD_NONE && !first) {
#pragma unroll
        for (int t = 0; t < L; ++t)
            st_at(rout + row0 + (size_t)t * nx, cv, rr[t]);
    }
    // MG_CORR: the iterate and f, loaded with the residual (MG_POST, whose
    // stencil on the coarse correction holds more registers in the load
    // phase, loads them after the solve)
    double zb[MG == MG_CORR ? L : 1], fb[MG == MG_CORR ? L : 1];
    if constexpr (MG == MG_CORR) {
#pragma unroll
        for (int t = 0; t < L; ++t) {
            zb[t] = ld_at(q + row0 + (size_t)t * nx, cv);
            fb[t] = partials ? ld_at(mg.f + row0 + (size_t)t * nx, cv) : 0.0;
        }
    }

    // Local forward sweep: pivots from the true incoming phi, z'' with zero
    // inflow; the right-hand side rounded to TZ.
    const size_t ncol = (size_t)nx * o.ny;
    TZ phi = s > 0 ? ld_s(phib + (size_t)(s * o.pst - 1) * ncol + (size_t)j * nx + i) : (TZ)0;
    TZ iD[L], zp[L];
    TZ zpp = 0, mu = 1;
#pragma unroll
    for (int t = 0; t < L; ++t) {
        const TZ lo = vz(t), up = vz(t + 1);
        const TZ inv = (TZ)1 / thomas_pivot(diag_base(o, fz, aT, k0 + t), lo, up, phi);
        iD[t] = inv;
        phi = -up * inv;
        zpp = ((TZ)rr[t] + lo * zpp) * inv;
        mu = (lo * inv) * mu;
    }
    sh_ab[s * kWave + lane] = Pair<TZ>{zpp, mu};
    __syncthreads();
    TZ zin = 0;
#pragma unroll
    for (int w = 0; w < kSeg - 1; ++w) {
        const Pair<TZ> ab = sh_ab[w * kWave + lane];
        const TZ nz_ = ab.a + ab.b * zin;
        zin = w < s ? nz_ : zin;
    }

    // Forward sweep again with the true inflow, then the local back
    // substitution with zero value above the segment.
    TZ prev = zin;
#pragma unroll
    for (int t = 0; t < L; ++t) {
        prev = ((TZ)rr[t] + vz(t) * prev) * iD[t];
        zp[t] = prev;
    }
    TZ znext = 0, H = 1;
#pragma unroll
    for (int t = L - 1; t >= 0; --t) {
        const TZ ph = -vz(t + 1) * iD[t];
        znext = zp[t] - ph * znext;
        H = -ph * H;
        zp[t] = znext;
    }
    __syncthreads();   // every wave has finished reading the first scan
    sh_ab[s * kWave + lane] = Pair<TZ>{znext, H};
    __syncthreads();
    TZ ztop = 0;
#pragma unroll
    for (int w = kSeg - 1; w > 0; --w) {
        const Pair<TZ> ab = sh_ab[w * kWave + lane];
        const TZ nt = ab.a + ab.b * ztop;
        ztop = (w > s && w < P) ? nt : ztop;
    }

    double kap = 0.0, r2mg = 0.0;
    H = 1;
#pragma unroll
    for (int t = L - 1; t >= 0; --t) {
        H = (vz(t + 1) * iD[t]) * H;
        TZ zv = zp[t] + ztop * H;
        if constexpr (MG == MG_FIRST)
            zv = (TZ)mg.omega * zv;
        if constexpr (MG == MG_SWEEP)
            zv = zsw[t] + mg.omega * zv;
        if constexpr (MG == MG_CHEB)
            zv = cheb_update(mg, zsw[t], zo[t], zv);
        if constexpr (MG == MG_CORR || MG == MG_POST) {
            // MG_POST loads the iterate (plus the coarse correction) and f
            // here, after the solve: its load phase holds the coarse
            // stencil's operands (issued all together here, they spill)
            double zq, fv;
            if constexpr (MG == MG_CORR) {
                zq = zb[t];
                fv = fb[t];
            } else {
                zq = ld_at(q + row0 + (size_t)t * nx, cv) +
                     ldc_at(mg.zc + (size_t)mg.ncx * ((size_t)o.nz * (size_t)(j / mg.fy) + (size_t)(k0 + t)),
                            (unsigned)(i / mg.fx) * 8u);
                fv = partials ? ld_at(mg.f + row0 + (size_t)t * nx, cv) : 0.0;
            }
            if (MG == MG_CORR && mg.cheb != 0)
                zv = cheb_update(mg, zq, mg.cheb == 2 ? ld_at(z + row0 + (size_t)t * nx, cz) : 0.0, zv);
            else
                zv = zq + mg.omega * zv;
            kap += fv * zv;
            r2mg += fv * fv;
        } else {
            kap += (double)rr[t] * (double)zv;
        }
        st_at(z + row0 + (size_t)t * nx, cz, zv);
    }
    if (DOTS && (MG == MG_NONE || partials != nullptr)) {
        double v[2] = {(MG == MG_CORR || MG == MG_POST) ? r2mg : r2, kap};
        double out[2];
        block_sum<2>(v, sh_red, out);
        if (threadIdx.x == 0) {
            partials[2 * (size_t)tile + 0] = out[0];
            partials[2 * (size_t)tile + 1] = out[1];
        }
    }
}

// Set-up: the Thomas multipliers phi_k at every segment boundary of every
// column (data independent; computed once per operator and precision, in T).
template <typename T>
__global__ void k_setup_phib(Op o, T *__restrict__ phib)
{
    const size_t ncol = (size_t)o.nx * o.ny;
    const size_t col = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= ncol)
        return;
    const int j = (int)(col / o.nx);
    const int i = (int)(col - (size_t)j * o.nx);
    const FacesT<T> f = column_faces_t<T>(o, i, j);
    const T aT = f.sum();
    T phi = 0;
    for (int k = 0; k < o.nz; ++k) {
        const T lo = f.area * (T)o.az[k], up = f.area * (T)o.az[k + 1];
        const T inv = (T)1 / thomas_pivot(diag_base(o, f, aT, k), lo, up, phi);
        phi = -up * inv;
        const int kk = k + 1;
        if (kk % o.L == 0 && kk / o.L < o.P)
            phib[(size_t)(kk / o.L - 1) * ncol + col] = phi;
    }
}

// Set-up of the explicit variant: the same boundary multipliers computed from
// stored column matrices tri = [sub | diag | sup].
__global__ void k_setup_phib_stored(Op o, const double *__restrict__ tri, double *__restrict__ phib)
{
    const size_t ncol = (size_t)o.nx * o.ny;
    const size_t n = ncol * o.nz;
    const size_t col = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= ncol)
        return;
    const int j = (int)(col / o.nx);
    const int i = (int)(col - (size_t)j * o.nx);
    double phi = 0.0;
    for (int k = 0; k < o.nz; ++k) {
        const size_t l = lin(o, i, j, k);
        const double lo = -tri[l];
        const double inv = 1.0 / (tri[n + l] + lo * phi);
        phi = tri[2 * n + l] * inv;   // super-diagonal / pivot
        const int kk = k + 1;
        if (kk % o.L == 0 && kk / o.L < o.P)
            phib[(size_t)(kk / o.L - 1) * ncol + col] = phi;
    }
}

// Assembly of the stored column matrices of M (section 6.2: the tridiagonal
// matrix of the preconditioner kept as three vectors of length N):
// sub = -|T| beta_k, diag = (|T| a_k + d_k alpha_T) + |T| beta_k + |T| beta_{k+1}
// (summed in that order, as the pivots of the matrix-free solve),
// sup = -|T| beta_{k+1} (zero couplings at the bottom and top faces).
__global__ void k_tridiag_assemble(Op o, double *__restrict__ tri)
{
    const size_t ncol = (size_t)o.nx * o.ny;
    const size_t n = ncol * o.nz;
    const size_t col = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= ncol)
        return;
    const int j = (int)(col / o.nx);
    const int i = (int)(col - (size_t)j * o.nx);
    const Faces f = column_faces(o, i, j);
    const double aT = f.sum();
    for (int k = 0; k < o.nz; ++k) {
        const size_t l = lin(o, i, j, k);
        const double lo = f.area * o.az[k], up = f.area * o.az[k + 1];
        tri[l] = -lo;
        tri[n + l] = (diag_base(o, f, aT, k) + lo) + up;
        tri[2 * n + l] = -up;
    }
}

// ---------------------------------------------------------------------------
// Sweep passes.
struct Sweep {
    int i, j, k0, len, ic;
    bool ok;
    int tile;
};

// Wave w of the workgroup sweeps levels [k0, k0 + len) of column i of row j.
// JT = 1: the tile is one row, its waves split the levels; JT > 1: the tile is
// JT rows of Ls levels, wave w takes row j0 + w (o.jt = JT, o.ny % JT == 0).
template <int JT = 1>
__device__ __forceinline__ Sweep sweep_of_thread(const Op &o, int Ls)
{
    Sweep sw;
    sw.tile = tile_of_block(blockIdx.x, gridDim.x);
    // strip g holds i-tiles [g*sg, g*sg + gw); the last strip may be narrower
    const int nj = JT > 1 ? o.ny / JT : o.ny;
    const int per_strip = o.sg * nj * o.nkt;
    const int g = sw.tile / per_strip;
    const int rem = sw.tile - g * per_strip;
    const int gw = min(o.sg, o.ntx - g * o.sg);
    const int kt = rem % o.nkt;
    const int r = rem / o.nkt;
    const int jb = r / gw;
    const int it = g * o.sg + (r - jb * gw);
    sw.i = it * kWave + (threadIdx.x & (kWave - 1));
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (JT > 1) {
        sw.j = jb * JT + w;
        sw.k0 = kt * Ls;
    } else {
        sw.j = jb;
        sw.k0 = (kt * o.Ws + w) * Ls;
    }
    sw.len = max(0, min(Ls, o.nz - sw.k0));
    sw.ok = sw.i < o.nx;
    sw.ic = sw.ok ? sw.i : o.nx - 1;
    return sw;
}

enum : int {
    SP_FIRST = 0,     // p = z, q = A z, <p,q>             (first interleaved pass)
    SP_APPLY = 2,     // y = A x
    SP_RESID = 3,     // y = b - A x
    SP_APPLY_DOT = 4, // y = A x, <x, y>  (standard PCG: q = A p, sigma)
    SP_FIRST_AP = 5,  // p = z, <z, A z>                    (no q stored)
    SP_FUSED_AP = 6,  // x += alpha p, p_new = z + beta p, <p_new, A z + beta A p>  (no q stored)
    SP_FUSED_NOX = 7, // Algorithm 2 with the x update deferred: p_new = z + beta p (to
                      //   p_out), q = A z + beta q, <p_new, q>
    SP_FUSED_X4 = 9   // SP_FUSED_NOX plus the four pending x updates of p_{k-4}
                      //   (p_out), p_{k-3}, p_{k-2} (older.a, older.b) and p_{k-1} (p)
};

// The two directions between p_out and p that SP_FUSED_X4 reads (p_{k-3},
// p_{k-2}); null in every other mode.
template <typename T>
struct Older {
    const T *a, *b;
};

// Stencil passes (section 4.2, eq. (18)): the 7-point operator recomputed in
// every cell from the column's face coefficients and the level's alpha_z.
// Block: 64 * Ws threads.
// SP_FIRST_AP / SP_FUSED_AP read the old search direction from p (with its
// neighbours) and write the new one to p_out, a different buffer: an in-place
// update would let a neighbour read an already-updated value.
// SP_FUSED_NOX / SP_FUSED_X4 update x every fourth step (the stencil passes
// of three steps skip it, the fourth applies the four terms in one read and
// write of x): p rotates over four buffers so that the older directions are
// still there; p_out holds p_{k-4} on entry and receives the new one (each
// point is read before it is written by the same thread, and p has no
// neighbour reads here).  Once the stop test has passed (st->done) every
// form returns at once: the updates still pending are applied by k_x_fixup.
// FULL: every tile is whole (nx a multiple of 64, nz a multiple of Ws * Ls),
// so no level or column guard is needed, and a wave fetches the outside
// neighbours of its two edge lanes (i-1 for lane 0, i+1 for lane 63) at all
// its levels with one load over 2 * Ls lanes, then hands them out with
// readlane.
// JT > 1 (whole tiles only): a tile is JT rows of Ls levels, one wave per row;
// each wave puts its z rows in LDS and takes z at j-1 and j+1 from the waves
// of the rows beside it, so only the tile's first and last waves load a
// neighbour row from memory.
template <int Ls, int MODE, bool FULL, typename TV = double, typename TI = double, int JT = 1>
__global__ __launch_bounds__(kMaxThreads) void k_stencil(const TI *__restrict__ zin,
                                                         const TV *__restrict__ bvec,
                                                         TV *__restrict__ u,
                                                         TV *__restrict__ p,
                                                         TV *__restrict__ y, Op o,
                                                         const SolveState *__restrict__ st,
                                                         double *__restrict__ partials,
                                                         TV *__restrict__ p_out, Older<TV> older)
{
    static_assert((MODE != SP_FIRST_AP && MODE != SP_FUSED_AP) ||
                      (std::is_same<TV, double>::value && std::is_same<TI, double>::value),
                  "the q-free forms are binary64 only");
    static_assert(JT == 1 || (FULL && MODE != SP_FIRST_AP && MODE != SP_FUSED_AP),
                  "row tiles: whole tiles, one operand");
    __shared__ double sh_red[kMaxThreads / kWave][1];
    TV alpha = 0, beta = 0;
    constexpr bool kDot = MODE == SP_FIRST || MODE == SP_APPLY_DOT ||
                          MODE == SP_FIRST_AP || MODE == SP_FUSED_AP || MODE == SP_FUSED_NOX ||
                          MODE == SP_FUSED_X4;
    constexpr bool kX4 = MODE == SP_FUSED_X4;
    constexpr bool kNox = MODE == SP_FUSED_NOX || kX4;   // p, q updates of Algorithm 2
    TV alpha_prev = 0, alpha_prev2 = 0, alpha_prev3 = 0;
    if (kDot) {
        if (st->done)
            return;
        alpha = (TV)st->alpha;
        beta = (TV)st->beta;
        if (kX4) {
            alpha_prev = (TV)st->alpha_prev;
            alpha_prev2 = (TV)st->alpha_prev2;
            alpha_prev3 = (TV)st->alpha_prev3;
        }
    }
    const Sweep sw = sweep_of_thread<JT>(o, Ls);
    const size_t ks = (size_t)o.nx;
    const size_t base = lin(o, sw.ic, sw.j, 0);

    double acc = 0.0;
    if (sw.len > 0) {
        const FacesT<TV> f = column_faces_t<TV>(o, sw.ic, sw.j);
        const int lane = threadIdx.x & (kWave - 1);
        const int ip = (sw.ic + 1 == o.nx) ? 0 : sw.ic + 1;
        const int im = (sw.ic == 0) ? o.nx - 1 : sw.ic - 1;
        const int jp = (sw.j + 1 == o.ny) ? 0 : sw.j + 1;
        const int jm = (sw.j == 0) ? o.ny - 1 : sw.j - 1;
        const size_t bxp = lin(o, ip, sw.j, 0), bxm = lin(o, im, sw.j, 0);
        const size_t byp = lin(o, sw.ic, jp, 0), bym = lin(o, sw.ic, jm, 0);
        const int k0 = sw.k0, len = sw.len;
        // i-1 is lane-1 except for lane 0; i+1 is lane+1 except for lane 63 and
        // for the last column of the grid (periodic wrap).  Those lanes load
        // their neighbour; the others take it from the adjacent lane.
        const bool needL = lane == 0;
        const bool needR = FULL ? lane == kWave - 1 : (lane == kWave - 1 || sw.ic + 1 >= o.nx);
        [[maybe_unused]] const size_t bxe = needL ? bxm : bxp;   // FULL: the edge lanes' outside neighbour
        auto lev = [&](int k) { return (size_t)min(max(k, 0), o.nz - 1) * ks; };
        const int wj = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // JT > 1: the tile's row

        // Load phase: every value of the wave's Ls levels is requested before
        // any is used, so a wave waits for one memory round trip, not Ls.
        constexpr bool kAp = MODE == SP_FUSED_AP;
        TV zv[Ls + 2], zyp[Ls], zym[Ls], zxl[Ls], zxr[Ls];   // the operand, widened to TV
        TV pv[kAp ? Ls + 2 : 1], pyp[kAp ? Ls : 1], pym[kAp ? Ls : 1], pxl[kAp ? Ls : 1], pxr[kAp ? Ls : 1];
        TV uo[Ls], po[Ls], qo[Ls], p2[kX4 ? Ls : 1], p3[kX4 ? Ls : 1], p4[kX4 ? Ls : 1];
        TV ev = 0;
        if constexpr (FULL) {
            // every outside neighbour of the wave's edge lanes in one load:
            // lane e < Ls takes the left neighbour of lane 0 at level k0 + e,
            // lane Ls + e the right neighbour of lane 63 (spread after the loads)
            const int i0 = sw.ic - lane;
            const int il = i0 == 0 ? o.nx - 1 : i0 - 1;
            const int ir = i0 + kWave == o.nx ? 0 : i0 + kWave;
            const int e = lane < Ls ? lane : lane - Ls;
            if (lane < 2 * Ls)
                ev = (TV)zin[lin(o, lane < Ls ? il : ir, sw.j, 0) + lev(k0 + e)];
        }
#pragma unroll
        for (int t = 0; t < Ls + 2; ++t) {
            const size_t off = lev(k0 - 1 + t);   // levels k0-1 .. k0+Ls, clamped to the grid
            zv[t] = (TV)zin[base + off];
            if constexpr (kAp)
                pv[t] = p[base + off];
        }
#pragma unroll
        for (int t = 0; t < Ls; ++t) {
            const size_t off = lev(k0 + t);
            if constexpr (JT > 1) {
                // rows j +- 1 inside the tile come from LDS below
                zyp[t] = wj == JT - 1 ? (TV)zin[byp + off] : (TV)0;
                zym[t] = wj == 0 ? (TV)zin[bym + off] : (TV)0;
            } else {
                zyp[t] = (TV)zin[byp + off];
                zym[t] = (TV)zin[bym + off];
            }
            if constexpr (!FULL) {   // whole tiles: ev, spread below
                zxl[t] = needL ? (TV)zin[bxm + off] : (TV)0;
                zxr[t] = needR ? (TV)zin[bxp + off] : (TV)0;
            }
            if constexpr (kAp) {
                pyp[t] = p[byp + off];
                pym[t] = p[bym + off];
                if constexpr (FULL) {
                    pxl[t] = (needL || needR) ? p[bxe + off] : 0.0;
                    pxr[t] = pxl[t];
                } else {
                    pxl[t] = needL ? p[bxm + off] : 0.0;
                    pxr[t] = needR ? p[bxp + off] : 0.0;
                }
            }
            if constexpr (MODE == SP_FUSED_AP || kX4)
                uo[t] = ld_s(u + base + off);
            if constexpr (kNox)
                po[t] = ld_s(p + base + off);
            if constexpr (kX4) {
                p2[t] = ld_s(p_out + base + off);
                p3[t] = ld_s(older.a + base + off);
                p4[t] = ld_s(older.b + base + off);
            }
            if constexpr (kNox)
                qo[t] = ld_s(y + base + off);
            if constexpr (MODE == SP_RESID)
                qo[t] = ld_s(bvec + base + off);
        }
        if constexpr (JT > 1) {
            __shared__ TV sh_z[JT][Ls][kWave];   // each wave's z rows
#pragma unroll
            for (int t = 0; t < Ls; ++t)
                sh_z[wj][t][lane] = zv[t + 1];
            __syncthreads();
#pragma unroll
            for (int t = 0; t < Ls; ++t) {
                if (wj > 0)
                    zym[t] = sh_z[wj - 1][t][lane];
                if (wj < JT - 1)
                    zyp[t] = sh_z[wj + 1][t][lane];
            }
        }
        if constexpr (FULL) {
#pragma unroll
            for (int t = 0; t < Ls; ++t) {
                zxl[t] = lane_value(ev, t);
                zxr[t] = lane_value(ev, Ls + t);
            }
        }

        // Compute phase.
#pragma unroll
        for (int t = 0; t < Ls; ++t) {
            if (FULL || t < len) {
                const int k = k0 + t;
                const TV lo = f.area * (TV)o.az[k], up = f.area * (TV)o.az[k + 1];
                const TV za = f.area * (TV)o.lev_a[k], dk = (TV)o.lev_d[k];
                const TV zc = zv[t + 1];
                const TV zl_s = __shfl_up(zc, 1, kWave);
                const TV zr_s = __shfl_down(zc, 1, kWave);
                const TV zl = needL ? zxl[t] : zl_s;
                const TV zr = needR ? zxr[t] : zr_s;
                // k = 0 / nz-1: the clamped neighbour is zc itself and lo / up is 0
                const TV Az = stencil_row(f, za, dk, lo, up, zc, zl, zr, zym[t], zyp[t], zv[t], zv[t + 2]);
                const size_t l = base + (size_t)k * ks;
                if constexpr (kAp) {
                    const double pc = pv[t + 1];
                    const double pl_s = __shfl_up(pc, 1, kWave);
                    const double pr_s = __shfl_down(pc, 1, kWave);
                    const double pl = needL ? pxl[t] : pl_s;
                    const double pr = needR ? pxr[t] : pr_s;
                    const double Ap = stencil_row<double>(f, za, dk, lo, up, pc, pl, pr, pym[t], pyp[t], pv[t],
                                                          pv[t + 2]);
                    if (FULL || sw.ok) {
                        st_s(u + l, uo[t] + alpha * pc);
                        const double pnew = zc + beta * pc;
                        st_s(p_out + l, pnew);
                        acc += pnew * (Az + beta * Ap);
                    }
                } else if (FULL || sw.ok) {
                    if (MODE == SP_FIRST) {
                        st_s(p + l, zc);
                        st_s(y + l, Az);
                        acc += (double)zc * (double)Az;
                    } else if (kNox) {
                        if constexpr (kX4)   // in the order of the steps, as one update a step
                            st_s(u + l, (((uo[t] + alpha_prev3 * p2[t]) + alpha_prev2 * p3[t]) +
                                         alpha_prev * p4[t]) + alpha * po[t]);
                        const TV pn = zc + beta * po[t];
                        const TV qn = Az + beta * qo[t];
                        st_s(p_out + l, pn);
                        st_s(y + l, qn);
                        acc += (double)pn * (double)qn;
                    } else if (MODE == SP_APPLY) {
                        st_s(y + l, Az);
                    } else if (MODE == SP_RESID) {
                        st_s(y + l, qo[t] - Az);
                    } else if (MODE == SP_APPLY_DOT) {
                        st_s(y + l, Az);
                        acc += (double)zc * (double)Az;
                    } else if (MODE == SP_FIRST_AP) {
                        st_s(p_out + l, zc);
                        acc += (double)zc * (double)Az;
                    }
                }
            }
        }
    }
    if (kDot) {
        double v[1] = {acc};
        double out[1];
        block_sum<1>(v, sh_red, out);
        if (threadIdx.x == 0)
            partials[2 * (size_t)sw.tile] = out[0];
    }
}

// Vector passes of the standard PCG loop, each fused with its dot product
// (sweep geometry).
// x += alpha p ; r -= alpha q ; <r,r>
template <int Ls>
__global__ __launch_bounds__(kMaxThreads) void k_update_xr(double *__restrict__ x,
                                                           const double *__restrict__ p,
                                                           double *__restrict__ r,
                                                           const double *__restrict__ q, Op o,
                                                           const SolveState *__restrict__ st,
                                                           double *__restrict__ partials)
{
    __shared__ double sh_red[kMaxThreads / kWave][1];
    if (st->done)
        return;
    const double alpha = st->alpha;
    const Sweep sw = sweep_of_thread(o, Ls);
    double acc = 0.0;
    if (sw.ok) {
        const size_t base = lin(o, sw.i, sw.j, 0);
#pragma unroll 4
        for (int t = 0; t < sw.len; ++t) {
            const size_t l = base + (size_t)(sw.k0 + t) * o.nx;
            st_s(x + l, ld_s(x + l) + alpha * ld_s(p + l));
            const double rn = ld_s(r + l) - alpha * ld_s(q + l);
            st_s(r + l, rn);
            acc += rn * rn;
        }
    }
    double v[1] = {acc};
    double out[1];
    block_sum<1>(v, sh_red, out);
    if (threadIdx.x == 0)
        partials[2 * (size_t)sw.tile] = out[0];
}

// p = z + beta p   (p = z on the first step)
template <int Ls>
__global__ __launch_bounds__(kMaxThreads) void k_update_p(double *__restrict__ p,
                                                          const double *__restrict__ z, Op o,
                                                          const SolveState *__restrict__ st,
                                                          int first)
{
    if (st->done)
        return;
    const double beta = st->beta;
    const Sweep sw = sweep_of_thread(o, Ls);
    if (!sw.ok)
        return;
    const size_t base = lin(o, sw.i, sw.j, 0);
#pragma unroll 4
    for (int t = 0; t < sw.len; ++t) {
        const size_t l = base + (size_t)(sw.k0 + t) * o.nx;
        st_s(p + l, first ? ld_s(z + l) : ld_s(z + l) + beta * ld_s(p + l));
    }
}

// ---------------------------------------------------------------------------
// Tensor-product multigrid: the passes between the column sweeps.  Levels
// keep nz and halve nx and / or ny (factors fx, fy in {1, 2}); prolongation is
// piecewise constant (a fine cell takes its coarse parent's value) and
// restriction is its transpose (the sum over the children), so the coarse
// operator P^T A P is again of the general form:

// Coarse coefficients: |T| summed over the children, the coarse edge between
// parents I and I+1 (J and J+1) the sum of the fine edges crossing it, zero
// in a dimension of size 1 (a column coupled with itself cancels).  Summed in
// the order (row b outer, column a inner).  One thread per coarse column.
__global__ void k_mg_coarsen(Op o, int ncx, int ncy, int fx, int fy, double *__restrict__ carea,
                             double *__restrict__ cax, double *__restrict__ cay)
{
    const size_t col = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= (size_t)ncx * ncy)
        return;
    const int J = (int)(col / ncx);
    const int I = (int)(col - (size_t)J * ncx);
    const size_t nx = (size_t)o.nx;
    double sa = 0.0, sx = 0.0, sy = 0.0;
    for (int b = 0; b < fy; ++b)
        for (int a = 0; a < fx; ++a)
            sa += o.area[(size_t)(fy * J + b) * nx + (size_t)(fx * I + a)];
    for (int b = 0; b < fy; ++b)
        sx += o.ex[(size_t)(fy * J + b) * nx + (size_t)(fx * I + fx - 1)];
    for (int a = 0; a < fx; ++a)
        sy += o.ey[(size_t)(fy * J + fy - 1) * nx + (size_t)(fx * I + a)];
    carea[col] = sa;
    cax[col] = ncx == 1 ? 0.0 : sx;
    cay[col] = ncy == 1 ? 0.0 : sy;
}

// Residual and restriction after the pre-smoothing sweeps: t = f - A z (kept
// for the sweep after the coarse correction, MG_POST) and fc = P^T t.  A
// workgroup owns 64 fine columns (one lane each) of the FY fine rows of one
// coarse row J over Ws * Ls levels; tiles run k-tile fastest, then the
// i-tile, then J.  A lane loads the FY rows and the rows below and above
// them once (with FY = 2 the two middle rows are each other's neighbours),
// computes the residual of its column in each of the FY rows, and with
// FX = 2 the two children in i are adjacent lanes.  The children are summed
// in the order (row outer, column inner).
template <int Ls, int FX, int FY>
__global__ __launch_bounds__(kMaxThreads) void k_mg_restrict(const double *__restrict__ f,
                                                             const double *__restrict__ zin,
                                                             double *__restrict__ t_out,
                                                             double *__restrict__ fc, Op o, int ncx,
                                                             const SolveState *__restrict__ st)
{
    if (st != nullptr && st->done)
        return;
    const int tile = tile_of_block(blockIdx.x, gridDim.x);
    const int kt = tile % o.nkt;
    const int rem = tile / o.nkt;
    const int it = rem % o.ntx;
    const int J = rem / o.ntx;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = it * kWave + lane;
    const bool ok = i < o.nx;
    const int ic = ok ? i : o.nx - 1;
    const int k0 = (kt * o.Ws + w) * Ls;
    const int len = max(0, min(Ls, o.nz - k0));
    if (len == 0)
        return;   // wave-uniform
    const size_t ks = (size_t)o.nx;
    const int ip = (ic + 1 == o.nx) ? 0 : ic + 1;
    const int im = (ic == 0) ? o.nx - 1 : ic - 1;
    const bool needL = lane == 0;
    const bool needR = lane == kWave - 1 || ic + 1 >= o.nx;
    auto lev = [&](int k) { return (size_t)min(max(k, 0), o.nz - 1) * ks; };
    // rows: jr[0] below, jr[1 .. FY] the children, jr[FY + 1] above
    int jr[FY + 2];
    jr[1] = FY * J;
    jr[0] = jr[1] == 0 ? o.ny - 1 : jr[1] - 1;
    if constexpr (FY == 2)
        jr[2] = jr[1] + 1;
    jr[FY + 1] = jr[FY] + 1 == o.ny ? 0 : jr[FY] + 1;
    double zc[FY][Ls + 2], zo[2][Ls], ze[FY][Ls], fv[FY][Ls];
#pragma unroll
    for (int b = 0; b < FY; ++b) {
        const size_t base = lin(o, ic, jr[b + 1], 0);
        const size_t bxe = lin(o, needL ? im : ip, jr[b + 1], 0);
#pragma unroll
        for (int t = 0; t < Ls + 2; ++t)
            zc[b][t] = zin[base + lev(k0 - 1 + t)];
#pragma unroll
        for (int t = 0; t < Ls; ++t) {
            ze[b][t] = (needL || needR) ? zin[bxe + lev(k0 + t)] : 0.0;
            fv[b][t] = ld_s(f + base + lev(k0 + t));
        }
    }
#pragma unroll
    for (int t = 0; t < Ls; ++t) {
        zo[0][t] = zin[lin(o, ic, jr[0], 0) + lev(k0 + t)];
        zo[1][t] = zin[lin(o, ic, jr[FY + 1], 0) + lev(k0 + t)];
    }
    double res[FY][Ls];
#pragma unroll
    for (int b = 0; b < FY; ++b) {
        const int j = jr[b + 1];
        const Faces fcs = column_faces(o, ic, j);
        const size_t base = lin(o, ic, j, 0);
#pragma unroll
        for (int t = 0; t < Ls; ++t) {
            const int k = min(k0 + t, o.nz - 1);
            const double lo = fcs.area * o.az[k], up = fcs.area * o.az[k + 1];
            const double c = zc[b][t + 1];
            const double zl_s = __shfl_up(c, 1, kWave);
            const double zr_s = __shfl_down(c, 1, kWave);
            // a lane that needs both sides (a grid of one column) loaded one
            // value: the same cell either way
            const double zl = needL ? ze[b][t] : zl_s;
            const double zr = needR ? ze[b][t] : zr_s;
            const double ym = b == 0 ? zo[0][t] : zc[b - 1][t + 1];
            const double yp = b == FY - 1 ? zo[1][t] : zc[b + 1][t + 1];
            const double Az = stencil_row<double>(fcs, fcs.area * o.lev_a[k], o.lev_d[k], lo, up, c, zl, zr,
                                                  ym, yp, zc[b][t], zc[b][t + 2]);
            const double r = fv[b][t] - Az;
            res[b][t] = (t < len && ok) ? r : 0.0;
            if (t < len && ok)
                st_s(t_out + base + (size_t)(k0 + t) * ks, r);
        }
    }
#pragma unroll
    for (int t = 0; t < Ls; ++t) {
        double v;
        if constexpr (FX == 2) {
            const double x0 = __shfl_xor(res[0][t], 1, kWave);
            if constexpr (FY == 2) {
                const double x1 = __shfl_xor(res[1][t], 1, kWave);
                v = ((res[0][t] + x0) + res[1][t]) + x1;
            } else {
                v = res[0][t] + x0;
            }
        } else if constexpr (FY == 2) {
            v = res[0][t] + res[1][t];
        } else {
            v = res[0][t];
        }
        if (t < len && ok && (FX == 1 || (lane & 1) == 0))
            st_s(fc + (size_t)(i / FX) + (size_t)ncx * ((size_t)(k0 + t) + (size_t)o.nz * (size_t)J), v);
    }
}

// ---------------------------------------------------------------------------
// Explicit operator in CSR form (section 6.2: the same 7-point operator stored
// as a compressed-sparse-row matrix).  Rows follow the field layout; a row
// holds the diagonal, its distinct horizontal neighbours (two per direction,
// one when the periodic direction has 2 cells, none when it has 1) and the
// vertical neighbours that exist; columns ascending.  The row length depends
// only on k, so row_ptr has a closed form and needs no scan.
struct CsrShape {
    int hx, hy;    // distinct horizontal neighbours per direction
    int base;      // 1 + hx + hy
};

__device__ __forceinline__ int csr_vert(int k, int nz) { return (k > 0) + (k < nz - 1); }
__device__ __forceinline__ int64_t csr_vert_prefix(int k, int nz)
{
    // sum over k' < k of csr_vert(k')
    return (int64_t)max(0, k - 1) + (int64_t)min(k, nz - 1);
}

__device__ __forceinline__ int64_t csr_row_start(const Op &o, const CsrShape &cs, int i, int j, int k)
{
    const int64_t l = (int64_t)lin(o, i, j, k);
    const int64_t V = csr_vert_prefix(o.nz, o.nz);
    return l * cs.base + (int64_t)j * o.nx * V + (int64_t)o.nx * csr_vert_prefix(k, o.nz) +
           (int64_t)i * csr_vert(k, o.nz);
}

// Fill row_ptr (N+1), col (nnz) and val (nnz).  Sweep geometry.
template <int Ls>
__global__ __launch_bounds__(kMaxThreads) void k_csr_assemble(Op o, CsrShape cs,
                                                              int64_t *__restrict__ row_ptr,
                                                              int32_t *__restrict__ col,
                                                              double *__restrict__ val)
{
    const Sweep sw = sweep_of_thread(o, Ls);
    if (!sw.ok || sw.len <= 0)
        return;
    const int i = sw.i, j = sw.j;
    const Faces f = column_faces(o, i, j);
    const int ip = (i + 1 == o.nx) ? 0 : i + 1;
    const int im = (i == 0) ? o.nx - 1 : i - 1;
    const int jp = (j + 1 == o.ny) ? 0 : j + 1;
    const int jm = (j == 0) ? o.ny - 1 : j - 1;
    for (int t = 0; t < sw.len; ++t) {
        const int k = sw.k0 + t;
        const double lo = f.area * o.az[k], up = f.area * o.az[k + 1];
        const double dk = o.lev_d[k];
        int32_t cc[7];
        double vv[7];
        int m = 0;
        double diag = f.area * o.lev_a[k];
        if (cs.hx == 2) {
            cc[m] = (int32_t)lin(o, ip, j, k); vv[m++] = -dk * f.xp;
            cc[m] = (int32_t)lin(o, im, j, k); vv[m++] = -dk * f.xm;
            diag += dk * (f.xp + f.xm);
        } else if (cs.hx == 1) {
            cc[m] = (int32_t)lin(o, ip, j, k); vv[m++] = -dk * (f.xp + f.xm);
            diag += dk * (f.xp + f.xm);
        }
        if (cs.hy == 2) {
            cc[m] = (int32_t)lin(o, i, jp, k); vv[m++] = -dk * f.yp;
            cc[m] = (int32_t)lin(o, i, jm, k); vv[m++] = -dk * f.ym;
            diag += dk * (f.yp + f.ym);
        } else if (cs.hy == 1) {
            cc[m] = (int32_t)lin(o, i, jp, k); vv[m++] = -dk * (f.yp + f.ym);
            diag += dk * (f.yp + f.ym);
        }
        if (k > 0) {
            cc[m] = (int32_t)lin(o, i, j, k - 1); vv[m++] = -lo;
            diag += lo;
        }
        if (k < o.nz - 1) {
            cc[m] = (int32_t)lin(o, i, j, k + 1); vv[m++] = -up;
            diag += up;
        }
        cc[m] = (int32_t)lin(o, i, j, k);
        vv[m++] = diag;
        // insertion sort by column (at most 7 entries)
        for (int a = 1; a < m; ++a) {
            const int32_t ck = cc[a];
            const double vk = vv[a];
            int b = a - 1;
            while (b >= 0 && cc[b] > ck) {
                cc[b + 1] = cc[b];
                vv[b + 1] = vv[b];
                --b;
            }
            cc[b + 1] = ck;
            vv[b + 1] = vk;
        }
        const int64_t start = csr_row_start(o, cs, i, j, k);
        const int64_t l = (int64_t)lin(o, i, j, k);
        row_ptr[l] = start;
        for (int a = 0; a < m; ++a) {
            col[start + a] = cc[a];
            val[start + a] = vv[a];
        }
        if (l == (int64_t)o.nx * o.ny * o.nz - 1)
            row_ptr[l + 1] = start + m;
    }
}

enum : int { CSR_APPLY = 0, CSR_RESID = 1, CSR_APPLY_DOT = 2 };

// y = A x from the CSR matrix; RESID: y = b - A x; APPLY_DOT: also <x, y> per
// workgroup.  A workgroup covers the rows of one sweep tile (64 columns x
// Ws * Ls levels of one row j: the sweep passes' tiles, so the same partial
// sums) and gives each row a group of kCsrG lanes: the lanes of a group read
// the row's entries side by side (a wave reads 8 consecutive rows' entries in
// one contiguous run) and add their products in a 3-step butterfly.
constexpr int kCsrG = 8;
template <int MODE>
__global__ __launch_bounds__(kMaxThreads) void k_csr_spmv(const int64_t *__restrict__ row_ptr,
                                                          const int32_t *__restrict__ col,
                                                          const double *__restrict__ val,
                                                          const double *__restrict__ x,
                                                          const double *__restrict__ bvec,
                                                          double *__restrict__ y, Op o,
                                                          const SolveState *__restrict__ st,
                                                          double *__restrict__ partials)
{
    __shared__ double sh_red[kMaxThreads / kWave][1];
    if (MODE == CSR_APPLY_DOT && st->done)
        return;
    const int tile = tile_of_block(blockIdx.x, gridDim.x);
    const int per_strip = o.sg * o.ny * o.nkt;
    const int g = tile / per_strip;
    const int rem = tile - g * per_strip;
    const int gw = min(o.sg, o.ntx - g * o.sg);
    const int kt = rem % o.nkt;
    const int r = rem / o.nkt;
    const int j = r / gw;
    const int i0 = (g * o.sg + (r - j * gw)) * kWave;
    const int k0 = kt * o.Ws * o.Ls;
    const int q = threadIdx.x & (kCsrG - 1);            // lane in the row's group
    const int grp = threadIdx.x / kCsrG;
    const int ngrp = blockDim.x / kCsrG;
    const int rows = kWave * o.Ws * o.Ls;               // the tile's rows: (level, column) pairs
    // kCsrU rows per group at a time, so that their dependent loads (row
    // pointers, then entries, then x) are in flight together; rows / ngrp =
    // 8 * Ls is a multiple of kCsrU, so every group runs the same trip count
    constexpr int kCsrU = 4;
    double acc = 0.0;
    for (int t0 = grp; t0 < rows; t0 += ngrp * kCsrU) {
        size_t l[kCsrU];
        bool in[kCsrU];
        int64_t e0[kCsrU], e1[kCsrU];
#pragma unroll
        for (int u = 0; u < kCsrU; ++u) {
            const int t = t0 + u * ngrp;
            const int i = i0 + (t & (kWave - 1)), k = k0 + t / kWave;
            in[u] = i < o.nx && k < o.nz;
            l[u] = in[u] ? lin(o, i, j, k) : 0;
            e0[u] = in[u] ? row_ptr[l[u]] : 0;
            e1[u] = in[u] ? row_ptr[l[u] + 1] : 0;
        }
        double v[kCsrU];
        int c[kCsrU];
#pragma unroll
        for (int u = 0; u < kCsrU; ++u) {
            const int64_t e = e0[u] + q;
            const bool has = e < e1[u];
            v[u] = has ? val[e] : 0.0;
            c[u] = has ? col[e] : -1;
        }
        double sum[kCsrU], xd[kCsrU];   // APPLY_DOT: x at the row's own point, from the gathers
#pragma unroll
        for (int u = 0; u < kCsrU; ++u) {
            const double xc = c[u] >= 0 ? x[c[u]] : 0.0;
            sum[u] = v[u] * xc;
            xd[u] = (MODE == CSR_APPLY_DOT && c[u] >= 0 && (size_t)c[u] == l[u]) ? xc : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kCsrU; ++u) {
            for (int64_t e = e0[u] + q + kCsrG; e < e1[u]; e += kCsrG) {   // rows of more than kCsrG entries
                const double xc = x[col[e]];
                sum[u] += val[e] * xc;
                if (MODE == CSR_APPLY_DOT && (size_t)col[e] == l[u])
                    xd[u] = xc;
            }
            double s = sum[u];
            s += __shfl_xor(s, 4, kCsrG);
            s += __shfl_xor(s, 2, kCsrG);
            s += __shfl_xor(s, 1, kCsrG);
            double xl = xd[u];   // one lane of the group holds x at the row's point, the others 0
            if (MODE == CSR_APPLY_DOT) {
                xl += __shfl_xor(xl, 4, kCsrG);
                xl += __shfl_xor(xl, 2, kCsrG);
                xl += __shfl_xor(xl, 1, kCsrG);
            }
            if (in[u] && q == 0) {
                if (MODE == CSR_RESID) {
                    st_s(y + l[u], ld_s(bvec + l[u]) - s);
                } else {
                    st_s(y + l[u], s);
                    if (MODE == CSR_APPLY_DOT)
                        acc += xl * s;
                }
            }
        }
    }
    if (MODE == CSR_APPLY_DOT) {
        double v[1] = {acc};
        double out[1];
        block_sum<1>(v, sh_red, out);
        if (threadIdx.x == 0)
            partials[2 * (size_t)tile] = out[0];
    }
}

// ---------------------------------------------------------------------------
// Reductions of the per-workgroup partial sums (entries are pairs; fixed
// order: deterministic) and the scalar recurrences of PCG (section 4.3,
// Algorithm 1).
constexpr int kRedThreads = 256;

// Stage 1: block b sums pairs [b*per, min(n, (b+1)*per)) into out[2b], out[2b+1].
__global__ __launch_bounds__(kRedThreads) void k_sum_stage(const double *__restrict__ in, int n,
                                                           int per, double *__restrict__ out)
{
    __shared__ double sh[2][kRedThreads];
    const int tid = threadIdx.x;
    const int lo = blockIdx.x * per;
    const int hi = min(n, lo + per);
    double a0 = 0.0, a1 = 0.0;
    for (int t = lo + tid; t < hi; t += kRedThreads) {
        a0 += in[2 * (size_t)t];
        a1 += in[2 * (size_t)t + 1];
    }
    sh[0][tid] = a0;
    sh[1][tid] = a1;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if (tid < w) {
            sh[0][tid] += sh[0][tid + w];
            sh[1][tid] += sh[1][tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        out[2 * (size_t)blockIdx.x] = sh[0][0];
        out[2 * (size_t)blockIdx.x + 1] = sh[1][0];
    }
}

template <int NV>
__device__ __forceinline__ void sum_partials(const double *__restrict__ partials, int nparts,
                                             int first_value, double (&tot)[NV])
{
    __shared__ double sh[NV][kRedThreads];
    const int tid = threadIdx.x;
    double acc[NV];
#pragma unroll
    for (int a = 0; a < NV; ++a)
        acc[a] = 0.0;
    for (int t = tid; t < nparts; t += kRedThreads) {
#pragma unroll
        for (int a = 0; a < NV; ++a)
            acc[a] += partials[2 * (size_t)t + first_value + a];
    }
#pragma unroll
    for (int a = 0; a < NV; ++a)
        sh[a][tid] = acc[a];
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if (tid < w) {
#pragma unroll
            for (int a = 0; a < NV; ++a)
                sh[a][tid] += sh[a][tid + w];
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < NV; ++a)
        tot[a] = sh[a][0];
}

__device__ __forceinline__ void finish(SolveState *st, int32_t status)
{
    st->done = 1;
    st->status = status;
}

__device__ __forceinline__ void publish(const SolveState *st, HostStatus *hs, int k)
{
    if (hs) {
        volatile HostStatus *v = hs;
        v->R = st->R;
        v->iters = st->iters;
        v->status = st->status;
        v->done = st->done;
        v->k = k;
    }
}

// After the preconditioner pass of step k: ||r_k||, the stop test, beta.
// Used by both loops (the standard loop passes kappa from its own pass).
__global__ __launch_bounds__(kRedThreads) void k_reduce_rz(const double *__restrict__ partials,
                                                           int nparts, SolveState *st,
                                                           double *__restrict__ hist, int k,
                                                           int maxit, double tol,
                                                           HostStatus *hs)
{
    if (st->done) {
        if (threadIdx.x == 0)
            publish(st, hs, k);
        return;
    }
    double tot[2];
    sum_partials<2>(partials, nparts, 0, tot);
    if (threadIdx.x != 0)
        return;
    const double R = sqrt(tot[0]);
    const double kappa = tot[1];
    st->R = R;
    st->kappa = kappa;
    hist[k] = R;
    if (k == 0) {
        st->R0 = R;
        st->iters = 0;
        st->alpha = 0.0;
        if (!isfinite(R))
            finish(st, ST_BREAKDOWN);
        else if (R == 0.0)
            finish(st, ST_OK);
        else if (maxit == 0)
            finish(st, ST_NOT_CONVERGED);
        else if (!(kappa > 0.0) || !isfinite(kappa))
            finish(st, ST_BREAKDOWN);
        else {
            st->beta = 0.0;
            st->kappa_old = kappa;
        }
    } else {
        st->iters = k;
        if (!isfinite(R))
            finish(st, ST_BREAKDOWN);
        else if (R == 0.0 || R / st->R0 < tol)
            finish(st, ST_OK);
        else if (k == maxit)
            finish(st, ST_NOT_CONVERGED);
        else if (!(kappa > 0.0) || !isfinite(kappa))
            finish(st, ST_BREAKDOWN);
        else {
            st->beta = kappa / st->kappa_old;
            st->kappa_old = kappa;
        }
    }
    publish(st, hs, k);
}

// After the stencil pass: sigma = <p, A p>, alpha = kappa / sigma (the three
// alphas before it are kept for the deferred x updates).  x_steps >= 0: the
// pass brought x up to x_0 + sum of alpha_i p_i over i < x_steps.  After a
// breakdown here the alphas stay as they were, so that k_x_fixup finds the
// step lengths of the pending updates, and this step's is never applied.
__global__ __launch_bounds__(kRedThreads) void k_reduce_sigma(const double *__restrict__ partials,
                                                              int nparts, SolveState *st,
                                                              int iters_if_breakdown, int x_steps)
{
    if (st->done)
        return;
    double tot[1];
    sum_partials<1>(partials, nparts, 0, tot);
    if (threadIdx.x != 0)
        return;
    const double sigma = tot[0];
    st->sigma = sigma;
    if (x_steps >= 0)
        st->x_steps = x_steps;
    if (!(sigma > 0.0) || !isfinite(sigma)) {
        st->iters = iters_if_breakdown;
        finish(st, ST_BREAKDOWN);
    } else {
        st->alpha_prev3 = st->alpha_prev2;
        st->alpha_prev2 = st->alpha_prev;
        st->alpha_prev = st->alpha;
        st->alpha = st->kappa_old / sigma;
    }
}

// Standard loop, after x += alpha p, r -= alpha q: ||r_k|| and the stop test.
__global__ __launch_bounds__(kRedThreads) void k_reduce_rr(const double *__restrict__ partials,
                                                           int nparts, SolveState *st,
                                                           double *__restrict__ hist, int k,
                                                           int maxit, double tol, HostStatus *hs)
{
    if (st->done) {
        if (threadIdx.x == 0)
            publish(st, hs, k);
        return;
    }
    double tot[1];
    sum_partials<1>(partials, nparts, 0, tot);
    if (threadIdx.x != 0)
        return;
    const double R = sqrt(tot[0]);
    st->R = R;
    hist[k] = R;
    st->iters = k;
    if (!isfinite(R))
        finish(st, ST_BREAKDOWN);
    else if (R == 0.0 || R / st->R0 < tol)
        finish(st, ST_OK);
    else if (k == maxit)
        finish(st, ST_NOT_CONVERGED);
    publish(st, hs, k);
}

// Standard loop, after z = M^{-1} r: kappa = <r,z>, beta = kappa / kappa_old.
__global__ __launch_bounds__(kRedThreads) void k_reduce_kappa(const double *__restrict__ partials,
                                                              int nparts, SolveState *st)
{
    if (st->done)
        return;
    double tot[1];
    sum_partials<1>(partials, nparts, 1, tot);
    if (threadIdx.x != 0)
        return;
    const double kappa = tot[0];
    st->kappa = kappa;
    if (!(kappa > 0.0) || !isfinite(kappa)) {
        finish(st, ST_BREAKDOWN);
    } else {
        st->beta = kappa / st->kappa_old;
        st->kappa_old = kappa;
    }
}

// The search directions of the last steps of an interleaved solve: p_i is in
// p[i mod 4] (a two-buffer rotation passes its buffers twice).
template <typename T>
struct DirRing {
    const T *p[4];
};

// After the last step of an interleaved solve (Algorithm 1 leaves the loop
// once the stop test passes): the x updates the stencil passes deferred,
// x += alpha_i p_i for x_steps <= i < iters, one after the other in the order
// of i.  alpha_{iters-1} is st->alpha, the ones before it alpha_prev ..
// alpha_prev3; at most four updates are pending (the deferral is at most
// four steps).  Every element is read and written by one thread.
template <typename TV>
__global__ __launch_bounds__(256) void k_x_fixup(TV *__restrict__ x, DirRing<TV> ring,
                                                 const SolveState *__restrict__ st, size_t n)
{
    const int K = st->iters, A = st->x_steps;
    if (K <= A || K - A > 4)
        return;
    const TV al[4] = {(TV)st->alpha, (TV)st->alpha_prev, (TV)st->alpha_prev2, (TV)st->alpha_prev3};
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t l = (size_t)blockIdx.x * blockDim.x + threadIdx.x; l < n; l += stride) {
        TV v = x[l];
        for (int i = A; i < K; ++i)
            v = v + al[K - 1 - i] * ring.p[i & 3][l];
        x[l] = v;
    }
}

__global__ void k_init_state(SolveState *st)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        SolveState z = {};
        *st = z;
    }
}

}   // namespace mfpcg
