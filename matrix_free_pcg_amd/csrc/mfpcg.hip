// Host side of the matrix-free PCG library: argument checking, the handle,
// the workspace layout, kernel launches and the two PCG loops.  See
// include/mfpcg.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/mfpcg.h"
#include "kernels.hpp"

using namespace mfpcg;

namespace {

thread_local std::string g_create_error = "no error";

struct EventPair {
    hipEvent_t a, b;
    int kid;
    int tag;   // iteration index of the launch (or -1)
};

}   // namespace

struct pcg_handle {
    int device = 0;
    hipStream_t stream = nullptr;
    Op op{};
    int col_tiles = 0;     // workgroups of a column pass
    int col_threads = 0;   // threads per column-pass workgroup
    bool col_full = false; // every column tile whole (nx % 64 == 0, nz % L == 0, 64 columns)
    int colf_L = 0;        // column passes without a stored table: segment length (a multiple of L)
    int colf_threads = 0;  // ... threads per workgroup
    bool colf_full = false;// ... every tile whole
    int pt_tiles = 0;      // workgroups of a point pass
    bool pt_full = false;  // every sweep tile whole (nx % 64 == 0, nz % (Ws * Ls) == 0)
    int st_jt = 0;         // sweep passes on whole tiles: rows per tile of the fused passes
                           //   (0: 4 in binary64, 8 in binary32; 1: one row, and the
                           //   operator-only passes then take one row too)
    size_t n = 0;          // nx*ny*nz
    // device tables, carved from the caller's buffer (pcg_handle_bytes; for a
    // coarse level, from the buffer given to pcg_mg_setup): the library
    // allocates no device memory
    double *d_az = nullptr, *d_phib = nullptr;
    double *d_coef = nullptr;         // lev_a, lev_d (nz each), area, ex, ey (ny*nx each)
    float *d_phib32 = nullptr;        // boundary multipliers in binary32 (single-precision solves)
    int32_t overrides = 0;            // PCG_TUNE_* bits: tuning variables that changed the geometry
    CsrShape csr{};
    HostStatus *h_status = nullptr;   // pinned host memory written by the reduce kernels
    hipEvent_t loop_ev = nullptr;     // marks the stop decision of a step (created once)
    std::string err = "no error";
    bool profiling = false;
    int profile_period = 1;   // pcg_profile_enable's sampling period (1: every launch)
    double prof_ms[PCG_KID_COUNT] = {};
    int64_t prof_n[PCG_KID_COUNT] = {};
    std::vector<hipEvent_t> free_events;
    std::vector<EventPair> pending;
    // multigrid hierarchy (pcg_mg_setup): the coarse levels 1 .. nlev-1 are
    // handles of their own, owned by this one; mg_fx / mg_fy[l] are the
    // factors from level l to level l+1
    std::vector<pcg_handle *> mg_levels;
    std::vector<int> mg_fx, mg_fy;
    int mg_nu = 0, mg_coarse_sweeps = 0;
    double mg_omega = 0.0;
    double mg_coarse_lo = 0.0;        // > 0: Chebyshev-accelerated coarsest sweeps on [lo, 2]
};

namespace {

int fail(pcg_handle *h, int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (h)
        h->err = buf;
    else
        g_create_error = buf;
    return code;
}

#define HIP_TRY(h, call)                                                                     \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail((h), PCG_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));     \
    } while (0)

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// ---- the fixed scratch array of pcg_solve_static ------------------------------
// A file-scope device array that serves as the workspace of the solve entry
// point that allocates nothing.  Each device that loads the library holds its
// own copy until the process ends.  On the host the array's name is not a
// device address: host code uses only the address hipGetSymbolAddress
// returns, resolved once per device (with that device current) when the
// first handle on the device is created.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Resolve the array's address on `device`, which must be current.
int scratch_setup(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return fail(nullptr, PCG_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", device, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device])
        return PCG_OK;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return fail(nullptr, PCG_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", device,
                    hipGetErrorString(e));
    g_scratch_ptr[device] = ptr;
    return PCG_OK;
}

void *scratch_of(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

// Column-pass geometry: C columns per workgroup and the segment length L
// (default: the smallest of 8, 16, 32 with C * ceil(nz / L) <= 1024).
// Sweep-pass geometry: Ls levels per wave (1, 2, 4 or 8), Ws waves per
// workgroup (default Ls = 4, Ws = min(4, ceil(nz / 4))).  MFPCG_COL_L, MFPCG_COL_C, MFPCG_ST_L
// and MFPCG_ST_W override the choice (tuning); MFPCG_COL_FULL=0 and MFPCG_ST_FULL=0
// disable the whole-tile kernels; MFPCG_COL_STRIP and MFPCG_ST_STRIP set the
// i-strip widths of the tile order (default: one strip per XCD).
// The value of a tuning variable, or dflt when it is unset or empty; a set
// variable adds its PCG_TUNE_* bit to *seen (when seen is not null).
int env_int(const char *name, int dflt, int32_t *seen = nullptr, int32_t bit = 0)
{
    const char *v = getenv(name);
    if (!(v && *v))
        return dflt;
    if (seen)
        *seen |= bit;
    return atoi(v);
}

struct Geometry {
    int L, C, Ls, Ws;
    int Lf;   // segment length of the column passes that need no stored table (a multiple of L)
    int32_t overrides;   // PCG_TUNE_* bits of the variables read
};

bool choose_geometry(int nz, Geometry *g, std::string *why)
{
    g->overrides = 0;
    int32_t *ov = &g->overrides;
    g->C = env_int("MFPCG_COL_C", 64, ov, PCG_TUNE_COL_C);
    if (g->C != 32 && g->C != 64) { *why = "MFPCG_COL_C must be 32 or 64"; return false; }
    int l = env_int("MFPCG_COL_L", 0, ov, PCG_TUNE_COL_L);
    if (l == 0) {
        for (int cand : {8, 16, 32}) {
            if ((size_t)g->C * ((nz + cand - 1) / cand) <= (size_t)kMaxThreads) { l = cand; break; }
        }
        if (l == 0) { *why = "nz too large for the column solve"; return false; }
    }
    if (l != 4 && l != 8 && l != 16 && l != 32) { *why = "MFPCG_COL_L must be 4, 8, 16 or 32"; return false; }
    if ((size_t)g->C * ((nz + l - 1) / l) > (size_t)kMaxThreads) { *why = "column workgroup exceeds 1024 threads"; return false; }
    g->L = l;
    // Segments of 16 levels measured faster than 8 for the fused and the
    // stand-alone column passes at nz = 32..128 (their threads keep more loads
    // in flight; the multigrid sweeps and the recomputed-product column pass
    // need 8, so the table stays at L).
    // Whole segments are preferred: nz a multiple of 8 but not 16 keeps 8.
    int lf = env_int("MFPCG_COL_LF", 0, ov, PCG_TUNE_COL_LF);
    if (lf == 0) {
        lf = l;
        if (l == 8 && nz >= 16 && (nz % 16 == 0 || nz % 8 != 0) &&
            (size_t)g->C * ((nz + 15) / 16) <= (size_t)kMaxThreads)
            lf = 16;
    }
    if (lf != l && lf != 2 * l && lf != 4 * l) { *why = "MFPCG_COL_LF must be 1, 2 or 4 times the segment length"; return false; }
    if (lf > 32) { *why = "MFPCG_COL_LF must be at most 32"; return false; }
    g->Lf = lf;
    g->Ls = env_int("MFPCG_ST_L", 4, ov, PCG_TUNE_ST_L);
    if (g->Ls != 1 && g->Ls != 2 && g->Ls != 4 && g->Ls != 8) { *why = "MFPCG_ST_L must be 1, 2, 4 or 8"; return false; }
    const int need = (nz + g->Ls - 1) / g->Ls;
    g->Ws = env_int("MFPCG_ST_W", std::min(4, need), ov, PCG_TUNE_ST_W);
    if (g->Ws < 1 || g->Ws > 16) { *why = "MFPCG_ST_W must be in 1..16"; return false; }
    return true;
}

// Partial sums: a pass writes one pair per workgroup; above kDirect pairs a
// first stage folds them per 1024 into at most kStageMax pairs.
constexpr int kDirect = 4096;
constexpr int kStagePer = 1024;

int stage_blocks(int nparts) { return nparts <= kDirect ? 0 : (nparts + kStagePer - 1) / kStagePer; }

struct Workspace {
    double *r, *z, *p, *q, *p2, *p3, *p4, *partials, *stage, *hist;
    SolveState *state;
};

size_t workspace_layout(const pcg_handle *h, int32_t maxit, char *base, Workspace *w)
{
    const size_t vec = align256(h->n * sizeof(double));
    const int np = std::max(h->col_tiles, h->pt_tiles);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    size_t o_r = take(vec), o_z = take(vec), o_p = take(vec), o_q = take(vec), o_p2 = take(vec);
    size_t o_p3 = take(vec), o_p4 = take(vec);
    size_t o_part = take((size_t)np * 2 * sizeof(double));
    size_t o_stage = take((size_t)std::max(1, stage_blocks(np)) * 2 * sizeof(double));
    size_t o_state = take(sizeof(SolveState));
    size_t o_hist = take((size_t)(maxit + 1) * sizeof(double));
    if (w && base) {
        w->r = (double *)(base + o_r);
        w->z = (double *)(base + o_z);
        w->p = (double *)(base + o_p);
        w->q = (double *)(base + o_q);
        w->p2 = (double *)(base + o_p2);
        w->p3 = (double *)(base + o_p3);
        w->p4 = (double *)(base + o_p4);
        w->partials = (double *)(base + o_part);
        w->stage = (double *)(base + o_stage);
        w->state = (SolveState *)(base + o_state);
        w->hist = (double *)(base + o_hist);
    }
    return off;
}

// Fold `n` partial pairs to a count the single-workgroup reduce kernels read
// quickly; returns the array they should read and its length.
const double *fold_partials(pcg_handle *h, const Workspace &w, int n, int *n_out)
{
    const int nb = stage_blocks(n);
    if (nb == 0) {
        *n_out = n;
        return w.partials;
    }
    k_sum_stage<<<dim3(nb), dim3(kRedThreads), 0, h->stream>>>(w.partials, n, kStagePer, w.stage);
    *n_out = nb;
    return w.stage;
}

// Waits until a reduce kernel has published step k's stop decision in the
// pinned status block.  The kernel writes the block with system-scope stores,
// each finished before the next, the step index last; so once the host reads
// an index >= k, the decision beside it is that step's.  The caller must know
// that no earlier solve can still publish (the first step of a solve waits on
// an event instead, which drains everything queued before it).  The host
// spins; after 50 ms without the index, and every 50 ms after that, it asks
// the stream whether it failed, or drained without publishing (an error).
// Recording an event per step instead would hold the next kernel back by
// about 5.6 us (the runtime's marker packet).
int wait_published(pcg_handle *h, int k, const char *who)
{
    volatile HostStatus *vs = (volatile HostStatus *)h->h_status;
    if (vs->k >= k)
        return PCG_OK;
    const auto t0 = std::chrono::steady_clock::now();
    auto next = std::chrono::milliseconds(50);
    for (;;) {
        for (int i = 0; i < 4096; ++i) {
            if (vs->k >= k)
                return PCG_OK;
            __builtin_ia32_pause();
        }
        if (std::chrono::steady_clock::now() - t0 < next)
            continue;
        const hipError_t e = hipStreamQuery(h->stream);
        if (vs->k >= k)
            return PCG_OK;
        if (e == hipSuccess)
            return fail(h, PCG_ERR_HIP, "%s: the stream drained without publishing step %d", who, k);
        if (e != hipErrorNotReady)
            return fail(h, PCG_ERR_HIP, "%s: step %d: %s", who, k, hipGetErrorString(e));
        next += std::chrono::milliseconds(50);
    }
}

// ---- per-kernel event timing ------------------------------------------------
hipEvent_t take_event(pcg_handle *h)
{
    if (!h->free_events.empty()) {
        hipEvent_t e = h->free_events.back();
        h->free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

// A recorded event shows on the GPU's timeline as a gap of about 5.6 us
// before the next kernel, so with a period P > 1 the passes of the solve
// loops (tags >= 0: the step) are timed on four consecutive steps in every P
// (the stencil pass's forms in the proportion of a whole solve: x is updated
// every fourth step), the other launches every time.
constexpr int kProfileWindow = 4;
bool timed_launch(const pcg_handle *h, int kid, int tag)
{
    if (!h->profiling)
        return false;
    const bool loop_pass = kid == PCG_KID_FUSED_PREC || kid == PCG_KID_FUSED_SPMV || kid == PCG_KID_MG_VCYCLE;
    return !loop_pass || tag < 0 || h->profile_period <= 1 || tag % h->profile_period < kProfileWindow;
}

struct Timed {
    pcg_handle *h;
    EventPair ev{};
    bool on;
    Timed(pcg_handle *hh, int kid, int tag) : h(hh), on(timed_launch(hh, kid, tag))
    {
        if (!on) return;
        ev.a = take_event(h);
        ev.b = take_event(h);
        ev.kid = kid;
        ev.tag = tag;
        if (!ev.a || !ev.b) { on = false; return; }
        (void)hipEventRecord(ev.a, h->stream);
    }
    ~Timed()
    {
        if (!on) return;
        (void)hipEventRecord(ev.b, h->stream);
        h->pending.push_back(ev);
    }
};

// Fold the recorded event pairs into the totals (the stream must be idle).
// Launches tagged `skip_tag` of kernel `skip_kid` are dropped (the final
// stencil pass of a solve, launched before the stop test was read: it returns at once).
void drain_events(pcg_handle *h, int skip_kid = -1, int skip_tag = -2)
{
    for (auto &e : h->pending) {
        float ms = 0.f;
        if (!(e.kid == skip_kid && e.tag == skip_tag) && hipEventElapsedTime(&ms, e.a, e.b) == hipSuccess) {
            h->prof_ms[e.kid] += ms;
            h->prof_n[e.kid] += 1;
        }
        h->free_events.push_back(e.a);
        h->free_events.push_back(e.b);
    }
    h->pending.clear();
}

// ---- launch helpers (template dispatch on the column geometry) ---------------
// TV: type of r, q (and of the stencil pass's vectors); TZ: type of z and of
// the column solve.  <double, double> is the binary64 solver; <float, float>
// and <double, float> only need the fused preconditioner pass and the
// stand-alone solve.
template <typename T> const T *phib_of(const pcg_handle *h);
template <> const double *phib_of<double>(const pcg_handle *h) { return h->d_phib; }
template <> const float *phib_of<float>(const pcg_handle *h) { return h->d_phib32; }

template <typename TV, typename TZ>
constexpr bool kBinary64 = std::is_same<TV, double>::value && std::is_same<TZ, double>::value;

// Segmentation of one column pass: the operator with its segment length,
// segment count and multiplier-table stride, and the workgroup shape.
struct ColGeo {
    Op o;
    int threads;
    bool full;
};

// The passes with a stored column matrix use the handle's segments (their
// multiplier table is computed for them); the others use colf_L, reading
// the handle's table at every (colf_L / L)-th boundary.
ColGeo col_geo(const pcg_handle *h, bool stored)
{
    ColGeo g{h->op, h->col_threads, h->col_full};
    if (!stored && h->colf_L != h->op.L) {
        g.o.L = h->colf_L;
        g.o.P = (h->op.nz + h->colf_L - 1) / h->colf_L;
        g.o.pst = h->colf_L / h->op.L;
        g.threads = h->colf_threads;
        g.full = h->colf_full;
    }
    return g;
}

template <int L, int C, typename TV, typename TZ>
void launch_column_lc(pcg_handle *h, const ColGeo &g, const TV *rin, const TV *q, TV *rout, TZ *z,
                      const SolveState *st, int first, double *partials, int upd, bool dots,
                      const double *tri)
{
    dim3 grid(h->col_tiles), block(g.threads);
    const Op &o = g.o;
    const TZ *phib = phib_of<TZ>(h);
    constexpr bool kD = kBinary64<TV, TZ>;
    if constexpr (C == kWave) {
        if (!tri && g.full) {
            if (upd == UPD_Q)
                k_column_full<L, UPD_Q, true, TV, TZ><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, phib, MgArgs{});
            else if (!dots)
                k_column_full<L, UPD_NONE, false, TV, TZ><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, phib, MgArgs{});
            else if constexpr (kD) {
                if (upd == UPD_AP)
                    k_column_full<L, UPD_AP, true><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, phib, MgArgs{});
                else
                    k_column_full<L, UPD_NONE, true><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, phib, MgArgs{});
            }
            return;
        }
    }
    if constexpr (kD) {
        if (tri) {
            if (dots)
                k_column_solve<L, C, UPD_NONE, true, true><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, tri, tri + 3 * h->n, MgArgs{});
            else
                k_column_solve<L, C, UPD_NONE, false, true><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, tri, tri + 3 * h->n, MgArgs{});
            return;
        }
    }
    if (upd == UPD_Q)
        k_column_solve<L, C, UPD_Q, true, false, TV, TZ><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, nullptr, phib, MgArgs{});
    else if (!dots)
        k_column_solve<L, C, UPD_NONE, false, false, TV, TZ><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, nullptr, phib, MgArgs{});
    else if constexpr (kD) {
        if (upd == UPD_AP)
            k_column_solve<L, C, UPD_AP, true, false><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, nullptr, phib, MgArgs{});
        else
            k_column_solve<L, C, UPD_NONE, true, false><<<grid, block, 0, h->stream>>>(rin, q, rout, z, o, st, first, partials, nullptr, phib, MgArgs{});
    }
}

template <int C, typename TV, typename TZ>
void launch_column_c(pcg_handle *h, const TV *rin, const TV *q, TV *rout, TZ *z,
                     const SolveState *st, int first, double *partials, int upd, bool dots,
                     const double *tri)
{
    // the recomputed-product form keeps the table's segments: with 16 levels
    // its operand arrays spill (1.65 ms per pass at 1024 x 1024 x 128, 1.18
    // with 8)
    const ColGeo g = col_geo(h, tri != nullptr || upd == UPD_AP);
    switch (g.o.L) {
    case 4: launch_column_lc<4, C>(h, g, rin, q, rout, z, st, first, partials, upd, dots, tri); break;
    case 8: launch_column_lc<8, C>(h, g, rin, q, rout, z, st, first, partials, upd, dots, tri); break;
    case 16: launch_column_lc<16, C>(h, g, rin, q, rout, z, st, first, partials, upd, dots, tri); break;
    default: launch_column_lc<32, C>(h, g, rin, q, rout, z, st, first, partials, upd, dots, tri); break;
    }
}

// z = M^{-1} r; upd selects the fused residual update (UPD_*); tri != nullptr
// selects the stored (explicit) column matrices (binary64 only).
template <typename TV, typename TZ>
void column(pcg_handle *h, const TV *rin, const TV *q, TV *rout, TZ *z,
            const SolveState *st, int first, double *partials, int upd, bool dots,
            const double *tri = nullptr)
{
    if (h->op.C == 64)
        launch_column_c<64>(h, rin, q, rout, z, st, first, partials, upd, dots, tri);
    else
        launch_column_c<32>(h, rin, q, rout, z, st, first, partials, upd, dots, tri);
}

// TV: the vectors' type; TI: the stencil operand's (z from a TZ column pass,
// or x).  <double, double> has every mode; <float, float> the modes of the
// single-precision solve and apply_A; <double, float> the stencil passes of
// the solve with a binary32 preconditioner.
template <int Ls, bool FULL, typename TV, typename TI>
void launch_stencil_f(pcg_handle *h, const Op &o, int mode, const TI *zin, const TV *b, TV *u, TV *p, TV *y,
                      const SolveState *st, double *partials, TV *p_out, Older<TV> older)
{
    dim3 grid(h->pt_tiles), block(kWave * o.Ws);
    constexpr bool kSame = std::is_same<TV, TI>::value;
    constexpr bool kD = kBinary64<TV, TI>;
    switch (mode) {
    case SP_FIRST: k_stencil<Ls, SP_FIRST, FULL, TV, TI><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
    case SP_FUSED_NOX: k_stencil<Ls, SP_FUSED_NOX, FULL, TV, TI><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
    case SP_FUSED_X4: k_stencil<Ls, SP_FUSED_X4, FULL, TV, TI><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
    case SP_APPLY:
        if constexpr (kSame)
            k_stencil<Ls, SP_APPLY, FULL, TV, TI><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older);
        break;
    case SP_RESID:
        if constexpr (kSame)
            k_stencil<Ls, SP_RESID, FULL, TV, TI><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older);
        break;
    case SP_APPLY_DOT:
        if constexpr (kD)
            k_stencil<Ls, SP_APPLY_DOT, FULL><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older);
        break;
    case SP_FIRST_AP:
        if constexpr (kD)
            k_stencil<Ls, SP_FIRST_AP, FULL><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older);
        break;
    default:
        if constexpr (kD)
            k_stencil<Ls, SP_FUSED_AP, FULL><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older);
        break;
    }
}

// Whole tiles of JT rows x Ls levels, one wave per row (k_stencil with JT).
template <int Ls, int JT, typename TV, typename TI>
void launch_stencil_jt(pcg_handle *h, const Op &o, int mode, const TI *zin, const TV *b, TV *u, TV *p,
                       TV *y, const SolveState *st, double *partials, TV *p_out, Older<TV> older)
{
    constexpr bool kSame = std::is_same<TV, TI>::value;
    dim3 grid((unsigned)((size_t)o.ntx * o.nkt * (o.ny / JT))), block(kWave * JT);
    if constexpr (Ls == 4) {   // the fused passes
        switch (mode) {
        case SP_FIRST: k_stencil<Ls, SP_FIRST, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
        case SP_FUSED_NOX: k_stencil<Ls, SP_FUSED_NOX, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
        case SP_FUSED_X4: k_stencil<Ls, SP_FUSED_X4, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
        default: break;
        }
    }
    // the pass that defers x with 8 levels per wave, on 4 or 8 rows
    if constexpr (Ls == 8 && (((JT == 4 || JT == 8) && kBinary64<TV, TI>) ||
                              (std::is_same<TV, float>::value && kSame && (JT == 4 || JT == 8)))) {
        if (mode == SP_FUSED_NOX)
            k_stencil<Ls, SP_FUSED_NOX, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older);
    }
    if constexpr (kSame && Ls == 8) {   // the operator-only passes
        switch (mode) {
        case SP_APPLY: k_stencil<Ls, SP_APPLY, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
        case SP_RESID: k_stencil<Ls, SP_RESID, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
        case SP_APPLY_DOT: k_stencil<Ls, SP_APPLY_DOT, true, TV, TI, JT><<<grid, block, 0, h->stream>>>(zin, b, u, p, y, o, st, partials, p_out, older); break;
        default: break;
        }
    }
}

// Tiles of the sweep passes.  On whole tiles (4 waves of 4 levels by
// default) the passes take row tiles, one wave per row j, the rows j +- 1
// inside a tile coming through LDS instead of the L2 (the fused pass
// 1.222 -> 1.170 ms at 1024 x 1024 x 128); otherwise one-row tiles of
// Ws x Ls levels.  The passes that apply the operator alone (y = A x,
// q = A p with <p,q>, r = b - A x) move one stream in and one out; with 4
// levels per wave they are latency-bound, so they sweep 8 levels per wave
// (13 % faster on one-row tiles).  stencil_tiles gives each pass's partial
// count.

// Rows per tile of the fused stencil passes (SP_FIRST, SP_FUSED_NOX,
// SP_FUSED_X4) on this handle, 0 when they take one-row tiles.  Measured at
// 1024 x 1024 x 128: 4 rows best in binary64 and the mixed solve (8 rows:
// 1.2 % and 6 % slower), 8 rows in binary32 (2.5 % faster than 4).
int fused_rows_jt(const pcg_handle *h, bool binary32)
{
    const Op &o = h->op;
    const int jt = h->st_jt ? h->st_jt : (binary32 ? 8 : 4);
    return jt > 1 && h->pt_full && o.Ls == 4 && o.Ws == 4 && o.ny % jt == 0 ? jt : 0;
}

// Rows per tile of the operator-only passes (SP_APPLY, SP_APPLY_DOT,
// SP_RESID; 8 levels per wave) on this handle, 0 when they take one-row
// tiles.  y = A x at 1024 x 1024 x 128: one row 0.541 ms, 2 rows 0.471 ms,
// 4 rows 0.439 ms (later 0.407), 8 rows 0.394 ms.
int op_rows_jt(const pcg_handle *h)
{
    const Op &o = h->op;
    if (h->st_jt == 1 || !h->pt_full || o.Ls != 4 || o.Ws != 4)
        return 0;
    return o.ny % 8 == 0 ? 8 : (o.ny % 4 == 0 ? 4 : (o.ny % 2 == 0 ? 2 : 0));
}

// Row-tile shape of a fused pass: levels per wave and rows (0 rows: one-row
// tiles).  The pass that defers x takes 8 levels per wave in binary64 (4 x 8
// tiles: 0.5 % faster than 4 x 4; in the mixed solve 1.8 % slower; on 8 rows
// where ny allows and no row count is forced, the binary64 solve another
// 0.5 % faster, while 8 rows for the fourth-step form cost 0.8 %) and in
// binary32 (8 x 8 tiles: the binary32 solve 1.8 % faster than with 8 x 4;
// 8 levels on 4 rows gain 0.3 %).
struct RowShape {
    int Ls, jt;
};
RowShape fused_shape(const pcg_handle *h, int mode, bool binary64, bool binary32)
{
    const int jt = fused_rows_jt(h, binary32);
    if (!jt)
        return {4, 0};
    if (binary64 && jt == 4 && mode == SP_FUSED_NOX)
        return {8, (!h->st_jt && h->op.ny % 8 == 0) ? 8 : 4};
    if (binary32 && (jt == 4 || jt == 8) && mode == SP_FUSED_NOX)
        return {8, jt};
    return {4, jt};
}

// Partial sums (tiles) of a stencil pass of this mode.
int stencil_tiles(const pcg_handle *h, int mode, bool binary64, bool binary32)
{
    if (mode == SP_FIRST || mode == SP_FUSED_NOX || mode == SP_FUSED_X4) {
        const RowShape rs = fused_shape(h, mode, binary64, binary32);
        if (rs.jt)
            return (int)((size_t)h->op.ntx * (h->op.nz / rs.Ls) * (h->op.ny / rs.jt));
    }
    if (mode == SP_APPLY_DOT && op_rows_jt(h) >= 4)
        return (int)((size_t)h->op.ntx * (h->op.nz / 8) * (h->op.ny / op_rows_jt(h)));
    return h->pt_tiles;
}

template <int Ls, typename TV, typename TI>
void launch_stencil(pcg_handle *h, int mode, const TI *zin, const TV *b, TV *u, TV *p, TV *y,
                    const SolveState *st, double *partials, TV *p_out, Older<TV> older)
{
    if constexpr (Ls == 4) {
        const bool op_only = mode == SP_APPLY || mode == SP_APPLY_DOT || mode == SP_RESID;
        const bool fused_rows = mode == SP_FIRST || mode == SP_FUSED_NOX || mode == SP_FUSED_X4;
        const RowShape rs = fused_rows ? fused_shape(h, mode, kBinary64<TV, TI>,
                                                     std::is_same<TV, float>::value && std::is_same<TI, float>::value)
                                       : RowShape{4, 0};
        if (rs.jt) {
            Op o2 = h->op;
            o2.Ls = rs.Ls;
            o2.jt = rs.jt;
            o2.Ws = rs.jt;
            o2.nkt = h->op.nz / rs.Ls;
            if (rs.Ls == 8 && rs.jt == 8)
                launch_stencil_jt<8, 8>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            else if (rs.Ls == 8)
                launch_stencil_jt<8, 4>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            else if (rs.jt == 8)
                launch_stencil_jt<4, 8>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            else
                launch_stencil_jt<4, 4>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            return;
        }
        const int ojt = op_rows_jt(h);
        if (op_only && ojt) {
            Op o2 = h->op;
            o2.Ls = 8;
            o2.Ws = ojt;
            o2.jt = ojt;
            o2.nkt = h->op.nz / 8;
            if (ojt == 8)
                launch_stencil_jt<8, 8>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            else if (ojt == 4)
                launch_stencil_jt<8, 4>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            else
                launch_stencil_jt<8, 2>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            return;
        }
        if (op_only && h->op.Ws % 2 == 0) {
            Op o2 = h->op;
            o2.Ls = 8;
            o2.Ws = h->op.Ws / 2;
            if (h->pt_full)
                launch_stencil_f<8, true>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            else
                launch_stencil_f<8, false>(h, o2, mode, zin, b, u, p, y, st, partials, p_out, older);
            return;
        }
    }
    if (h->pt_full)
        launch_stencil_f<Ls, true>(h, h->op, mode, zin, b, u, p, y, st, partials, p_out, older);
    else
        launch_stencil_f<Ls, false>(h, h->op, mode, zin, b, u, p, y, st, partials, p_out, older);
}

template <typename TV, typename TI>
void stencil(pcg_handle *h, int mode, const TI *zin, const TV *b, TV *u, TV *p, TV *y,
             const SolveState *st, double *partials, TV *p_out = nullptr, Older<TV> older = {})
{
    switch (h->op.Ls) {
    case 1: launch_stencil<1>(h, mode, zin, b, u, p, y, st, partials, p_out, older); break;
    case 2: launch_stencil<2>(h, mode, zin, b, u, p, y, st, partials, p_out, older); break;
    case 4: launch_stencil<4>(h, mode, zin, b, u, p, y, st, partials, p_out, older); break;
    default: launch_stencil<8>(h, mode, zin, b, u, p, y, st, partials, p_out, older); break;
    }
}

template <int Ls>
void launch_vec(pcg_handle *h, int which, double *x, const double *p, double *r, const double *q,
                const SolveState *st, double *partials, int first)
{
    dim3 grid(h->pt_tiles), block(kWave * h->op.Ws);
    if (which == 0)
        k_update_xr<Ls><<<grid, block, 0, h->stream>>>(x, p, r, q, h->op, st, partials);
    else
        k_update_p<Ls><<<grid, block, 0, h->stream>>>(r, q, h->op, st, first);
}

void vec(pcg_handle *h, int which, double *x, const double *p, double *r, const double *q,
         const SolveState *st, double *partials, int first)
{
    switch (h->op.Ls) {
    case 1: launch_vec<1>(h, which, x, p, r, q, st, partials, first); break;
    case 2: launch_vec<2>(h, which, x, p, r, q, st, partials, first); break;
    case 4: launch_vec<4>(h, which, x, p, r, q, st, partials, first); break;
    default: launch_vec<8>(h, which, x, p, r, q, st, partials, first); break;
    }
}

void update_xr(pcg_handle *h, double *x, const double *p, double *r, const double *q,
               const SolveState *st, double *partials)
{
    vec(h, 0, x, p, r, q, st, partials, 0);
}

// p = z + beta p: the second kernel takes (p, z) in the (r, q) slots.
void update_p(pcg_handle *h, double *p, const double *z, const SolveState *st, int first)
{
    vec(h, 1, nullptr, nullptr, p, z, st, nullptr, first);
}

void csr_spmv(pcg_handle *h, int mode, const int64_t *rp, const int32_t *col, const double *val,
              const double *x, const double *b, double *y, const SolveState *st, double *partials)
{
    dim3 grid(h->pt_tiles), block(kWave * h->op.Ws);
    if (mode == CSR_APPLY)
        k_csr_spmv<CSR_APPLY><<<grid, block, 0, h->stream>>>(rp, col, val, x, b, y, h->op, st, partials);
    else if (mode == CSR_RESID)
        k_csr_spmv<CSR_RESID><<<grid, block, 0, h->stream>>>(rp, col, val, x, b, y, h->op, st, partials);
    else
        k_csr_spmv<CSR_APPLY_DOT><<<grid, block, 0, h->stream>>>(rp, col, val, x, b, y, h->op, st, partials);
}

void csr_assemble(pcg_handle *h, int64_t *rp, int32_t *col, double *val)
{
    dim3 grid(h->pt_tiles), block(kWave * h->op.Ws);
    switch (h->op.Ls) {
    case 1: k_csr_assemble<1><<<grid, block, 0, h->stream>>>(h->op, h->csr, rp, col, val); break;
    case 2: k_csr_assemble<2><<<grid, block, 0, h->stream>>>(h->op, h->csr, rp, col, val); break;
    case 4: k_csr_assemble<4><<<grid, block, 0, h->stream>>>(h->op, h->csr, rp, col, val); break;
    default: k_csr_assemble<8><<<grid, block, 0, h->stream>>>(h->op, h->csr, rp, col, val); break;
    }
}

int64_t csr_nnz(const pcg_handle *h)
{
    const int64_t ncol = (int64_t)h->op.nx * h->op.ny;
    const int64_t V = 2 * (int64_t)h->op.nz - 2;
    return (int64_t)h->n * h->csr.base + ncol * V;
}

int check_vectors(pcg_handle *h, const void *a, const void *b, const char *what,
                  size_t elem = sizeof(double))
{
    if (!a || !b)
        return fail(h, PCG_ERR_INVALID, "%s: null device pointer", what);
    const size_t bytes = h->n * elem;
    const char *pa = (const char *)a, *pb = (const char *)b;
    if (pa < pb + bytes && pb < pa + bytes)
        return fail(h, PCG_ERR_INVALID, "%s: input and output overlap", what);
    return PCG_OK;
}

int set_device(pcg_handle *h)
{
    HIP_TRY(h, hipSetDevice(h->device));
    return PCG_OK;
}

struct SolveArgs {
    const void *b;   // device vectors of elem-byte elements
    void *x;
    size_t elem;
    double tol;
    int32_t maxit;
    void *ws;
    size_t ws_bytes;
    int32_t *iters_out;
    double *hist_host;
    int32_t *hist_len_out;
    double *final_rel;
};

size_t mg_layout(const pcg_handle *h, int32_t maxit, char *base, Workspace *w, struct MgWork *mw);

int solve_prologue(pcg_handle *h, const SolveArgs &a, Workspace *w, const char *who, bool mg = false)
{
    if (!h)
        return PCG_ERR_INVALID;
    if (a.maxit < 0)
        return fail(h, PCG_ERR_INVALID, "%s: maxit must be >= 0", who);
    if (std::isnan(a.tol))
        return fail(h, PCG_ERR_INVALID, "%s: tol is NaN", who);
    int rc = check_vectors(h, a.b, a.x, who, a.elem);
    if (rc != PCG_OK)
        return rc;
    if (!a.ws)
        return fail(h, PCG_ERR_INVALID, "%s: null workspace", who);
    if (((uintptr_t)a.ws & 255u) != 0)
        return fail(h, PCG_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
    const size_t need = mg ? mg_layout(h, a.maxit, nullptr, nullptr, nullptr)
                           : workspace_layout(h, a.maxit, nullptr, nullptr);
    if (a.ws_bytes < need)
        return fail(h, PCG_ERR_INVALID, "%s: workspace has %zu bytes, needs %zu", who, a.ws_bytes, need);
    const char *ws = (const char *)a.ws, *xb = (const char *)a.x;
    const size_t vb = h->n * a.elem;
    if (xb < ws + need && ws < xb + vb)
        return fail(h, PCG_ERR_INVALID, "%s: x overlaps the workspace", who);
    const char *bb = (const char *)a.b;
    if (bb < ws + need && ws < bb + vb)
        return fail(h, PCG_ERR_INVALID, "%s: b overlaps the workspace", who);
    rc = set_device(h);
    if (rc != PCG_OK)
        return rc;
    workspace_layout(h, a.maxit, (char *)a.ws, w);
    return PCG_OK;
}

int solve_epilogue(pcg_handle *h, const SolveArgs &a, const Workspace &w, int skip_kid, int skip_tag)
{
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    HIP_TRY(h, hipGetLastError());
    if (h->profiling)
        drain_events(h, skip_kid, skip_tag);
    SolveState st;
    HIP_TRY(h, hipMemcpy(&st, w.state, sizeof st, hipMemcpyDeviceToHost));
    const int iters = st.iters;
    if (a.iters_out)
        *a.iters_out = iters;
    if (a.hist_host && iters >= 0) {
        const int cnt = (st.status == ST_BREAKDOWN && iters == 0 && !std::isfinite(st.R0)) ? 1 : iters + 1;
        HIP_TRY(h, hipMemcpy(a.hist_host, w.hist, (size_t)cnt * sizeof(double), hipMemcpyDeviceToHost));
        if (a.hist_len_out)
            *a.hist_len_out = cnt;
    } else if (a.hist_len_out) {
        *a.hist_len_out = iters + 1;
    }
    if (a.final_rel) {
        double hk = 0.0;
        HIP_TRY(h, hipMemcpy(&hk, w.hist + iters, sizeof(double), hipMemcpyDeviceToHost));
        *a.final_rel = (st.R0 == 0.0) ? 0.0 : hk / st.R0;
    }
    if (st.status == ST_OK)
        return PCG_OK;
    if (st.status == ST_NOT_CONVERGED)
        return PCG_NOT_CONVERGED;
    return fail(h, PCG_ERR_BREAKDOWN, "PCG breakdown after %d steps (sigma = %g, kappa = %g, |r| = %g)",
                iters, st.sigma, st.kappa, st.R);
}

}   // namespace

// ============================================================================
extern "C" {

const char *pcg_version(void) { return "mfpcg 0.1 (gfx950, fp64)"; }

const char *pcg_last_error(const pcg_handle *h)
{
    return h ? h->err.c_str() : g_create_error.c_str();
}

int32_t pcg_tuning_overrides(const pcg_handle *h)
{
    return h ? h->overrides : 0;
}

}   // extern "C"

namespace {

// The operator in the general form the kernels read (see Op in kernels.hpp).
struct HostCoeffs {
    std::vector<double> a, d, beta, area, ex, ey;
};

// Geometry checks shared by both create functions.
int check_grid(const char *who, const pcg_grid *grid, Geometry *g)
{
    const int nx = grid->nx, ny = grid->ny, nz = grid->nz;
    if (nx < 1 || ny < 1 || nz < 1)
        return fail(nullptr, PCG_ERR_INVALID, "%s: grid %d x %d x %d must be positive", who, nx, ny, nz);
    if (nz > 512)
        return fail(nullptr, PCG_ERR_UNSUPPORTED, "%s: nz = %d > 512 is not supported", who, nz);
    std::string why;
    if (!choose_geometry(nz, g, &why))
        return fail(nullptr, PCG_ERR_UNSUPPORTED, "%s: %s (nz = %d)", who, why.c_str(), nz);
    const size_t ntx = ((size_t)nx + kWave - 1) / kWave;
    const size_t ntc = ((size_t)nx + g->C - 1) / g->C;
    const size_t nkt = ((size_t)nz + (size_t)g->Ls * g->Ws - 1) / ((size_t)g->Ls * g->Ws);
    if (ntx * nkt * (size_t)ny > (size_t)0x7fffffff || ntc * (size_t)ny > (size_t)0x7fffffff)
        return fail(nullptr, PCG_ERR_UNSUPPORTED, "%s: too many tiles", who);
    return PCG_OK;
}

// Each entry of v[0..n) finite and >= lo (strictly > lo when strict).
int check_array(const char *who, const char *name, const double *v, size_t n, bool strict)
{
    if (!v)
        return fail(nullptr, PCG_ERR_INVALID, "%s: %s is NULL", who, name);
    for (size_t t = 0; t < n; ++t) {
        const double x = v[t];
        if (!std::isfinite(x) || (strict ? !(x > 0.0) : !(x >= 0.0)))
            return fail(nullptr, PCG_ERR_INVALID, "%s: %s[%zu] = %g must be finite and %s 0", who, name, t, x,
                        strict ? ">" : ">=");
    }
    return PCG_OK;
}

// Launch geometry of one level (see Op and the kernels' decompositions).
void init_geometry(pcg_handle *h, int nx, int ny, int nz, const Geometry &g)
{
    const int L = g.L, C = g.C;
    const size_t ntx = ((size_t)nx + kWave - 1) / kWave;
    const size_t ntc = ((size_t)nx + C - 1) / C;
    const size_t nkt = ((size_t)nz + (size_t)g.Ls * g.Ws - 1) / ((size_t)g.Ls * g.Ws);
    const size_t ncol = (size_t)nx * ny;
    const int P = (nz + L - 1) / L;
    h->col_tiles = (int)(ntc * ny);
    h->col_threads = ((C * P + kWave - 1) / kWave) * kWave;
    int32_t ov = g.overrides;
    const bool col_whole = env_int("MFPCG_COL_FULL", 1, &ov, PCG_TUNE_COL_FULL) != 0;
    h->col_full = C == kWave && nx % kWave == 0 && nz % L == 0 && col_whole;
    h->colf_L = g.Lf;
    h->colf_threads = ((C * ((nz + g.Lf - 1) / g.Lf) + kWave - 1) / kWave) * kWave;
    h->colf_full = C == kWave && nx % kWave == 0 && nz % g.Lf == 0 && col_whole;
    h->pt_tiles = (int)(ntx * nkt * ny);
    h->pt_full = nx % kWave == 0 && nz % (g.Ls * g.Ws) == 0 &&
                 env_int("MFPCG_ST_FULL", 1, &ov, PCG_TUNE_ST_FULL) != 0;
    {   // MFPCG_ST_JT: rows per fused-pass tile, 1 (one-row tiles), 4 or 8 (see launch_stencil)
        const int jt = env_int("MFPCG_ST_JT", 0, &ov, PCG_TUNE_ST_JT);
        h->st_jt = (jt == 1 || jt == 4 || jt == 8) ? jt : 0;
    }
    h->n = ncol * (size_t)nz;
    h->op.nx = nx;
    h->op.ny = ny;
    h->op.nz = nz;
    h->op.L = L;
    h->op.P = P;
    h->op.C = C;
    h->op.pst = 1;
    h->op.jt = 1;
    h->op.ntc = (int)ntc;
    h->csr.hx = nx == 1 ? 0 : (nx == 2 ? 1 : 2);
    h->csr.hy = ny == 1 ? 0 : (ny == 2 ? 1 : 2);
    h->csr.base = 1 + h->csr.hx + h->csr.hy;
    h->op.Ls = g.Ls;
    h->op.Ws = g.Ws;
    h->op.nkt = (int)nkt;
    h->op.ntx = (int)ntx;
    // one strip of i-tiles per XCD (MFPCG_ST_STRIP overrides; 1 = i-tile slowest)
    h->op.sg = std::max(1, std::min((int)ntx, env_int("MFPCG_ST_STRIP", (int)((ntx + kXcds - 1) / kXcds),
                                                      &ov, PCG_TUNE_ST_STRIP)));
    h->op.csg = std::max(1, std::min((int)ntc, env_int("MFPCG_COL_STRIP", (int)((ntc + kXcds - 1) / kXcds),
                                                       &ov, PCG_TUNE_COL_STRIP)));
    h->overrides = ov;
}

// Device tables of a level: the nz+1 vertical faces, per-level a and d and
// per-column |T| and the two edge coefficients, the segment-boundary Thomas
// multipliers in binary64 and binary32; each part 256-byte aligned.  Returns
// the bytes; with base and h set, points h's tables (and its Op) into base.
size_t table_layout(int nx, int ny, int nz, int P, char *base, pcg_handle *h)
{
    const size_t ncol = (size_t)nx * ny;
    const size_t nb = ncol * (size_t)(P > 1 ? P - 1 : 1);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t o_az = take(sizeof(double) * ((size_t)nz + 1));
    const size_t o_coef = take(sizeof(double) * (2 * (size_t)nz + 3 * ncol));
    const size_t o_phib = take(sizeof(double) * nb);
    const size_t o_phib32 = take(sizeof(float) * nb);
    if (base && h) {
        h->d_az = (double *)(base + o_az);
        h->d_coef = (double *)(base + o_coef);
        h->d_phib = (double *)(base + o_phib);
        h->d_phib32 = (float *)(base + o_phib32);
        h->op.az = h->d_az;
        h->op.lev_a = h->d_coef;
        h->op.lev_d = h->d_coef + nz;
        h->op.area = h->d_coef + 2 * (size_t)nz;
        h->op.ex = h->op.area + ncol;
        h->op.ey = h->op.ex + ncol;
        h->op.phib = h->d_phib;
    }
    return off;
}

// Check a caller-provided device buffer of at least `need` bytes.
int check_buffer(pcg_handle *h, const char *who, const char *what, const void *buf, size_t bytes, size_t need)
{
    if (!buf)
        return fail(h, PCG_ERR_INVALID, "%s: %s is NULL", who, what);
    if (((uintptr_t)buf & 255u) != 0)
        return fail(h, PCG_ERR_INVALID, "%s: %s must be 256-byte aligned", who, what);
    if (bytes < need)
        return fail(h, PCG_ERR_INVALID, "%s: %s has %zu bytes, needs %zu", who, what, bytes, need);
    return PCG_OK;
}

// The Thomas multipliers at the segment boundaries (binary64 and binary32
// tables), then wait for the set-up to finish.
int setup_multipliers(pcg_handle *h, const char *who)
{
    const size_t ncol = (size_t)h->op.nx * h->op.ny;
    if (h->op.P > 1) {
        const int threads = 256;
        const size_t blocks = (ncol + threads - 1) / threads;
        k_setup_phib<double><<<dim3((unsigned)blocks), dim3(threads), 0, h->stream>>>(h->op, h->d_phib);
        k_setup_phib<float><<<dim3((unsigned)blocks), dim3(threads), 0, h->stream>>>(h->op, h->d_phib32);
    }
    hipError_t e;
    if ((e = hipStreamSynchronize(h->stream)) != hipSuccess || (e = hipGetLastError()) != hipSuccess) {
        h->err = std::string(who) + ": set-up failed: " + hipGetErrorString(e);
        return PCG_ERR_HIP;
    }
    return PCG_OK;
}

// Create the handle in the caller's table buffer, copy the coefficients and
// compute the Thomas multipliers at the segment boundaries (binary64 and
// binary32 tables).
int create_handle(const char *who, const pcg_grid *grid, const Geometry &g, const HostCoeffs &hc,
                  void *hip_stream, void *tables, size_t tables_bytes, pcg_handle **out)
{
    const int nx = grid->nx, ny = grid->ny, nz = grid->nz;
    const size_t ncol = (size_t)nx * ny;
    const size_t need = table_layout(nx, ny, nz, (nz + g.L - 1) / g.L, nullptr, nullptr);
    int rc = check_buffer(nullptr, who, "tables_dev", tables, tables_bytes, need);
    if (rc != PCG_OK)
        return rc;
    pcg_handle *h = new pcg_handle();
    auto bail = [&](int code) {
        g_create_error = h->err;
        pcg_destroy(h);
        return code;
    };
    if (hipGetDevice(&h->device) != hipSuccess) {
        h->err = std::string(who) + ": hipGetDevice failed";
        return bail(PCG_ERR_HIP);
    }
    h->stream = (hipStream_t)hip_stream;
    init_geometry(h, nx, ny, nz, g);
    table_layout(nx, ny, nz, h->op.P, (char *)tables, h);
    hipError_t e;
    if ((e = hipHostMalloc((void **)&h->h_status, sizeof(HostStatus), hipHostMallocCoherent)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h->loop_ev, hipEventDisableTiming)) != hipSuccess) {
        h->h_status = nullptr;
        h->err = std::string(who) + ": pinned status word / event: " + hipGetErrorString(e);
        return bail(PCG_ERR_HIP);
    }
    memset(h->h_status, 0, sizeof(HostStatus));
    if ((rc = scratch_setup(h->device)) != PCG_OK) {
        h->err = g_create_error;
        return bail(rc);
    }
    const size_t ncoef = 2 * (size_t)nz + 3 * ncol;
    std::vector<double> coef;
    coef.reserve(ncoef);
    for (const auto *v : {&hc.a, &hc.d, &hc.area, &hc.ex, &hc.ey})
        coef.insert(coef.end(), v->begin(), v->end());
    if ((e = hipMemcpy(h->d_az, hc.beta.data(), sizeof(double) * (nz + 1), hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(h->d_coef, coef.data(), sizeof(double) * ncoef, hipMemcpyHostToDevice)) != hipSuccess) {
        h->err = std::string(who) + ": copy failed: " + hipGetErrorString(e);
        return bail(PCG_ERR_HIP);
    }
    if ((rc = setup_multipliers(h, who)) != PCG_OK)
        return bail(rc);
    *out = h;
    return PCG_OK;
}

}   // namespace

extern "C" {

size_t pcg_handle_bytes(const pcg_grid *grid)
{
    if (!grid)
        return 0;
    Geometry g{};
    const std::string keep = g_create_error;
    if (check_grid("pcg_handle_bytes", grid, &g) != PCG_OK) {
        g_create_error = keep;
        return 0;
    }
    return table_layout(grid->nx, grid->ny, grid->nz, (grid->nz + g.L - 1) / g.L, nullptr, nullptr);
}

int pcg_create(const pcg_grid *grid, const pcg_coeffs *c, void *hip_stream, void *tables,
               size_t tables_bytes, pcg_handle **out)
{
    const char *who = "pcg_create";
    if (!out)
        return fail(nullptr, PCG_ERR_INVALID, "pcg_create: out is NULL");
    *out = nullptr;
    if (!grid || !c)
        return fail(nullptr, PCG_ERR_INVALID, "pcg_create: null grid or coefficients");
    Geometry g{};
    int rc = check_grid(who, grid, &g);
    if (rc != PCG_OK)
        return rc;
    const int nx = grid->nx, ny = grid->ny, nz = grid->nz;
    if (!(c->delta > 0.0) || !std::isfinite(c->delta))
        return fail(nullptr, PCG_ERR_INVALID, "pcg_create: delta must be finite and > 0");
    if ((rc = check_array(who, "alpha_z_face", c->alpha_z_face, (size_t)nz + 1, false)) != PCG_OK)
        return rc;
    if (c->alpha_z_face[0] != 0.0 || c->alpha_z_face[nz] != 0.0)
        return fail(nullptr, PCG_ERR_INVALID, "pcg_create: faces 0 and nz carry no flux and must be 0");
    const size_t ncol = (size_t)nx * ny;
    std::vector<double> ah(ncol);
    if (c->alpha_h_kind == PCG_AH_CONST) {
        if (!(c->alpha_h_const >= 0.0) || !std::isfinite(c->alpha_h_const))
            return fail(nullptr, PCG_ERR_INVALID, "pcg_create: alpha_h_const must be finite and >= 0");
        for (auto &v : ah) v = c->alpha_h_const;
    } else if (c->alpha_h_kind == PCG_AH_FIELD) {
        if ((rc = check_array(who, "alpha_h_field", c->alpha_h_field, ncol, false)) != PCG_OK)
            return rc;
        ah.assign(c->alpha_h_field, c->alpha_h_field + ncol);
    } else {
        return fail(nullptr, PCG_ERR_INVALID, "pcg_create: unknown alpha_h_kind %d", c->alpha_h_kind);
    }
    // the special case of the general form: |T| = 1, a = delta, d = 1,
    // beta = alpha_z, and the edge coefficient between two cells the mean of
    // their alpha_h (section 3, eqs. (6)-(7): one symmetric value per edge)
    HostCoeffs hc;
    hc.a.assign(nz, c->delta);
    hc.d.assign(nz, 1.0);
    hc.beta.assign(c->alpha_z_face, c->alpha_z_face + nz + 1);
    hc.area.assign(ncol, 1.0);
    hc.ex.resize(ncol);
    hc.ey.resize(ncol);
    for (int j = 0; j < ny; ++j)
        for (int i = 0; i < nx; ++i) {
            const size_t t = (size_t)j * nx + i;
            hc.ex[t] = 0.5 * (ah[t] + ah[(size_t)j * nx + (i + 1 == nx ? 0 : i + 1)]);
            hc.ey[t] = 0.5 * (ah[t] + ah[(size_t)(j + 1 == ny ? 0 : j + 1) * nx + i]);
        }
    return create_handle(who, grid, g, hc, hip_stream, tables, tables_bytes, out);
}

int pcg_create_general(const pcg_grid *grid, const pcg_coeffs_general *c, void *hip_stream,
                       void *tables, size_t tables_bytes, pcg_handle **out)
{
    const char *who = "pcg_create_general";
    if (!out)
        return fail(nullptr, PCG_ERR_INVALID, "%s: out is NULL", who);
    *out = nullptr;
    if (!grid || !c)
        return fail(nullptr, PCG_ERR_INVALID, "%s: null grid or coefficients", who);
    Geometry g{};
    int rc = check_grid(who, grid, &g);
    if (rc != PCG_OK)
        return rc;
    const int nx = grid->nx, ny = grid->ny, nz = grid->nz;
    const size_t ncol = (size_t)nx * ny;
    if ((rc = check_array(who, "a", c->a, (size_t)nz, true)) != PCG_OK ||
        (rc = check_array(who, "d", c->d, (size_t)nz, false)) != PCG_OK ||
        (rc = check_array(who, "beta_face", c->beta_face, (size_t)nz + 1, false)) != PCG_OK ||
        (rc = check_array(who, "area", c->area, ncol, true)) != PCG_OK ||
        (rc = check_array(who, "alpha_x", c->alpha_x, ncol, false)) != PCG_OK ||
        (rc = check_array(who, "alpha_y", c->alpha_y, ncol, false)) != PCG_OK)
        return rc;
    if (c->beta_face[0] != 0.0 || c->beta_face[nz] != 0.0)
        return fail(nullptr, PCG_ERR_INVALID, "%s: faces 0 and nz carry no flux and must be 0", who);
    HostCoeffs hc;
    hc.a.assign(c->a, c->a + nz);
    hc.d.assign(c->d, c->d + nz);
    hc.beta.assign(c->beta_face, c->beta_face + nz + 1);
    hc.area.assign(c->area, c->area + ncol);
    hc.ex.assign(c->alpha_x, c->alpha_x + ncol);
    hc.ey.assign(c->alpha_y, c->alpha_y + ncol);
    return create_handle(who, grid, g, hc, hip_stream, tables, tables_bytes, out);
}

int pcg_destroy(pcg_handle *h)
{
    if (!h)
        return PCG_OK;
    (void)hipSetDevice(h->device);
    if (h->stream || h->d_az)
        (void)hipStreamSynchronize(h->stream);
    for (auto &e : h->pending) {
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    for (auto e : h->free_events)
        (void)hipEventDestroy(e);
    if (h->loop_ev) (void)hipEventDestroy(h->loop_ev);
    if (h->h_status) (void)hipHostFree(h->h_status);
    for (auto *c : h->mg_levels)
        pcg_destroy(c);
    delete h;   // the device tables belong to the caller
    return PCG_OK;
}

int pcg_set_stream(pcg_handle *h, void *hip_stream)
{
    if (!h)
        return PCG_ERR_INVALID;
    h->stream = (hipStream_t)hip_stream;
    for (auto *c : h->mg_levels)
        c->stream = h->stream;
    return PCG_OK;
}

int pcg_apply_A(pcg_handle *h, const double *x, double *y)
{
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_vectors(h, x, y, "pcg_apply_A");
    if (rc != PCG_OK)
        return rc;
    if ((rc = set_device(h)) != PCG_OK)
        return rc;
    {
        Timed t(h, PCG_KID_APPLY_A, -1);
        stencil<double, double>(h, SP_APPLY, x, nullptr, nullptr, nullptr, y, nullptr, nullptr);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_apply_A_f32(pcg_handle *h, const float *x, float *y)
{
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_vectors(h, x, y, "pcg_apply_A_f32", sizeof(float));
    if (rc != PCG_OK)
        return rc;
    if ((rc = set_device(h)) != PCG_OK)
        return rc;
    {
        Timed t(h, PCG_KID_APPLY_A, -1);
        stencil<float, float>(h, SP_APPLY, x, nullptr, nullptr, nullptr, y, nullptr, nullptr);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_precond_f32(pcg_handle *h, const float *r, float *z)
{
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_vectors(h, r, z, "pcg_precond_f32", sizeof(float));
    if (rc != PCG_OK)
        return rc;
    if ((rc = set_device(h)) != PCG_OK)
        return rc;
    {
        Timed t(h, PCG_KID_PRECOND, -1);
        column<float, float>(h, r, nullptr, nullptr, z, nullptr, 0, nullptr, UPD_NONE, false);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_precond(pcg_handle *h, const double *r, double *z)
{
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_vectors(h, r, z, "pcg_precond");
    if (rc != PCG_OK)
        return rc;
    if ((rc = set_device(h)) != PCG_OK)
        return rc;
    {
        Timed t(h, PCG_KID_PRECOND, -1);
        column<double, double>(h, r, nullptr, nullptr, z, nullptr, 0, nullptr, UPD_NONE, false);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

size_t pcg_solve_workspace_bytes(const pcg_handle *h, int32_t maxit)
{
    if (!h || maxit < 0)
        return 0;
    return workspace_layout(h, maxit, nullptr, nullptr);
}

}   // extern "C"

namespace {

// ---- tensor-product multigrid -------------------------------------------------
// Level l of the hierarchy (0: the handle itself).
pcg_handle *mg_level(pcg_handle *h, int l) { return l == 0 ? h : h->mg_levels[(size_t)l - 1]; }

// Per level: the right-hand side f (levels >= 1; level 0 works on the
// solve's residual), the two iterate buffers U, V (the cycle's result lands
// in V; level 0's V is the solve's z) and W, which holds a residual (the
// restriction's t = f - A z, or w = f - A z of a two-pass sweep) that the
// next column pass reads while it writes an iterate buffer.
struct MgWork {
    std::vector<double *> f, U, V, W;
};

size_t mg_layout(const pcg_handle *h, int32_t maxit, char *base, Workspace *w, MgWork *mw)
{
    Workspace tmp{};
    Workspace *wl = w ? w : &tmp;
    size_t off = workspace_layout(h, maxit, base, wl);
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t nl = 1 + h->mg_levels.size();
    if (mw) {
        mw->f.assign(nl, nullptr);
        mw->U.assign(nl, nullptr);
        mw->V.assign(nl, nullptr);
        mw->W.assign(nl, nullptr);
    }
    const size_t o0 = take(h->n * sizeof(double)), ow0 = take(h->n * sizeof(double));
    if (mw && base) {
        mw->U[0] = (double *)(base + o0);
        mw->V[0] = wl->z;
        mw->W[0] = (double *)(base + ow0);
    }
    for (size_t l = 1; l < nl; ++l) {
        const size_t bytes = h->mg_levels[l - 1]->n * sizeof(double);
        const size_t of = take(bytes), ou = take(bytes), ov = take(bytes), ow = take(bytes);
        if (mw && base) {
            mw->f[l] = (double *)(base + of);
            mw->U[l] = (double *)(base + ou);
            mw->V[l] = (double *)(base + ov);
            mw->W[l] = (double *)(base + ow);
        }
    }
    return off;
}

// Multigrid forms of the column solve on a coarsest level of 16 or 32
// columns per workgroup (at most 8 levels per segment; never the fused r
// update, which only level 0 applies).
template <int MG, int L, int C>
void launch_mg_column_narrow(pcg_handle *h, const double *rin, const double *q, double *rout, double *z,
                             const SolveState *st, double *partials, const MgArgs &a)
{
    dim3 grid(h->col_tiles), block(h->col_threads);   // <= 16 C threads: P <= 16 (mg_coarse_columns)
    constexpr int UPD = kSweepForm<MG> ? UPD_AP : UPD_NONE;
    k_column_solve<L, C, UPD, true, false, double, double, MG><<<grid, block, 0, h->stream>>>(
        rin, q, rout, z, h->op, st, 0, kSweepForm<MG> ? nullptr : partials, nullptr, h->d_phib, a);
}

// Multigrid forms of the column solve (64-column tiles, or the narrow tiles
// of a coarsest level).  DOTS is instantiated on; the kernels skip the dot
// products when partials is null.
template <int MG, int L>
void launch_mg_column_l(pcg_handle *h, const double *rin, const double *q, double *rout, double *z,
                        const SolveState *st, int first, double *partials, int upd, const MgArgs &a)
{
    dim3 grid(h->col_tiles), block(h->col_threads);
    const Op &o = h->op;
    const bool fused_q = MG == MG_FIRST && upd == UPD_Q;
    if constexpr (L <= 8) {
        if (h->op.C == 16) {
            launch_mg_column_narrow<MG, L, 16>(h, rin, q, rout, z, st, partials, a);
            return;
        }
        if (h->op.C == 32) {
            launch_mg_column_narrow<MG, L, 32>(h, rin, q, rout, z, st, partials, a);
            return;
        }
    }
    if constexpr (kSweepForm<MG>) {
        if (h->col_full)
            k_column_full<L, UPD_AP, true, double, double, MG><<<grid, block, 0, h->stream>>>(
                rin, q, rout, z, o, st, 0, nullptr, h->d_phib, a);
        else
            k_column_solve<L, kWave, UPD_AP, true, false, double, double, MG><<<grid, block, 0, h->stream>>>(
                rin, q, rout, z, o, st, 0, nullptr, nullptr, h->d_phib, a);
    } else if (h->col_full) {
        if (fused_q)
            k_column_full<L, UPD_Q, true, double, double, MG_FIRST><<<grid, block, 0, h->stream>>>(
                rin, q, rout, z, o, st, first, partials, h->d_phib, a);
        else
            k_column_full<L, UPD_NONE, true, double, double, MG><<<grid, block, 0, h->stream>>>(
                rin, q, rout, z, o, st, first, partials, h->d_phib, a);
    } else {
        if (fused_q)
            k_column_solve<L, kWave, UPD_Q, true, false, double, double, MG_FIRST><<<grid, block, 0, h->stream>>>(
                rin, q, rout, z, o, st, first, partials, nullptr, h->d_phib, a);
        else
            k_column_solve<L, kWave, UPD_NONE, true, false, double, double, MG><<<grid, block, 0, h->stream>>>(
                rin, q, rout, z, o, st, first, partials, nullptr, h->d_phib, a);
    }
}

template <int MG>
void launch_mg_column(pcg_handle *h, const double *rin, const double *q, double *rout, double *z,
                      const SolveState *st, int first, double *partials, int upd, const MgArgs &a)
{
    if constexpr (MG == MG_FIRST) {
        // The first sweep holds no operands beyond r (and q): on a level whose
        // column passes take longer segments than its table (the finest), it
        // takes them too, as the PCG's own column pass does.
        if (h->colf_L == 16 && h->colf_L != h->op.L && h->colf_full) {
            const ColGeo g = col_geo(h, false);
            dim3 grid(h->col_tiles), block(g.threads);
            if (upd == UPD_Q)
                k_column_full<16, UPD_Q, true, double, double, MG_FIRST><<<grid, block, 0, h->stream>>>(
                    rin, q, rout, z, g.o, st, first, partials, h->d_phib, a);
            else
                k_column_full<16, UPD_NONE, true, double, double, MG_FIRST><<<grid, block, 0, h->stream>>>(
                    rin, q, rout, z, g.o, st, first, partials, h->d_phib, a);
            return;
        }
    }
    switch (h->op.L) {
    case 4: launch_mg_column_l<MG, 4>(h, rin, q, rout, z, st, first, partials, upd, a); break;
    case 8: launch_mg_column_l<MG, 8>(h, rin, q, rout, z, st, first, partials, upd, a); break;
    case 16: launch_mg_column_l<MG, 16>(h, rin, q, rout, z, st, first, partials, upd, a); break;
    default: launch_mg_column_l<MG, 32>(h, rin, q, rout, z, st, first, partials, upd, a); break;
    }
}

void mg_column(pcg_handle *h, int mode, const double *rin, const double *q, double *rout, double *z,
               const SolveState *st, int first, double *partials, int upd, const MgArgs &a)
{
    if (mode == MG_FIRST)
        launch_mg_column<MG_FIRST>(h, rin, q, rout, z, st, first, partials, upd, a);
    else if (mode == MG_CORR)
        launch_mg_column<MG_CORR>(h, rin, q, rout, z, st, first, partials, upd, a);
    else if (mode == MG_SWEEP)
        launch_mg_column<MG_SWEEP>(h, rin, q, rout, z, st, first, partials, upd, a);
    else if (mode == MG_CHEB)
        launch_mg_column<MG_CHEB>(h, rin, q, rout, z, st, first, partials, upd, a);
    else
        launch_mg_column<MG_POST>(h, rin, q, rout, z, st, first, partials, upd, a);
}

template <int Ls>
void launch_mg_restrict(pcg_handle *h, int fx, int fy, const double *f, const double *z, double *t,
                        double *fc, int ncx, const SolveState *st)
{
    const size_t ncy = (size_t)(h->op.ny / fy);
    dim3 grid((unsigned)((size_t)h->op.ntx * ncy * h->op.nkt)), block(kWave * h->op.Ws);
    if (fx == 2 && fy == 2)
        k_mg_restrict<Ls, 2, 2><<<grid, block, 0, h->stream>>>(f, z, t, fc, h->op, ncx, st);
    else if (fx == 2)
        k_mg_restrict<Ls, 2, 1><<<grid, block, 0, h->stream>>>(f, z, t, fc, h->op, ncx, st);
    else
        k_mg_restrict<Ls, 1, 2><<<grid, block, 0, h->stream>>>(f, z, t, fc, h->op, ncx, st);
}

// t = f - A z and fc = P^T t (level h to the next with factors fx, fy).
void mg_restrict(pcg_handle *h, int fx, int fy, const double *f, const double *z, double *t, double *fc,
                 int ncx, const SolveState *st)
{
    switch (h->op.Ls) {
    case 1: launch_mg_restrict<1>(h, fx, fy, f, z, t, fc, ncx, st); break;
    case 2: launch_mg_restrict<2>(h, fx, fy, f, z, t, fc, ncx, st); break;
    case 4: launch_mg_restrict<4>(h, fx, fy, f, z, t, fc, ncx, st); break;
    default: launch_mg_restrict<8>(h, fx, fy, f, z, t, fc, ncx, st); break;
    }
}

// z = B f on level l: one V(nu, nu) cycle (horizontal semi-coarsening,
// piecewise-constant transfers, Galerkin coarse operators, the column solve
// as damped block-Jacobi smoother).  rin is the level's right-hand side; on
// level 0 of a solve the first sweep also applies r -= alpha q (upd = UPD_Q,
// rout = rin = r) and the last sweep forms the partial sums <r, r>, <r, z>
// (partials).  The result lands in V; after the first sweep every sweep
// writes the buffer that does not hold the current iterate:
//   first sweep   z = omega M^{-1} f
//   sweep         z' = z + omega M^{-1} (f - A z), one column pass reading z's
//                 neighbours (the last sweep of level 0, which forms the dot
//                 products: a stencil pass for w = f - A z, then the column pass)
//   restriction   t = f - A z, f_c = P^T t
//   correction    z' = (z + P z_c) + omega M^{-1} (t - A P z_c), one column
//                 pass over the buffer of t
// On the coarsest level: the exact column solve for one column, else
// coarse_sweeps sweeps from z = 0; with a lower end coarse_lo > 0 those
// sweeps are the steps of the Chebyshev semi-iteration on [coarse_lo, 2]
// (first z_1 = M^{-1} f / theta, then the three-term update, each step's
// z_{k+1} written over z_{k-1}).
void mg_cycle(pcg_handle *h0, const MgWork &mw, int l, const double *rin, const double *q, double *rout,
              int upd, const SolveState *st, int first, double *partials)
{
    pcg_handle *h = mg_level(h0, l);
    const int nlev = 1 + (int)h0->mg_levels.size();
    const double *f = (upd != UPD_NONE) ? rout : rin;
    double *V = mw.V[(size_t)l], *U = mw.U[(size_t)l], *Wr = mw.W[(size_t)l];
    const MgArgs a{nullptr, f, h0->mg_omega, 0, 1, 1};
    auto sweep = [&](double *cur, double *oth, double *parts) {
        if (!parts && h->op.L <= 8) {   // one pass: the residual formed in the column kernel
                                         // (longer segments would spill its registers)
            mg_column(h, MG_SWEEP, f, cur, nullptr, oth, st, 0, nullptr, UPD_AP, a);
            return;
        }
        stencil<double, double>(h, SP_RESID, cur, f, nullptr, nullptr, Wr, nullptr, nullptr);
        mg_column(h, MG_CORR, Wr, cur, nullptr, oth, st, 0, parts, UPD_NONE, a);
    };
    if (l == nlev - 1) {
        if ((size_t)h->op.nx * h->op.ny == 1) {
            column<double, double>(h, rin, q, rout, V, st, first, partials, upd, partials != nullptr);
            return;
        }
        const int cs = h0->mg_coarse_sweeps;
        double *cur = ((cs - 1) % 2 == 0) ? V : U;
        double *oth = (cur == V) ? U : V;
        if (h0->mg_coarse_lo > 0.0) {
            const double lo = h0->mg_coarse_lo, hi = 2.0;
            const double theta = 0.5 * (hi + lo), delta = 0.5 * (hi - lo), s = theta / delta;
            MgArgs a1 = a;
            a1.omega = 1.0 / theta;
            mg_column(h, MG_FIRST, rin, q, rout, cur, st, first, cs == 1 ? partials : nullptr, upd, a1);
            double rho_prev = 1.0 / s;
            for (int k = 1; k < cs; ++k) {
                const double rho = 1.0 / (2.0 * s - rho_prev);
                MgArgs ak = a;
                ak.c1 = rho * rho_prev;
                ak.c2 = 2.0 * rho / delta;
                ak.cheb = k == 1 ? 1 : 2;
                double *parts = k == cs - 1 ? partials : nullptr;
                if (!parts && h->op.L <= 8) {
                    mg_column(h, MG_CHEB, f, cur, nullptr, oth, st, 0, nullptr, UPD_AP, ak);
                } else {
                    stencil<double, double>(h, SP_RESID, cur, f, nullptr, nullptr, Wr, nullptr, nullptr);
                    mg_column(h, MG_CORR, Wr, cur, nullptr, oth, st, 0, parts, UPD_NONE, ak);
                }
                std::swap(cur, oth);
                rho_prev = rho;
            }
            return;
        }
        mg_column(h, MG_FIRST, rin, q, rout, cur, st, first, cs == 1 ? partials : nullptr, upd, a);
        for (int sw = 1; sw < cs; ++sw) {
            sweep(cur, oth, sw == cs - 1 ? partials : nullptr);
            std::swap(cur, oth);
        }
        return;
    }
    const int nu = h0->mg_nu;
    double *cur = U, *oth = V;
    mg_column(h, MG_FIRST, rin, q, rout, cur, st, first, nullptr, upd, a);
    for (int sw = 1; sw < nu; ++sw) {
        sweep(cur, oth, nullptr);
        std::swap(cur, oth);
    }
    pcg_handle *c = mg_level(h0, l + 1);
    const int fx = h0->mg_fx[(size_t)l], fy = h0->mg_fy[(size_t)l];
    mg_restrict(h, fx, fy, f, cur, Wr, mw.f[(size_t)l + 1], c->op.nx, st);
    mg_cycle(h0, mw, l + 1, mw.f[(size_t)l + 1], nullptr, nullptr, UPD_NONE, st, 0, nullptr);
    const MgArgs ap{mw.V[(size_t)l + 1], f, h0->mg_omega, c->op.nx, fx, fy};
    mg_column(h, MG_POST, Wr, cur, nullptr, oth, st, 0, nu == 1 ? partials : nullptr, UPD_NONE, ap);
    std::swap(cur, oth);
    for (int sw = 1; sw < nu; ++sw) {
        sweep(cur, oth, sw == nu - 1 ? partials : nullptr);
        std::swap(cur, oth);
    }
}

// The interleaved loop of section 4.3, Algorithm 1.  ap = false: Algorithms 2
// and 3 as printed (q = A z + beta q stored by the stencil pass, r -= alpha q
// in the preconditioner pass), with the x updates of three steps deferred to
// the stencil pass of the fourth, which applies the four terms in the order of
// the steps (x is read and written every fourth step, the three older
// directions read then: 82 instead of 88 bytes per point per step); the
// directions rotate over four buffers so that the deferred ones are still
// there, and k_x_fixup applies what is pending when the loop stops.
// ap = true: q is never stored -- the preconditioner pass recomputes A p from
// p and the stencil pass forms <p_new, A z + beta A p_old>; p alternates
// between two buffers (the stencil pass reads the old direction around each
// point while writing the new one).
// TV, TZ: see the launch helpers; ap only for binary64.
// mg != nullptr: the preconditioner pass is one multigrid V-cycle (binary64).
template <typename TV, typename TZ>
int interleaved_loop(pcg_handle *h, const SolveArgs &a, const Workspace &w, bool ap, const char *who,
                     const MgWork *mg = nullptr)
{
    constexpr bool kD = kBinary64<TV, TZ>;
    if (ap && !kD)
        return fail(h, PCG_ERR_UNSUPPORTED, "%s: the q-free loop is binary64 only", who);
    HostStatus *hs = nullptr;
    HIP_TRY(h, hipHostGetDevicePointer((void **)&hs, h->h_status, 0));
    h->h_status->done = 0;
    const TV *b = (const TV *)a.b;
    TV *x = (TV *)a.x;
    const int32_t maxit = a.maxit;
    const double tol = a.tol;
    // the workspace's vector slots hold binary64 vectors; narrower types use
    // the front of each slot
    TV *r = (TV *)w.r, *q = (TV *)w.q;
    TZ *z = (TZ *)w.z;
    // p_i lives in pbuf[i mod 4]: four buffers with q stored (x is updated
    // every fourth step), two on the q-free path (the stencil pass reads the
    // old direction around each point while it writes the new one), each
    // named twice
    TV *pbuf[4] = {(TV *)w.p, ap ? (TV *)w.q : (TV *)w.p2, ap ? (TV *)w.p : (TV *)w.p3,
                   ap ? (TV *)w.q : (TV *)w.p4};
    k_init_state<<<1, 64, 0, h->stream>>>(w.state);
    // a2: r0 = b - A x0
    stencil<TV, TV>(h, SP_RESID, x, b, nullptr, nullptr, r, nullptr, nullptr);
    hipEvent_t ev = h->loop_ev;
    int last = 0;
    for (int k = 0; k <= maxit; ++k) {
        int nred = 0;
        const double *red = nullptr;
        // search direction read this iteration (written by the previous one)
        // and the buffer of the new one
        TV *pin = ap ? pbuf[(k + 1) & 1] : q;
        TV *pcur = pbuf[(k + 3) & 3];    // p_{k-1}
        TV *pnext = pbuf[k & 3];         // p_{k-4} (q-free: p_{k-2}) on entry, p_k on exit
        const Older<TV> older{pbuf[(k + 1) & 3], pbuf[(k + 2) & 3]};   // p_{k-3}, p_{k-2}
        // the stencil pass's form and whether it brings x up to date
        const bool xstep = ap ? k > 0 : (k > 0 && k % 4 == 0);
        const int smode = ap ? (k == 0 ? SP_FIRST_AP : SP_FUSED_AP)
                             : (k == 0 ? SP_FIRST : (xstep ? SP_FUSED_X4 : SP_FUSED_NOX));
        // a3: r -= alpha q (or alpha A p); z = M^{-1} r; partial <r,r>, <r,z>  (Algorithm 3)
        if constexpr (kD) {
            if (mg) {
                Timed t(h, PCG_KID_MG_VCYCLE, k);
                mg_cycle(h, *mg, 0, nullptr, pin, r, UPD_Q, w.state, k == 0, w.partials);
            }
        }
        if (!mg) {
            Timed t(h, PCG_KID_FUSED_PREC, k);
            column<TV, TZ>(h, nullptr, pin, r, z, w.state, k == 0, w.partials, ap ? UPD_AP : UPD_Q, true);
        }
        // a4: ||r_k||, stop test, beta
        red = fold_partials(h, w, h->col_tiles, &nred);
        k_reduce_rz<<<1, kRedThreads, 0, h->stream>>>(red, nred, w.state, w.hist, k, maxit, tol, hs);
        if (k == 0)
            (void)hipEventRecord(ev, h->stream);
        // a5: x += alpha p; p = z + beta p; q = A z + beta q (or A p_new on the
        //     fly); partial <p,q>  (Algorithm 2); only x += alpha p once the
        //     stop test has passed (a7)
        {
            Timed t(h, PCG_KID_FUSED_SPMV, k);
            if (ap) {
                if constexpr (kD)
                    stencil<TV, TZ>(h, smode, z, nullptr, x, pcur, nullptr, w.state, w.partials, pnext);
            } else if (k == 0) {
                stencil<TV, TZ>(h, SP_FIRST, z, nullptr, x, pnext, q, w.state, w.partials);
            } else {
                stencil<TV, TZ>(h, smode, z, nullptr, x, pcur, q, w.state, w.partials, pnext, older);
            }
        }
        // a6: sigma, alpha
        red = fold_partials(h, w, stencil_tiles(h, smode, kBinary64<TV, TZ>, std::is_same<TV, float>::value), &nred);
        k_reduce_sigma<<<1, kRedThreads, 0, h->stream>>>(red, nred, w.state, k, xstep ? k : -1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(h, PCG_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
        if (k == 0) {
            e = hipEventSynchronize(ev);
            if (e != hipSuccess)
                return fail(h, PCG_ERR_HIP, "%s: hipEventSynchronize: %s", who, hipGetErrorString(e));
        } else {
            const int rc = wait_published(h, k, who);
            if (rc != PCG_OK)
                return rc;
        }
        last = k;
        if (((volatile HostStatus *)h->h_status)->done)
            break;
    }
    // a7: the x updates still pending when the loop stopped
    const DirRing<TV> ring{{pbuf[0], pbuf[1], pbuf[2], pbuf[3]}};
    const size_t nb = std::min<size_t>((h->n + 255) / 256, 8192);
    k_x_fixup<TV><<<dim3((unsigned)std::max<size_t>(nb, 1)), dim3(256), 0, h->stream>>>(x, ring, w.state, h->n);
    return solve_epilogue(h, a, w, PCG_KID_FUSED_SPMV, last);
}

}   // namespace

extern "C" {

int pcg_solve(pcg_handle *h, const double *b, double *x, double tol, int32_t maxit, void *ws,
              size_t ws_bytes, int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
              double *final_rel)
{
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, "pcg_solve");
    if (rc != PCG_OK)
        return rc;
    return interleaved_loop<double, double>(h, a, w, false, "pcg_solve");
}

int pcg_solve_no_q(pcg_handle *h, const double *b, double *x, double tol, int32_t maxit, void *ws,
                   size_t ws_bytes, int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
                   double *final_rel)
{
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, "pcg_solve_no_q");
    if (rc != PCG_OK)
        return rc;
    return interleaved_loop<double, double>(h, a, w, true, "pcg_solve_no_q");
}

int pcg_solve_f32(pcg_handle *h, const float *b, float *x, double tol, int32_t maxit, void *ws,
                  size_t ws_bytes, int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
                  double *final_rel)
{
    SolveArgs a{b, x, sizeof(float), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, "pcg_solve_f32");
    if (rc != PCG_OK)
        return rc;
    return interleaved_loop<float, float>(h, a, w, false, "pcg_solve_f32");
}

int pcg_solve_mixed(pcg_handle *h, const double *b, double *x, double tol, int32_t maxit, void *ws,
                    size_t ws_bytes, int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
                    double *final_rel)
{
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, "pcg_solve_mixed");
    if (rc != PCG_OK)
        return rc;
    return interleaved_loop<double, float>(h, a, w, false, "pcg_solve_mixed");
}

size_t pcg_solve_static_max_bytes(void) { return kScratchBytes; }

int pcg_solve_static(pcg_handle *h, const double *b, double *x, double tol, int32_t maxit,
                     int32_t *iters_out, double *hist_host, int32_t *hist_len_out, double *final_rel)
{
    const char *who = "pcg_solve_static";
    if (!h)
        return PCG_ERR_INVALID;
    if (maxit < 0)
        return fail(h, PCG_ERR_INVALID, "%s: maxit must be >= 0", who);
    void *ws = scratch_of(h->device);
    if (!ws)
        return fail(h, PCG_ERR_HIP, "%s: the scratch array has no address on device %d", who, h->device);
    const size_t need = workspace_layout(h, maxit, nullptr, nullptr);
    if (need > kScratchBytes)
        return fail(h, PCG_ERR_INVALID,
                    "%s: grid %d x %d x %d with maxit %d needs %zu bytes of workspace; the fixed scratch "
                    "array holds %zu (use pcg_solve with a workspace)",
                    who, h->op.nx, h->op.ny, h->op.nz, maxit, need, kScratchBytes);
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, kScratchBytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, who);
    if (rc != PCG_OK)
        return rc;
    // per-kernel timing would create events on first use: not recorded here
    const bool profiling = h->profiling;
    h->profiling = false;
    rc = interleaved_loop<double, double>(h, a, w, false, who);
    h->profiling = profiling;
    return rc;
}

}   // extern "C"

namespace {

// One coarse level from the fine level h (factors fx, fy): its tables in
// `tables` (table_layout bytes), the coefficients by Galerkin coarsening, the
// Thomas multipliers.
int create_coarse(pcg_handle *h, int fx, int fy, int C, char *tables, pcg_handle **out)
{
    const char *who = "pcg_mg_setup";
    pcg_handle *c = new pcg_handle();
    c->device = h->device;
    c->stream = h->stream;
    const Geometry g{h->op.L, C, h->op.Ls, h->op.Ws, h->op.L, 0};
    const int nz = h->op.nz;
    init_geometry(c, h->op.nx / fx, h->op.ny / fy, nz, g);
    table_layout(c->op.nx, c->op.ny, nz, c->op.P, tables, c);
    int rc = PCG_OK;
    hipError_t e;
    if ((e = hipMemcpyAsync(c->d_az, h->d_az, sizeof(double) * (nz + 1), hipMemcpyDeviceToDevice,
                            h->stream)) != hipSuccess ||
        (e = hipMemcpyAsync(c->d_coef, h->d_coef, sizeof(double) * 2 * (size_t)nz,
                            hipMemcpyDeviceToDevice, h->stream)) != hipSuccess) {
        c->err = std::string(who) + ": copy failed: " + hipGetErrorString(e);
        rc = PCG_ERR_HIP;
    } else {
        const size_t ncol = (size_t)c->op.nx * c->op.ny;
        double *area = c->d_coef + 2 * (size_t)nz;
        k_mg_coarsen<<<dim3((unsigned)((ncol + 255) / 256)), dim3(256), 0, h->stream>>>(
            h->op, c->op.nx, c->op.ny, fx, fy, area, area + ncol, area + 2 * ncol);
        rc = setup_multipliers(c, who);
    }
    if (rc != PCG_OK) {
        h->err = c->err;
        pcg_destroy(c);
        return rc;
    }
    *out = c;
    return PCG_OK;
}

// Columns per workgroup of the coarsest level's column passes.  Its
// coarse_sweeps sweeps run back to back on a small grid: with 64-column tiles
// the 64 x 64 coarsest level of a 1024 x 1024 grid is 64 workgroups, a
// quarter of the chip, and each sweep's time is set by the per-CU work of
// the CUs in use.  Halve the tile width (down to 16) while the level has
// fewer tiles than the chip has CUs.  Segments of at most 8 levels, at most
// 16 per column (the narrow forms are instantiated and bounded for those);
// a single column keeps 64 (its exact solve is one tile either way).
// MFPCG_MG_COARSE_C (16, 32 or 64) overrides the choice.
int mg_coarse_columns(pcg_handle *h, int nx, int ny, int *C)
{
    *C = kWave;
    if (h->op.L > 8 || h->op.P > 16 || (size_t)nx * ny == 1)
        return PCG_OK;
    const int v = env_int("MFPCG_MG_COARSE_C", 0, &h->overrides, PCG_TUNE_MG_COARSE_C);
    if (v != 0) {
        if (v != 16 && v != 32 && v != 64)
            return fail(h, PCG_ERR_INVALID, "pcg_mg_setup: MFPCG_MG_COARSE_C must be 16, 32 or 64");
        *C = v;
        return PCG_OK;
    }
    while (*C > 16 && (size_t)((nx + *C - 1) / *C) * ny < (size_t)kCus)
        *C /= 2;
    return PCG_OK;
}

// The coarsening factors of the hierarchy pcg_mg_setup builds for these
// parameters (one (fx, fy) pair per coarse level) and the bytes of the
// coarse levels' tables.
size_t mg_plan(const pcg_handle *h, int max_levels, std::vector<int> *fxs, std::vector<int> *fys)
{
    int nx = h->op.nx, ny = h->op.ny, nlev = 1;
    size_t bytes = 0;
    while ((max_levels == 0 || nlev < max_levels) && (size_t)nx * ny > 1) {
        const int fx = (nx > 1 && nx % 2 == 0) ? 2 : 1;
        const int fy = (ny > 1 && ny % 2 == 0) ? 2 : 1;
        if (fx == 1 && fy == 1)
            break;
        nx /= fx;
        ny /= fy;
        ++nlev;
        bytes += table_layout(nx, ny, h->op.nz, h->op.P, nullptr, nullptr);
        if (fxs) fxs->push_back(fx);
        if (fys) fys->push_back(fy);
    }
    return bytes;
}

void mg_clear(pcg_handle *h)
{
    for (auto *c : h->mg_levels)
        pcg_destroy(c);
    h->mg_levels.clear();
    h->mg_fx.clear();
    h->mg_fy.clear();
    h->mg_nu = 0;
}

}   // namespace

extern "C" {

size_t pcg_mg_setup_bytes(const pcg_handle *h, const pcg_mg_params *p)
{
    if (!h || !p || p->max_levels < 0 || p->max_levels > 64)
        return 0;
    return mg_plan(h, p->max_levels, nullptr, nullptr);
}

int pcg_mg_setup(pcg_handle *h, const pcg_mg_params *p, void *levels, size_t levels_bytes)
{
    const char *who = "pcg_mg_setup";
    if (!h)
        return PCG_ERR_INVALID;
    if (!p)
        return fail(h, PCG_ERR_INVALID, "%s: params is NULL", who);
    if (p->nu < 1 || p->nu > 16)
        return fail(h, PCG_ERR_INVALID, "%s: nu = %d must be in 1..16", who, p->nu);
    if (!(p->omega > 0.0 && p->omega <= 1.0))
        return fail(h, PCG_ERR_INVALID, "%s: omega = %g must be in (0, 1]", who, p->omega);
    if (p->max_levels < 0 || p->max_levels > 64)
        return fail(h, PCG_ERR_INVALID, "%s: max_levels = %d must be in 0..64", who, p->max_levels);
    if (p->coarse_sweeps < 1 || p->coarse_sweeps > 1024)
        return fail(h, PCG_ERR_INVALID, "%s: coarse_sweeps = %d must be in 1..1024", who, p->coarse_sweeps);
    if (!(p->coarse_lo >= 0.0 && p->coarse_lo < 2.0))
        return fail(h, PCG_ERR_INVALID, "%s: coarse_lo = %g must be in [0, 2)", who, p->coarse_lo);
    if (h->op.C != kWave)
        return fail(h, PCG_ERR_UNSUPPORTED, "%s: the multigrid sweeps need 64-column column tiles", who);
    std::vector<int> fxs, fys;
    const size_t need = mg_plan(h, p->max_levels, &fxs, &fys);
    int rc = PCG_OK;
    if (need > 0 && (rc = check_buffer(h, who, "levels_dev", levels, levels_bytes, need)) != PCG_OK)
        return rc;
    if ((rc = set_device(h)) != PCG_OK)
        return rc;
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    mg_clear(h);
    pcg_handle *cur = h;
    char *base = (char *)levels;
    for (size_t l = 0; l < fxs.size(); ++l) {
        pcg_handle *c = nullptr;
        int C = kWave;
        if (l + 1 == fxs.size() &&
            (rc = mg_coarse_columns(h, cur->op.nx / fxs[l], cur->op.ny / fys[l], &C)) != PCG_OK) {
            mg_clear(h);
            return rc;
        }
        if ((rc = create_coarse(cur, fxs[l], fys[l], C, base, &c)) != PCG_OK) {
            if (cur != h)
                h->err = cur->err;
            mg_clear(h);
            return rc;
        }
        base += table_layout(c->op.nx, c->op.ny, c->op.nz, c->op.P, nullptr, nullptr);
        h->mg_levels.push_back(c);
        h->mg_fx.push_back(fxs[l]);
        h->mg_fy.push_back(fys[l]);
        cur = c;
    }
    h->mg_nu = p->nu;
    h->mg_omega = p->omega;
    h->mg_coarse_sweeps = p->coarse_sweeps;
    h->mg_coarse_lo = p->coarse_lo;
    return PCG_OK;
}

int pcg_mg_num_levels(const pcg_handle *hc, int32_t *levels)
{
    pcg_handle *h = const_cast<pcg_handle *>(hc);
    if (!h || !levels)
        return PCG_ERR_INVALID;
    if (h->mg_nu == 0)
        return fail(h, PCG_ERR_INVALID, "pcg_mg_num_levels: call pcg_mg_setup first");
    *levels = 1 + (int32_t)h->mg_levels.size();
    return PCG_OK;
}

int pcg_mg_level(pcg_handle *h, int32_t level, int32_t *nx, int32_t *ny, double *area, double *ax, double *ay)
{
    if (!h)
        return PCG_ERR_INVALID;
    if (h->mg_nu == 0)
        return fail(h, PCG_ERR_INVALID, "pcg_mg_level: call pcg_mg_setup first");
    if (level < 0 || level > (int32_t)h->mg_levels.size())
        return fail(h, PCG_ERR_INVALID, "pcg_mg_level: level %d out of range", level);
    pcg_handle *l = mg_level(h, level);
    if (nx)
        *nx = l->op.nx;
    if (ny)
        *ny = l->op.ny;
    const size_t ncol = (size_t)l->op.nx * l->op.ny;
    int rc = set_device(h);
    if (rc != PCG_OK)
        return rc;
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    if (area)
        HIP_TRY(h, hipMemcpy(area, l->op.area, ncol * sizeof(double), hipMemcpyDeviceToHost));
    if (ax)
        HIP_TRY(h, hipMemcpy(ax, l->op.ex, ncol * sizeof(double), hipMemcpyDeviceToHost));
    if (ay)
        HIP_TRY(h, hipMemcpy(ay, l->op.ey, ncol * sizeof(double), hipMemcpyDeviceToHost));
    return PCG_OK;
}

size_t pcg_mg_workspace_bytes(const pcg_handle *h, int32_t maxit)
{
    if (!h || maxit < 0 || h->mg_nu == 0)
        return 0;
    return mg_layout(h, maxit, nullptr, nullptr, nullptr);
}

int pcg_mg_vcycle(pcg_handle *h, const double *r, double *z, void *ws, size_t ws_bytes)
{
    const char *who = "pcg_mg_vcycle";
    if (!h)
        return PCG_ERR_INVALID;
    if (h->mg_nu == 0)
        return fail(h, PCG_ERR_INVALID, "%s: call pcg_mg_setup first", who);
    SolveArgs a{r, z, sizeof(double), 0.0, 0, ws, ws_bytes, nullptr, nullptr, nullptr, nullptr};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, who, true);
    if (rc != PCG_OK)
        return rc;
    MgWork mw;
    mg_layout(h, 0, (char *)ws, &w, &mw);
    mw.V[0] = z;
    {
        Timed t(h, PCG_KID_MG_VCYCLE, -1);
        mg_cycle(h, mw, 0, r, nullptr, nullptr, UPD_NONE, nullptr, 0, nullptr);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_solve_mg(pcg_handle *h, const double *b, double *x, double tol, int32_t maxit, void *ws,
                 size_t ws_bytes, int32_t *iters_out, double *hist_host, int32_t *hist_len_out,
                 double *final_rel)
{
    const char *who = "pcg_solve_mg";
    if (!h)
        return PCG_ERR_INVALID;
    if (h->mg_nu == 0)
        return fail(h, PCG_ERR_INVALID, "%s: call pcg_mg_setup first", who);
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, who, true);
    if (rc != PCG_OK)
        return rc;
    MgWork mw;
    mg_layout(h, maxit, (char *)ws, &w, &mw);
    return interleaved_loop<double, double>(h, a, w, false, who, &mw);
}

}   // extern "C"

namespace {

// The explicit operator of section 6.2 (CSR matrix + stored column matrices),
// or none for the matrix-free operator.
struct Explicit {
    const int64_t *row_ptr;
    const int32_t *col;
    const double *val;
    const double *tri;
};

// Standard PCG (section 4.1): q = A p with sigma; x, r updates with <r,r>;
// z = M^{-1} r with <r,z>; p = z + beta p.  The host reads the stop decision
// after the r update while the preconditioner pass already runs.
int standard_loop(pcg_handle *h, const SolveArgs &a, const Workspace &w, const Explicit *ex,
                  const char *who)
{
    HostStatus *hs = nullptr;
    HIP_TRY(h, hipHostGetDevicePointer((void **)&hs, h->h_status, 0));
    h->h_status->done = 0;
    hipEvent_t ev = h->loop_ev;
    const double *b = (const double *)a.b;
    double *x = (double *)a.x;
    const int32_t maxit = a.maxit;
    const double tol = a.tol;
    const double *tri = ex ? ex->tri : nullptr;
    int nred = 0;
    const double *red = nullptr;
    k_init_state<<<1, 64, 0, h->stream>>>(w.state);
    if (ex)
        csr_spmv(h, CSR_RESID, ex->row_ptr, ex->col, ex->val, x, b, w.r, nullptr, nullptr);
    else
        stencil<double, double>(h, SP_RESID, x, b, nullptr, nullptr, w.r, nullptr, nullptr);
    {
        Timed t(h, PCG_KID_PRECOND, 0);
        column<double, double>(h, w.r, nullptr, nullptr, w.z, w.state, 1, w.partials, UPD_NONE, true, tri);
    }
    red = fold_partials(h, w, h->col_tiles, &nred);
    k_reduce_rz<<<1, kRedThreads, 0, h->stream>>>(red, nred, w.state, w.hist, 0, maxit, tol, hs);
    {
        Timed t(h, PCG_KID_VECTOR, 0);
        update_p(h, w.p, w.z, w.state, 1);
    }
    (void)hipEventRecord(ev, h->stream);
    hipError_t e = hipEventSynchronize(ev);
    bool done = (e == hipSuccess) && ((volatile HostStatus *)h->h_status)->done;
    for (int k = 1; e == hipSuccess && !done && k <= maxit; ++k) {
        {   // q = A p ; sigma = <p,q>
            Timed t(h, PCG_KID_APPLY_A, k);
            if (ex)
                csr_spmv(h, CSR_APPLY_DOT, ex->row_ptr, ex->col, ex->val, w.p, nullptr, w.q, w.state, w.partials);
            else
                stencil<double, double>(h, SP_APPLY_DOT, w.p, nullptr, nullptr, nullptr, w.q, w.state, w.partials);
        }
        red = fold_partials(h, w, ex ? h->pt_tiles : stencil_tiles(h, SP_APPLY_DOT, true, false), &nred);
        k_reduce_sigma<<<1, kRedThreads, 0, h->stream>>>(red, nred, w.state, k - 1, -1);
        {   // x += alpha p ; r -= alpha q ; <r,r>
            Timed t(h, PCG_KID_VECTOR, k);
            update_xr(h, x, w.p, w.r, w.q, w.state, w.partials);
        }
        red = fold_partials(h, w, h->pt_tiles, &nred);
        k_reduce_rr<<<1, kRedThreads, 0, h->stream>>>(red, nred, w.state, w.hist, k, maxit, tol, hs);
        {   // z = M^{-1} r ; kappa = <r,z>
            Timed t(h, PCG_KID_PRECOND, k);
            column<double, double>(h, w.r, nullptr, nullptr, w.z, w.state, 1, w.partials, UPD_NONE, true, tri);
        }
        red = fold_partials(h, w, h->col_tiles, &nred);
        k_reduce_kappa<<<1, kRedThreads, 0, h->stream>>>(red, nred, w.state);
        {   // p = z + beta p
            Timed t(h, PCG_KID_VECTOR, k);
            update_p(h, w.p, w.z, w.state, 0);
        }
        e = hipGetLastError();
        if (e != hipSuccess)
            break;
        const int rc = wait_published(h, k, who);
        if (rc != PCG_OK)
            return rc;
        done = ((volatile HostStatus *)h->h_status)->done;
    }
    if (e != hipSuccess)
        return fail(h, PCG_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
    return solve_epilogue(h, a, w, -1, -2);
}

int csr_supported(pcg_handle *h, const char *who)
{
    if (h->n >= (size_t)0x7fffffff)
        return fail(h, PCG_ERR_UNSUPPORTED, "%s: N = %zu >= 2^31 does not fit int32 column indices", who, h->n);
    return PCG_OK;
}

int check_explicit(pcg_handle *h, const Explicit &ex, const char *who)
{
    if (!ex.row_ptr || !ex.col || !ex.val || !ex.tri)
        return fail(h, PCG_ERR_INVALID, "%s: null CSR or tridiagonal pointer", who);
    return csr_supported(h, who);
}

}   // namespace

extern "C" {

int pcg_solve_standard(pcg_handle *h, const double *b, double *x, double tol, int32_t maxit,
                       void *ws, size_t ws_bytes, int32_t *iters_out, double *hist_host,
                       int32_t *hist_len_out, double *final_rel)
{
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    Workspace w{};
    int rc = solve_prologue(h, a, &w, "pcg_solve_standard");
    if (rc != PCG_OK)
        return rc;
    return standard_loop(h, a, w, nullptr, "pcg_solve_standard");
}

int pcg_csr_nnz(const pcg_handle *hc, int64_t *nnz)
{
    pcg_handle *h = const_cast<pcg_handle *>(hc);
    if (!h || !nnz)
        return PCG_ERR_INVALID;
    int rc = csr_supported(h, "pcg_csr_nnz");
    if (rc != PCG_OK)
        return rc;
    *nnz = csr_nnz(h);
    return PCG_OK;
}

int pcg_csr_assemble(pcg_handle *h, int64_t *row_ptr, int32_t *col, double *val)
{
    if (!h)
        return PCG_ERR_INVALID;
    if (!row_ptr || !col || !val)
        return fail(h, PCG_ERR_INVALID, "pcg_csr_assemble: null pointer");
    int rc = csr_supported(h, "pcg_csr_assemble");
    if (rc != PCG_OK || (rc = set_device(h)) != PCG_OK)
        return rc;
    csr_assemble(h, row_ptr, col, val);
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_csr_spmv(pcg_handle *h, const int64_t *row_ptr, const int32_t *col, const double *val,
                 const double *x, double *y)
{
    if (!h)
        return PCG_ERR_INVALID;
    if (!row_ptr || !col || !val)
        return fail(h, PCG_ERR_INVALID, "pcg_csr_spmv: null CSR pointer");
    int rc = check_vectors(h, x, y, "pcg_csr_spmv");
    if (rc != PCG_OK || (rc = csr_supported(h, "pcg_csr_spmv")) != PCG_OK || (rc = set_device(h)) != PCG_OK)
        return rc;
    {
        Timed t(h, PCG_KID_CSR_SPMV, -1);
        csr_spmv(h, CSR_APPLY, row_ptr, col, val, x, nullptr, y, nullptr, nullptr);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

size_t pcg_tridiag_bytes(const pcg_handle *h)
{
    if (!h)
        return 0;
    const size_t ncol = (size_t)h->op.nx * h->op.ny;
    return sizeof(double) * (3 * h->n + ncol * (size_t)(h->op.P > 1 ? h->op.P - 1 : 1));
}

int pcg_tridiag_factor(pcg_handle *h, double *tri, size_t tri_bytes)
{
    const char *who = "pcg_tridiag_factor";
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_buffer(h, who, "tri_dev", tri, tri_bytes, pcg_tridiag_bytes(h));
    if (rc != PCG_OK || (rc = set_device(h)) != PCG_OK)
        return rc;
    const size_t ncol = (size_t)h->op.nx * h->op.ny;
    if (h->op.P > 1) {
        const int threads = 256;
        k_setup_phib_stored<<<dim3((unsigned)((ncol + threads - 1) / threads)), dim3(threads), 0, h->stream>>>(
            h->op, tri, tri + 3 * h->n);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_tridiag_assemble(pcg_handle *h, double *tri, size_t tri_bytes)
{
    const char *who = "pcg_tridiag_assemble";
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_buffer(h, who, "tri_dev", tri, tri_bytes, pcg_tridiag_bytes(h));
    if (rc != PCG_OK || (rc = set_device(h)) != PCG_OK)
        return rc;
    const size_t ncol = (size_t)h->op.nx * h->op.ny;
    const int threads = 256;
    k_tridiag_assemble<<<dim3((unsigned)((ncol + threads - 1) / threads)), dim3(threads), 0, h->stream>>>(h->op, tri);
    HIP_TRY(h, hipGetLastError());
    return pcg_tridiag_factor(h, tri, tri_bytes);
}

int pcg_tridiag_precond(pcg_handle *h, const double *tri, size_t tri_bytes, const double *r, double *z)
{
    const char *who = "pcg_tridiag_precond";
    if (!h)
        return PCG_ERR_INVALID;
    int rc = check_vectors(h, r, z, who);
    if (rc != PCG_OK || (rc = check_buffer(h, who, "tri_dev", tri, tri_bytes, pcg_tridiag_bytes(h))) != PCG_OK ||
        (rc = set_device(h)) != PCG_OK)
        return rc;
    {
        Timed t(h, PCG_KID_PRECOND, -1);
        column<double, double>(h, r, nullptr, nullptr, z, nullptr, 0, nullptr, UPD_NONE, false, tri);
    }
    HIP_TRY(h, hipGetLastError());
    return PCG_OK;
}

int pcg_solve_csr(pcg_handle *h, const int64_t *row_ptr, const int32_t *col, const double *val,
                  const double *tri, size_t tri_bytes, const double *b, double *x, double tol,
                  int32_t maxit, void *ws, size_t ws_bytes, int32_t *iters_out, double *hist_host,
                  int32_t *hist_len_out, double *final_rel)
{
    SolveArgs a{b, x, sizeof(double), tol, maxit, ws, ws_bytes, iters_out, hist_host, hist_len_out, final_rel};
    if (!h)
        return PCG_ERR_INVALID;
    Explicit ex{row_ptr, col, val, tri};
    int rc = check_explicit(h, ex, "pcg_solve_csr");
    if (rc != PCG_OK ||
        (rc = check_buffer(h, "pcg_solve_csr", "tri_dev", tri, tri_bytes, pcg_tridiag_bytes(h))) != PCG_OK)
        return rc;
    Workspace w{};
    rc = solve_prologue(h, a, &w, "pcg_solve_csr");
    if (rc != PCG_OK)
        return rc;
    return standard_loop(h, a, w, &ex, "pcg_solve_csr");
}

int pcg_profile_enable(pcg_handle *h, int32_t enable)
{
    if (!h)
        return PCG_ERR_INVALID;
    if (enable < 0)
        return fail(h, PCG_ERR_INVALID, "pcg_profile_enable: enable = %d must be >= 0", enable);
    h->profiling = enable != 0;
    h->profile_period = enable > 1 ? enable : 1;
    return PCG_OK;
}

int pcg_profile_reset(pcg_handle *h)
{
    if (!h)
        return PCG_ERR_INVALID;
    if (!h->pending.empty()) {
        HIP_TRY(h, hipStreamSynchronize(h->stream));
        drain_events(h);
    }
    for (int t = 0; t < PCG_KID_COUNT; ++t) {
        h->prof_ms[t] = 0.0;
        h->prof_n[t] = 0;
    }
    return PCG_OK;
}

int pcg_profile_read(const pcg_handle *hc, int32_t kid, double *ms_total, int64_t *launches)
{
    pcg_handle *h = const_cast<pcg_handle *>(hc);
    if (!h || kid < 0 || kid >= PCG_KID_COUNT)
        return PCG_ERR_INVALID;
    if (!h->pending.empty()) {
        HIP_TRY(h, hipStreamSynchronize(h->stream));
        drain_events(h);
    }
    if (ms_total)
        *ms_total = h->prof_ms[kid];
    if (launches)
        *launches = h->prof_n[kid];
    return PCG_OK;
}

}   // extern "C"
