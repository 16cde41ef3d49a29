// stream_probe.hip - a measurement tool, not part of the solver: the HBM
// bandwidth that a plain streaming kernel reaches on this GPU when it reads
// R and writes W vectors once per element, the stream mixes of the solver's
// passes (column pass: 2 in / 2 out; stencil pass: 3 / 2 on the steps that
// defer the x update, 7 / 3 on every fourth step), in float64 (8 bytes per lane access) and float32 (4 bytes,
// the binary32 solve's element).  It gives the measured ceiling beside the
// published peak for those mixes.  C ABI, loaded by bench.py --stream-probe.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxBlock = 1024;

template <typename T>
struct Streams {
    const T *in[7];
    T *out[3];
};

template <bool NT, typename T>
__device__ __forceinline__ T ld(const T *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void st(T *p, T v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Each thread handles E elements blockDim.x apart, all loads issued before
// any store.  Workgroup b owns elements [b * B * E, (b + 1) * B * E) with
// B = blockDim.x; the grid covers n exactly (the host checks n % (B * E) == 0).
template <typename T, int R, int W, bool NT, int E>
__global__ __launch_bounds__(kMaxBlock) void k_stream(Streams<T> s)
{
    const size_t B = blockDim.x;
    const size_t b0 = (size_t)blockIdx.x * B * E + threadIdx.x;
    T v[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[r][e] = ld<NT>(s.in[r] + b0 + B * e);
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            T acc = 0;
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc += (T)(r + w + 1) * v[r][e];
            st<NT>(s.out[w] + b0 + B * e, acc);
        }
}

template <typename T, int R, int W, int E>
void launch_e(bool nt, const Streams<T> &s, unsigned grid, unsigned block, hipStream_t st)
{
    if (nt)
        k_stream<T, R, W, true, E><<<grid, block, 0, st>>>(s);
    else
        k_stream<T, R, W, false, E><<<grid, block, 0, st>>>(s);
}

template <typename T, int R, int W>
void launch(bool nt, int elems, const Streams<T> &s, unsigned grid, unsigned block, hipStream_t st)
{
    switch (elems) {
    case 1: launch_e<T, R, W, 1>(nt, s, grid, block, st); break;
    case 2: launch_e<T, R, W, 2>(nt, s, grid, block, st); break;
    case 4: launch_e<T, R, W, 4>(nt, s, grid, block, st); break;
    default: launch_e<T, R, W, 8>(nt, s, grid, block, st); break;
    }
}

template <typename T>
using Launcher = void (*)(bool, int, const Streams<T> &, unsigned, unsigned, hipStream_t);

template <typename T>
Launcher<T> pick(int r, int w)
{
    static const Launcher<T> table[7][3] = {
        {launch<T, 1, 1>, launch<T, 1, 2>, launch<T, 1, 3>},
        {launch<T, 2, 1>, launch<T, 2, 2>, launch<T, 2, 3>},
        {launch<T, 3, 1>, launch<T, 3, 2>, launch<T, 3, 3>},
        {launch<T, 4, 1>, launch<T, 4, 2>, launch<T, 4, 3>},
        {launch<T, 5, 1>, launch<T, 5, 2>, launch<T, 5, 3>},
        {launch<T, 6, 1>, launch<T, 6, 2>, launch<T, 6, 3>},
        {launch<T, 7, 1>, launch<T, 7, 2>, launch<T, 7, 3>}};
    return table[r - 1][w - 1];
}

// Argument checks, timing and launches shared by both element types.
template <typename T>
int run(int32_t reads, int32_t writes, int32_t nontemporal, int32_t elems, int32_t block, int64_t n,
        const T *const *in_dev, T *const *out_dev, int32_t reps, void *stream, double *ms_per_launch)
{
    if (reads < 1 || reads > 7 || writes < 1 || writes > 3 ||
        (elems != 1 && elems != 2 && elems != 4 && elems != 8) || block < 64 || block > kMaxBlock ||
        block % 64 != 0 || n <= 0 || n % ((int64_t)block * elems) != 0 ||
        n / ((int64_t)block * elems) > 0x7fffffff || !in_dev || !out_dev || reps < 1 || !ms_per_launch)
        return -1;
    Streams<T> s{};
    for (int r = 0; r < reads; ++r) {
        if (!in_dev[r])
            return -1;
        s.in[r] = in_dev[r];
    }
    for (int w = 0; w < writes; ++w) {
        if (!out_dev[w])
            return -1;
        s.out[w] = out_dev[w];
    }
    const unsigned grid = (unsigned)(n / ((int64_t)block * elems));
    hipStream_t st = (hipStream_t)stream;
    const Launcher<T> f = pick<T>(reads, writes);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess)
        return -3;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -3;
    }
    for (int i = 0; i < 3; ++i)
        f(nontemporal != 0, elems, s, grid, (unsigned)block, st);
    hipError_t e = hipEventRecord(e0, st);
    for (int i = 0; e == hipSuccess && i < reps; ++i)
        f(nontemporal != 0, elems, s, grid, (unsigned)block, st);
    if (e == hipSuccess)
        e = hipEventRecord(e1, st);
    if (e == hipSuccess)
        e = hipEventSynchronize(e1);
    if (e == hipSuccess)
        e = hipGetLastError();
    float ms = 0.0f;
    if (e == hipSuccess)
        e = hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (e != hipSuccess)
        return -3;
    *ms_per_launch = (double)ms / reps;
    return 0;
}

}   // namespace

extern "C" {

// Time `reps` launches of the (reads, writes) streaming kernel on `stream`
// (a hipStream_t, NULL for the null stream) after 3 untimed ones, and store
// the average milliseconds per launch in *ms_per_launch.
//   reads 1..7, writes 1..3; elems (per thread) 1, 2, 4 or 8; block 64..1024,
//   a multiple of 64; n > 0 a multiple of block * elems; in_dev / out_dev:
//   HOST arrays of `reads` / `writes` device pointers to n doubles each
//   (n floats for mfprobe_stream_f32), the outputs distinct from each other
//   and from the inputs.
//   nontemporal != 0: non-temporal loads and stores (as the solver's
//   single-use streams), else ordinary ones.
// Returns 0, -1 for invalid arguments (nothing launched), -3 on a HIP error.
int mfprobe_stream(int32_t reads, int32_t writes, int32_t nontemporal, int32_t elems, int32_t block,
                   int64_t n, const double *const *in_dev, double *const *out_dev, int32_t reps,
                   void *stream, double *ms_per_launch)
{
    return run<double>(reads, writes, nontemporal, elems, block, n, in_dev, out_dev, reps, stream,
                       ms_per_launch);
}

int mfprobe_stream_f32(int32_t reads, int32_t writes, int32_t nontemporal, int32_t elems, int32_t block,
                       int64_t n, const float *const *in_dev, float *const *out_dev, int32_t reps,
                       void *stream, double *ms_per_launch)
{
    return run<float>(reads, writes, nontemporal, elems, block, n, in_dev, out_dev, reps, stream,
                      ms_per_launch);
}

}   // extern "C"
