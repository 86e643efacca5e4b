// k_refs.hip -- reference-set build ("DeltaKV: Residual-Based KV Cache
// Compression via Long-Range Similarity", section 3, "Struttura della
// Compressione": a fixed-stride subset of the tokens is kept verbatim).
//
// One wave per reference row: the row is copied bit for bit and its fp32
// squared norm (used to seed the approximate distance scores of the top-k
// search) is written beside it.  Pure copy, HBM bound.
#include "dk_common.h"
#include "dk_launch.h"

namespace dk {
namespace {

// One reference row by one wave: copy, and the fp32 squared norm (lane-strided
// partial sums, then a wave reduction).
template <typename T>
__device__ __forceinline__ void copy_ref_row(const T *__restrict__ src, T *__restrict__ dst,
                                             float *__restrict__ sqn_dst, int d, int lane) {
    float acc = 0.f;
    for (int i = lane; i < d; i += 64) {
        T v = src[i];
        dst[i] = v;
        float f = to_f32(v);
        acc += f * f;
    }
    acc = wave_sum(acc);
    if (lane == 0) *sqn_dst = acc;
}

// (paged layout, pm.tbl non-null: the row goes to its pool page)
template <typename T>
__global__ __launch_bounds__(256) void build_refs_kernel(const T *__restrict__ x, int64_t t0,
                                                         int64_t nrows, int s, int d,
                                                         int64_t Rcap, int64_t j0, int64_t nj,
                                                         T *__restrict__ refs,
                                                         float *__restrict__ sqn, PageMap pm) {
    const int lane = threadIdx.x & 63;
    const int64_t jj = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (jj >= nj) return;
    const int64_t unit = blockIdx.y;
    const int64_t j = j0 + jj;
    const int64_t row = pm.tbl ? pg_ref_row(pm, unit, j) : unit * Rcap + j;
    copy_ref_row<T>(x + (unit * nrows + (j * s - t0)) * d, refs + row * d, sqn + row, d, lane);
}

// Batched appends at a reference position t: the row of every unit of every
// cache of the set becomes reference t / s.  One wave per (unit, cache):
// grid (ceil(U / 4), n).
// (paged caches, pg.npp != 0: the row goes to its pool page)
__global__ __launch_bounds__(256) void append_refs_kernel(AppendSet set, int64_t t, int s, int d,
                                                          int64_t Rcap, int U, PageMap pg) {
    const int lane = threadIdx.x & 63;
    const int unit = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= U) return;
    const int item = blockIdx.y;
    const int64_t j = t / s;
    const int64_t row = pg.npp ? pg_ref_row(item_pages(pg, set, item), unit, j)
                               : (int64_t)unit * Rcap + j;
    const bf16_t *x = (const bf16_t *)set.x[item];
    copy_ref_row<bf16_t>(x + (int64_t)unit * d, (bf16_t *)set.refs[item] + row * d,
                         set.sqn[item] + row, d, lane);
}

}  // namespace

hipError_t launch_append_refs(const Dims &dm, int64_t t, int n, const AppendSet &set,
                              hipStream_t st) {
    const int U = dm.B * dm.H;
    hipLaunchKernelGGL(append_refs_kernel, dim3((unsigned)((U + 3) / 4), (unsigned)n), dim3(256),
                       0, st, set, t, dm.s, dm.d, dm.R, U, set_pages(dm));
    return hipGetLastError();
}

hipError_t launch_build_refs(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                             const CacheArgs &c, hipStream_t st) {
    const int64_t j0 = refs_upto(t0, dm.s);
    const int64_t nj = refs_upto(t1, dm.s) - j0;
    if (nj <= 0) return hipSuccess;
    dim3 grid((unsigned)((nj + 3) / 4), (unsigned)(dm.B * dm.H));
    const PageMap pm = dm.pr ? page_map(dm, c) : PageMap{};
    if (dm.dtype == 0)
        hipLaunchKernelGGL(build_refs_kernel<float>, grid, dim3(256), 0, st,
                           (const float *)x, t0, t1 - t0, dm.s, dm.d, dm.R, j0, nj,
                           (float *)c.refs, c.sqn, pm);
    else
        hipLaunchKernelGGL(build_refs_kernel<bf16_t>, grid, dim3(256), 0, st,
                           (const bf16_t *)x, t0, t1 - t0, dm.s, dm.d, dm.R, j0, nj,
                           (bf16_t *)c.refs, c.sqn, pm);
    return hipGetLastError();
}

}  // namespace dk
