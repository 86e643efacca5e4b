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

template <typename T>
__global__ __launch_bounds__(256) void build_refs_kernel(const T *__restrict__ x, int64_t t0,
                                                         int64_t nrows, int s, int d,
                                                         int64_t Rcap, int64_t j0, int64_t nj,
                                                         T *__restrict__ refs,
                                                         float *__restrict__ sqn) {
    const int lane = threadIdx.x & 63;
    const int64_t jj = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (jj >= nj) return;
    const int64_t unit = blockIdx.y;
    const int64_t j = j0 + jj;
    const T *src = x + (unit * nrows + (j * s - t0)) * d;
    T *dst = refs + (unit * Rcap + j) * d;
    float acc = 0.f;
    for (int i = lane; i < d; i += 64) {
        T v = src[i];
        dst[i] = v;
        float f = to_f32(v);
        acc += f * f;
    }
    acc = wave_sum(acc);
    if (lane == 0) sqn[unit * Rcap + j] = acc;
}

}  // namespace

hipError_t launch_build_refs(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                             const CacheArgs &c, hipStream_t st) {
    const int64_t j0 = refs_upto(t0, dm.s);
    const int64_t nj = refs_upto(t1, dm.s) - j0;
    if (nj <= 0) return hipSuccess;
    dim3 grid((unsigned)((nj + 3) / 4), (unsigned)(dm.B * dm.H));
    if (dm.dtype == 0)
        hipLaunchKernelGGL(build_refs_kernel<float>, grid, dim3(256), 0, st,
                           (const float *)x, t0, t1 - t0, dm.s, dm.d, dm.R, j0, nj,
                           (float *)c.refs, c.sqn);
    else
        hipLaunchKernelGGL(build_refs_kernel<bf16_t>, grid, dim3(256), 0, st,
                           (const bf16_t *)x, t0, t1 - t0, dm.s, dm.d, dm.R, j0, nj,
                           (bf16_t *)c.refs, c.sqn);
    return hipGetLastError();
}

}  // namespace dk
