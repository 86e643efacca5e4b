// k_select.hip -- choice of the k nearest reference rows of each compressed
// token ("DeltaKV: Residual-Based KV Cache Compression via Long-Range
// Similarity", section 3, "Processo di Compressione", step 1: the k most
// similar earlier tokens of the strided reference set, by L2 distance).
//
// Exact scan: one wave per token.  Lane l scores the candidate references
// j = l, l + 64, ... (those with j * s < p) with the squared distance summed
// in fp64 in coordinate order and with no fused multiply-add, keeps its own
// sorted top-k list, and the wave merges the 64 lists by k rounds of a
// lexicographic (distance, ordinal) minimum.  This decides the ranking in the
// same arithmetic as the ordering rule stated in the C ABI, so its result is
// unique and exact.  It serves the fp32 path, and the bf16 path's tokens whose
// approximate (MFMA) ranking could not be certified.
#include <limits.h>

#include "dk_common.h"
#include "dk_launch.h"

namespace dk {
namespace {

constexpr int kMaxK = 8;

// Squared distance between the fp64 row xs (LDS) and reference row r, summed
// in order with separately rounded products and sums.
template <typename T, int D>
__device__ __forceinline__ double exact_sq_dist(const double *xs, const T *__restrict__ r) {
#pragma clang fp contract(off)
    double acc = 0.0;
    if constexpr (sizeof(T) == 2) {
        const uint4 *rv = reinterpret_cast<const uint4 *>(r);
#pragma unroll 4
        for (int c = 0; c < D / 8; ++c) {
            uint4 u = rv[c];
            uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                double lo = (double)__uint_as_float(w[e] << 16);
                double hi = (double)__uint_as_float(w[e] & 0xffff0000u);
                double d0 = xs[c * 8 + 2 * e] - lo;
                double s0 = d0 * d0;
                acc = acc + s0;
                double d1 = xs[c * 8 + 2 * e + 1] - hi;
                double s1 = d1 * d1;
                acc = acc + s1;
            }
        }
    } else {
        const float4 *rv = reinterpret_cast<const float4 *>(r);
#pragma unroll 4
        for (int c = 0; c < D / 4; ++c) {
            float4 u = rv[c];
            float w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                double df = xs[c * 4 + e] - (double)w[e];
                double sq = df * df;
                acc = acc + sq;
            }
        }
    }
    return acc;
}

// Exact top-k of one token per wave.  Work item w of the launch is token
// ordinal q = q0 + w of unit `blockIdx.y` (range mode, list == nullptr), or
// the w-th entry of `list` (list mode: entries are unit << 32 | (q - q0),
// count in *list_count).
template <typename T, int D>
__global__ __launch_bounds__(256) void select_exact_kernel(
    const T *__restrict__ x, int64_t t0, int64_t nrows, int s, const T *__restrict__ refs,
    int64_t Rcap, int64_t Ncap, int64_t q0, int64_t nq, int k, uint16_t *__restrict__ idx,
    const uint64_t *__restrict__ list, const uint32_t *__restrict__ list_count) {
    __shared__ double xs_all[4][D];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    double *xs = xs_all[wv];

    int64_t unit, qrel;
    if (list) {
        const int64_t w = (int64_t)blockIdx.x * 4 + wv;
        if (w >= (int64_t)*list_count) return;
        const uint64_t e = list[w];
        unit = (int64_t)(e >> 32);
        qrel = (int64_t)(e & 0xffffffffu);
    } else {
        unit = blockIdx.y;
        qrel = (int64_t)blockIdx.x * 4 + wv;
        if (qrel >= nq) return;
    }
    const int64_t q = q0 + qrel;
    const int64_t p = tok_pos(q, s);
    const T *xrow = x + (unit * nrows + (p - t0)) * D;
    for (int i = lane; i < D; i += 64) xs[i] = to_f64(xrow[i]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int64_t ncand = (p + s - 1) / s;  // j * s < p
    const T *ubase = refs + unit * Rcap * D;

    double bd[kMaxK];
    int bj[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
        bd[i] = __builtin_inf();
        bj[i] = INT_MAX;
    }
    for (int64_t j = lane; j < ncand; j += 64) {
        double cd = exact_sq_dist<T, D>(xs, ubase + j * D);
        int cj = (int)j;
        if (!(cd < bd[kMaxK - 1] || (cd == bd[kMaxK - 1] && cj < bj[kMaxK - 1]))) continue;
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) {
            const bool lt = cd < bd[i] || (cd == bd[i] && cj < bj[i]);
            const double td = bd[i];
            const int tj = bj[i];
            bd[i] = lt ? cd : td;
            bj[i] = lt ? cj : tj;
            cd = lt ? td : cd;
            cj = lt ? tj : cj;
        }
    }
    uint16_t *out = idx + (unit * Ncap + q) * k;
    for (int r = 0; r < k; ++r) {
        double md = bd[0];
        int mj = bj[0];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double od = __shfl_xor(md, o, 64);
            const int oj = __shfl_xor(mj, o, 64);
            if (od < md || (od == md && oj < mj)) {
                md = od;
                mj = oj;
            }
        }
        if (mj != INT_MAX && bj[0] == mj) {  // the owning lane pops its head
#pragma unroll
            for (int i = 0; i + 1 < kMaxK; ++i) {
                bd[i] = bd[i + 1];
                bj[i] = bj[i + 1];
            }
            bd[kMaxK - 1] = __builtin_inf();
            bj[kMaxK - 1] = INT_MAX;
        }
        if (lane == 0) out[r] = (mj == INT_MAX) ? kIdxUnused : (uint16_t)mj;
    }
}

template <typename T, int D>
hipError_t launch_exact_t(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                          int64_t nq, const CacheArgs &c, const uint64_t *list,
                          const uint32_t *list_count, int64_t list_cap, hipStream_t st) {
    dim3 grid;
    if (list)
        grid = dim3((unsigned)((list_cap + 3) / 4), 1);
    else
        grid = dim3((unsigned)((nq + 3) / 4), (unsigned)(dm.B * dm.H));
    hipLaunchKernelGGL((select_exact_kernel<T, D>), grid, dim3(256), 0, st, (const T *)x, t0,
                       t1 - t0, dm.s, (const T *)c.refs, dm.R, dm.N, q0, nq, dm.k, c.idx, list,
                       list_count);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select_exact(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                               int64_t q0, int64_t nq, const CacheArgs &c,
                               const uint64_t *list, const uint32_t *list_count,
                               int64_t list_cap, hipStream_t st) {
    if (dm.dtype == 0)
        return dm.d == 64 ? launch_exact_t<float, 64>(dm, x, t0, t1, q0, nq, c, list,
                                                      list_count, list_cap, st)
                          : launch_exact_t<float, 128>(dm, x, t0, t1, q0, nq, c, list,
                                                       list_count, list_cap, st);
    return dm.d == 64 ? launch_exact_t<bf16_t, 64>(dm, x, t0, t1, q0, nq, c, list, list_count,
                                                   list_cap, st)
                      : launch_exact_t<bf16_t, 128>(dm, x, t0, t1, q0, nq, c, list,
                                                    list_count, list_cap, st);
}

}  // namespace dk
