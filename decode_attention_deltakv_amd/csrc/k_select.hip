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

#include <algorithm>

#include "dk_common.h"
#include "dk_launch.h"
#include "dk_mfma.h"

namespace dk {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Reference-range splits of the matrix-core top-k search: when the token tiles
// of a call give fewer than two blocks per CU (a prompt compressed in chunks),
// each tile's references are split so that the call has about kSplitTarget
// blocks, at least 512 references (8 stages) per split.  Each split warms up
// its own candidate lists (insertions while they fill), so half a round of
// resident blocks measures faster than a full one.
constexpr int64_t kSplitTarget = 384;

void topk_split_plan(const Dims &dm, int64_t t1, int64_t nq, int *nsplit, int *chunk) {
    const int64_t U = (int64_t)dm.B * dm.H;
    const int64_t blocks = std::max<int64_t>(1, (nq + 255) / 256 * U);
    const int64_t R = std::max<int64_t>(1, refs_upto(t1, dm.s));
    int64_t n = 1;
    if (blocks < 512) n = std::max<int64_t>(1, std::min((kSplitTarget + blocks - 1) / blocks, (R + 511) / 512));
    int64_t c = (R + n - 1) / n;
    c = (c + 63) / 64 * 64;
    *nsplit = (int)((R + c - 1) / c);
    *chunk = (int)c;
}

// Workspace beyond the fallback list that the split search needs.
// Candidate list length of the matrix-core search for k <= 4 and k <= 8:
// the k best plus a margin, so that the list's last entry usually clears the
// k-th exact distance by more than the certificate's error terms (a shorter
// list means fewer insertions; a failed certificate costs an exact scan).
constexpr int kListLen4 = 7;
constexpr int kListLen8 = 12;

// Workspace sizes below are taken at the plans' upper bounds on the split
// count, which never decrease as references accumulate, so a workspace sized
// for a later position serves every earlier one.
size_t topk_split_ws_bytes(const Dims &dm, int64_t t1, int64_t nq) {
    const int64_t U0 = (int64_t)dm.B * dm.H;
    const int64_t blocks = std::max<int64_t>(1, (nq + 255) / 256 * U0);
    const int64_t R = std::max<int64_t>(1, refs_upto(t1, dm.s));
    // topk_split_plan's count n bounds its realised split count
    const int64_t nsplit =
        blocks < 512 ? std::max<int64_t>(1, std::min((kSplitTarget + blocks - 1) / blocks, (R + 511) / 512))
                     : 1;
    if (nsplit <= 1) return 0;
    const int LK = dm.k <= 4 ? kListLen4 : kListLen8;
    const int64_t U = (int64_t)dm.B * dm.H;
    const int64_t ntiles = (nq + 255) / 256;
    return align256((size_t)nsplit * U * nq * LK * sizeof(float)) +
           align256((size_t)nsplit * U * ntiles * sizeof(float));
}

// Reference chunk per block and block count of the split exact scans (a few
// tokens of a streaming append, or the listed tokens the matrix-core search
// could not certify): at least 256 references per block, at most kSplitMax
// blocks per token.
static void split_plan(const Dims &dm, int64_t t1, int *chunk, int *nsplit) {
    const int64_t rmax = std::max<int64_t>(1, refs_upto(t1, dm.s));
    const int64_t c = std::max<int64_t>(256, (rmax + kSplitMax - 1) / kSplitMax);
    *chunk = (int)c;
    *nsplit = (int)((rmax + c - 1) / c);
}

// Listed tokens whose exact scan is split over waves; further entries of a
// fallback list take one block each.
constexpr int64_t kListSplitCap = 4096;
constexpr int kMaxK = 8;

// Reference chunk per wave and wave count per token of the split scan of a
// fallback list: 64 references (one per lane) per wave, more (a multiple of
// 64) once a token would need over 128 waves, which bounds the candidates
// its merge reads.
static void list_split_plan(const Dims &dm, int64_t t1, int *chunk, int *nsplit) {
    const int64_t rmax = std::max<int64_t>(1, refs_upto(t1, dm.s));
    const int64_t c = ((rmax + 127) / 128 + 63) / 64 * 64;
    *chunk = (int)c;
    *nsplit = (int)((rmax + c - 1) / c);
}

size_t exact_list_ws_bytes(const Dims &dm, int64_t t1, int64_t nitems) {
    // list_split_plan's chunk is at least 64 and at least rmax / 128
    const int64_t rmax = std::max<int64_t>(1, refs_upto(t1, dm.s));
    const int64_t nsplit = std::min<int64_t>((rmax + 63) / 64, 128);
    // (a list holds at most one entry per unit and token of the call)
    return (size_t)std::min<int64_t>(kListSplitCap, std::max<int64_t>(1, nitems)) * nsplit *
           kMaxK * (sizeof(double) + sizeof(int));
}

namespace {

// threads of the block-per-token exact scan
constexpr int kExactThreads = 1024;

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

// The same distance for four reference rows at once (four independent sums,
// each in coordinate order): one pass over xs, four add chains in flight.
template <int D>
__device__ __forceinline__ void exact_sq_dist4(const double *xs, const bf16_t *r0,
                                               const bf16_t *r1, const bf16_t *r2,
                                               const bf16_t *r3, double (&acc)[4]) {
#pragma clang fp contract(off)
    const uint4 *rv[4] = {reinterpret_cast<const uint4 *>(r0), reinterpret_cast<const uint4 *>(r1),
                          reinterpret_cast<const uint4 *>(r2), reinterpret_cast<const uint4 *>(r3)};
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = 0.0;
#pragma unroll 2
    for (int c = 0; c < D / 8; ++c) {
        uint4 u[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) u[v] = rv[v][c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double xe = xs[c * 8 + e];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t wv = (e >> 1) == 0 ? u[v].x : (e >> 1) == 1 ? u[v].y
                                  : (e >> 1) == 2 ? u[v].z : u[v].w;
                const double rr = (double)__uint_as_float((e & 1) ? (wv & 0xffff0000u) : (wv << 16));
                const double df = xe - rr;
                const double sq = df * df;
                acc[v] = acc[v] + sq;
            }
        }
    }
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

    const int64_t nwork = list ? (int64_t)*list_count : nq;
    const int64_t wstep = list ? (int64_t)gridDim.x * 4 : (int64_t)1 << 62;
    for (int64_t wi = (int64_t)blockIdx.x * 4 + wv; wi < nwork; wi += wstep) {
    int64_t unit, qrel;
    if (list) {
        const uint64_t e = list[wi];
        unit = (int64_t)(e >> 32);
        qrel = (int64_t)(e & 0xffffffffu);
    } else {
        unit = blockIdx.y;
        qrel = wi;
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Exact top-k of listed tokens, one block per token (grid-stride over the
// list): the NT threads split the candidate references (bf16: four per
// thread and pass, so four independent fp64 sums are in flight), each keeps
// a sorted top-k of its share, and the block merges the lists by k rounds of
// a lexicographic (distance, ordinal) minimum.  Same arithmetic as the
// wave-per-token scan (the result does not depend on NT); used for the few
// tokens the matrix-core search could not certify.
template <typename T, int D, int NT = kExactThreads>
__global__ __launch_bounds__(NT) void select_exact_block_kernel(
    const T *__restrict__ x, int64_t t0, int64_t nrows, int s, const T *__restrict__ refs,
    int64_t Rcap, int64_t Ncap, int64_t q0, int k, uint16_t *__restrict__ idx,
    const uint64_t *__restrict__ list, const uint32_t *__restrict__ list_count, int64_t nunits,
    int64_t nq, int64_t first) {
    constexpr int NW = NT / 64;
    __shared__ double xs[D];
    __shared__ double wd[NW];
    __shared__ int wj[NW];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // work items: the listed (unit, token) entries from `first` on, or
    // without a list every token of [q0, q0 + nq) of every unit
    const int64_t n = list ? (int64_t)*list_count : nunits * nq;
    for (int64_t wi = first + blockIdx.x; wi < n; wi += gridDim.x) {
        const uint64_t e = list ? list[wi] : (((uint64_t)(wi / nq) << 32) | (uint64_t)(wi % nq));
        const int64_t unit = (int64_t)(e >> 32);
        const int64_t q = q0 + (int64_t)(e & 0xffffffffu);
        const int64_t p = tok_pos(q, s);
        const T *xrow = x + (unit * nrows + (p - t0)) * D;
        __syncthreads();
        for (int i = tid; i < D; i += NT) xs[i] = to_f64(xrow[i]);
        __syncthreads();
        const int ncand = (int)((p + s - 1) / s);
        const T *ubase = refs + unit * Rcap * D;
        double bd[kMaxK];
        int bj[kMaxK];
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) {
            bd[i] = __builtin_inf();
            bj[i] = INT_MAX;
        }
        auto offer = [&](double cd, int cj) {
            if (!(cd < bd[kMaxK - 1] || (cd == bd[kMaxK - 1] && cj < bj[kMaxK - 1]))) return;
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
        };
        if constexpr (sizeof(T) == 2) {
            // four references per thread and pass: j, j + NT, j + 2 NT, j + 3 NT
            for (int j = tid; j < ncand; j += 4 * NT) {
                int jv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) jv[v] = min(j + v * NT, ncand - 1);
                double cd[4];
                exact_sq_dist4<D>(xs, ubase + (int64_t)jv[0] * D, ubase + (int64_t)jv[1] * D,
                                  ubase + (int64_t)jv[2] * D, ubase + (int64_t)jv[3] * D, cd);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (j + v * NT < ncand) offer(cd[v], j + v * NT);
            }
        } else {
            for (int j = tid; j < ncand; j += NT) offer(exact_sq_dist<T, D>(xs, ubase + (int64_t)j * D), j);
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
            if (lane == 0) {
                wd[wv] = md;
                wj[wv] = mj;
            }
            __syncthreads();
            md = wd[0];
            mj = wj[0];
#pragma unroll
            for (int i = 1; i < NW; ++i)
                if (wd[i] < md || (wd[i] == md && wj[i] < mj)) {
                    md = wd[i];
                    mj = wj[i];
                }
            __syncthreads();
            if (mj != INT_MAX && bj[0] == mj) {
#pragma unroll
                for (int i = 0; i + 1 < kMaxK; ++i) {
                    bd[i] = bd[i + 1];
                    bj[i] = bj[i + 1];
                }
                bd[kMaxK - 1] = __builtin_inf();
                bj[kMaxK - 1] = INT_MAX;
            }
            if (tid == 0) out[r] = (mj == INT_MAX) ? kIdxUnused : (uint16_t)mj;
        }
    }
}

// Exact kMaxK best (distance, ordinal) pairs of one token row over the
// references [ja, jb) of one unit, by a block of 256 threads: each thread
// keeps a sorted list of its share (the same fp64 arithmetic as the scans
// above), then kMaxK rounds of a block-wide lexicographic minimum write the
// merged list to od / oj (unused slots: +inf, INT_MAX).  Every thread of the
// block must call it; xs, wd and wj are the block's LDS scratch.
// (rows: reference ordinal -> its row, e.g. ubase + j D, or a pool row of a
// paged cache)
template <typename T, int D, typename Rows>
__device__ __forceinline__ void block_range_topk(const T *__restrict__ xrow, Rows rows,
                                 int64_t ja, int64_t jb, double *xs, double *wd, int *wj,
                                 double *__restrict__ od, int *__restrict__ oj) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    __syncthreads();
    for (int i = tid; i < D; i += 256) xs[i] = to_f64(xrow[i]);
    __syncthreads();
    double bd[kMaxK];
    int bj[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
        bd[i] = __builtin_inf();
        bj[i] = INT_MAX;
    }
    for (int64_t j = ja + tid; j < jb; j += 256) {
        double cd = exact_sq_dist<T, D>(xs, rows(j));
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
    for (int r = 0; r < kMaxK; ++r) {
        double md = bd[0];
        int mj = bj[0];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double odd = __shfl_xor(md, o, 64);
            const int ojj = __shfl_xor(mj, o, 64);
            if (odd < md || (odd == md && ojj < mj)) {
                md = odd;
                mj = ojj;
            }
        }
        if (lane == 0) {
            wd[wv] = md;
            wj[wv] = mj;
        }
        __syncthreads();
        md = wd[0];
        mj = wj[0];
#pragma unroll
        for (int i = 1; i < 4; ++i)
            if (wd[i] < md || (wd[i] == md && wj[i] < mj)) {
                md = wd[i];
                mj = wj[i];
            }
        __syncthreads();
        if (mj != INT_MAX && bj[0] == mj) {
#pragma unroll
            for (int i = 0; i + 1 < kMaxK; ++i) {
                bd[i] = bd[i + 1];
                bj[i] = bj[i + 1];
            }
            bd[kMaxK - 1] = __builtin_inf();
            bj[kMaxK - 1] = INT_MAX;
        }
        if (tid == 0) {
            od[r] = md;
            oj[r] = mj;
        }
    }
}

// The k best (distance, ordinal) of nsplit partial lists of one token (each
// kMaxK long, sorted; only their first k entries can make the result), by
// one wave; written to out (kIdxUnused past the candidates).  Candidates are
// read eight per lane at a time, all loads before the insertions.
__device__ __forceinline__ void wave_merge_lists(int nsplit, int k, const double *__restrict__ cd_,
                                 const int *__restrict__ cj_, uint16_t *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    double bd[kMaxK];
    int bj[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
        bd[i] = __builtin_inf();
        bj[i] = INT_MAX;
    }
    const int n = nsplit * k;
    for (int base = 0; base < n; base += 8 * 64) {
        double vd[8];
        int vj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = base + 64 * u + lane;
            const int at = (c / k) * kMaxK + c % k;
            vd[u] = c < n ? cd_[at] : __builtin_inf();
            vj[u] = c < n ? cj_[at] : INT_MAX;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            double cd = vd[u];
            int cj = vj[u];
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
    }
    for (int r = 0; r < k; ++r) {
        double md = bd[0];
        int mj = bj[0];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double odd = __shfl_xor(md, o, 64);
            const int ojj = __shfl_xor(mj, o, 64);
            if (odd < md || (odd == md && ojj < mj)) {
                md = odd;
                mj = ojj;
            }
        }
        if (mj != INT_MAX && bj[0] == mj) {
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

// Exact top-k of a few tokens with their candidate references split over many
// blocks (a streaming append has one token per unit but up to 65535
// references): block (split, item) scans references [split * chunk, ...) of
// token item and writes its kMaxK best pairs; select_merge_kernel takes the
// k best over all splits.  grid (nsplit, units * nq).
template <typename T, int D>
__global__ __launch_bounds__(256) void select_split_kernel(
    const T *__restrict__ x, int64_t t0, int64_t nrows, int s, const T *__restrict__ refs,
    int64_t Rcap, int64_t q0, int64_t nq, int chunk, double *__restrict__ pd,
    int *__restrict__ pj) {
    __shared__ double xs[D];
    __shared__ double wd[4];
    __shared__ int wj[4];
    const int64_t item = blockIdx.y;
    const int64_t unit = item / nq, q = q0 + item % nq;
    const int64_t p = tok_pos(q, s);
    const int64_t ncand = (p + s - 1) / s;
    const int64_t ja = (int64_t)blockIdx.x * chunk, jb = min(ncand, ja + (int64_t)chunk);
    const size_t o = (size_t)(item * gridDim.x + blockIdx.x) * kMaxK;
    const T *ubase = refs + unit * Rcap * D;
    block_range_topk<T, D>(x + (unit * nrows + (p - t0)) * D,
                           [=](int64_t j) { return ubase + j * D; }, ja, jb, xs,
                           wd, wj, pd + o, pj + o);
}

// The k best (distance, ordinal) of the nsplit partial lists of one token;
// one wave per token.
__global__ __launch_bounds__(64) void select_merge_kernel(int nsplit, int k, int64_t q0,
                                                          int64_t nq, int64_t Ncap,
                                                          const double *__restrict__ pd,
                                                          const int *__restrict__ pj,
                                                          uint16_t *__restrict__ idx) {
    const int64_t item = blockIdx.x;
    const int64_t unit = item / nq, q = q0 + item % nq;
    wave_merge_lists(nsplit, k, pd + item * nsplit * kMaxK, pj + item * nsplit * kMaxK,
                     idx + (unit * Ncap + q) * k);
}

// Batched appends: the exact top-k of the one new token t of every unit of
// every cache of the set over its references [0, ceil(t / s)), split over
// blocks as above.  grid (nsplit, U, n); lists at ((item U + unit) nsplit +
// split) kMaxK.
template <int D>
__global__ __launch_bounds__(256) void append_split_kernel(AppendSet set, int64_t t, int s,
                                                           int64_t Rcap, int chunk,
                                                           double *__restrict__ pd,
                                                           int *__restrict__ pj, PageMap pg) {
    __shared__ double xs[D];
    __shared__ double wd[4];
    __shared__ int wj[4];
    const int item = blockIdx.z, U = gridDim.y;
    const int64_t unit = blockIdx.y;
    const int64_t ncand = (t + s - 1) / s;
    const int64_t ja = (int64_t)blockIdx.x * chunk, jb = min(ncand, ja + (int64_t)chunk);
    const size_t o = (size_t)(((int64_t)item * U + unit) * gridDim.x + blockIdx.x) * kMaxK;
    const bf16_t *rb = (const bf16_t *)set.refs[item];
    if (pg.npp) {   // paged: each reference row found through the cache's table
        const PageMap pm = item_pages(pg, set, item);
        block_range_topk<bf16_t, D>((const bf16_t *)set.x[item] + unit * D,
                                    [=](int64_t j) { return rb + pg_ref_row(pm, unit, j) * D; },
                                    ja, jb, xs, wd, wj, pd + o, pj + o);
    } else {
        const bf16_t *ub = rb + unit * Rcap * D;
        block_range_topk<bf16_t, D>((const bf16_t *)set.x[item] + unit * D,
                                    [=](int64_t j) { return ub + j * D; }, ja, jb, xs, wd, wj,
                                    pd + o, pj + o);
    }
}

// The k best over the split lists of one (unit, cache), one wave each:
// grid (U, n); the index row of token ordinal q.
__global__ __launch_bounds__(64) void append_merge_kernel(AppendSet set, int nsplit, int k,
                                                          int64_t q, int64_t Ncap,
                                                          const double *__restrict__ pd,
                                                          const int *__restrict__ pj, PageMap pg) {
    const int item = blockIdx.y, U = gridDim.x;
    const int64_t unit = blockIdx.x;
    const int64_t o = ((int64_t)item * U + unit) * nsplit * kMaxK;
    const int64_t row = pg.npp ? pg_tok_row(item_pages(pg, set, item), unit, q) : unit * Ncap + q;
    wave_merge_lists(nsplit, k, pd + o, pj + o, set.idx[item] + row * k);
}

// Squared distance of one bf16 reference row (already loaded, u) from the
// fp64 row xs: the same arithmetic and order as exact_sq_dist.
template <int D>
__device__ __forceinline__ double exact_sq_dist_regs(const double *xs, const uint4 (&u)[D / 8]) {
#pragma clang fp contract(off)
    // an opaque offset keeps the row's LDS reads inside a caller's loop
    // (hoisted, they would hold the whole fp64 row in registers)
    int off = 0;
    asm volatile("" : "+v"(off));
    xs += off;
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        const uint32_t w[4] = {u[c].x, u[c].y, u[c].z, u[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = (double)__uint_as_float(w[e] << 16);
            const double hi = (double)__uint_as_float(w[e] & 0xffff0000u);
            const double d0 = xs[c * 8 + 2 * e] - lo;
            const double s0 = d0 * d0;
            acc = acc + s0;
            const double d1 = xs[c * 8 + 2 * e + 1] - hi;
            const double s1 = d1 * d1;
            acc = acc + s1;
        }
    }
    return acc;
}

template <int D>
__device__ __forceinline__ void load_row(const bf16_t *__restrict__ r, uint4 (&u)[D / 8]) {
    const uint4 *rv = reinterpret_cast<const uint4 *>(r);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) u[c] = rv[c];
}

// The same split scan for the first min(*list_count, cap) entries of a
// fallback list (entries unit << 32 | (q - q0); the count is known on the
// device only), one wave per work item (entry e, split sp), grid-stride: lane
// l scores references ja + l, ja + l + 64, ... below jb, keeps a sorted list,
// and kMaxK rounds of a wave-wide lexicographic minimum write the item's list.
template <int D>
__global__ __launch_bounds__(256) void select_list_split_kernel(
    const bf16_t *__restrict__ x, int64_t t0, int64_t nrows, int s,
    const bf16_t *__restrict__ refs, int64_t Rcap, int64_t q0, const uint64_t *__restrict__ list,
    const uint32_t *__restrict__ list_count, int64_t cap, int nsplit, int chunk,
    double *__restrict__ pd, int *__restrict__ pj) {
    __shared__ double xs_all[4][D];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    double *xs = xs_all[wv];
    const int64_t n = min((int64_t)*list_count, cap) * nsplit;
    const int64_t wstep = (int64_t)gridDim.x * 4;
    for (int64_t wi = (int64_t)blockIdx.x * 4 + wv; wi < n; wi += wstep) {
        const int64_t e = wi / nsplit;
        const int sp = (int)(wi % nsplit);
        const uint64_t ent = list[e];
        const int64_t unit = (int64_t)(ent >> 32);
        const int64_t q = q0 + (int64_t)(ent & 0xffffffffu);
        const int64_t p = tok_pos(q, s);
        const int64_t ncand = (p + s - 1) / s;
        const int64_t ja = (int64_t)sp * chunk, jb = min(ncand, ja + (int64_t)chunk);
        const bf16_t *xrow = x + (unit * nrows + (p - t0)) * D;
        const bf16_t *ubase = refs + unit * Rcap * D;
        // the lane's first reference row is requested before the token row
        // is staged, so the two memory round trips overlap
        uint4 u[D / 8];
        load_row<D>(ubase + (ja < jb ? min(ja + lane, jb - 1) : 0) * D, u);
        for (int i = lane; i < D; i += 64) xs[i] = (double)bf2f(xrow[i]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        double bd[kMaxK];
        int bj[kMaxK];
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) {
            bd[i] = __builtin_inf();
            bj[i] = INT_MAX;
        }
        for (int64_t j = ja + lane; j < jb; j += 64) {
            if (j != ja + lane) load_row<D>(ubase + j * D, u);
            double cd = exact_sq_dist_regs<D>(xs, u);
            int cj = (int)j;
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
        double *od = pd + wi * kMaxK;
        int *oj = pj + wi * kMaxK;
        for (int r = 0; r < kMaxK; ++r) {
            double md = bd[0];
            int mj = bj[0];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const double odd = __shfl_xor(md, o, 64);
                const int ojj = __shfl_xor(mj, o, 64);
                if (odd < md || (odd == md && ojj < mj)) {
                    md = odd;
                    mj = ojj;
                }
            }
            if (mj != INT_MAX && bj[0] == mj) {
#pragma unroll
                for (int i = 0; i + 1 < kMaxK; ++i) {
                    bd[i] = bd[i + 1];
                    bj[i] = bj[i + 1];
                }
                bd[kMaxK - 1] = __builtin_inf();
                bj[kMaxK - 1] = INT_MAX;
            }
            if (lane == 0) {
                od[r] = md;
                oj[r] = mj;
            }
        }
        // the next item rewrites xs
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

__global__ void zero_u32_kernel(uint32_t *p) {
    if (threadIdx.x == 0) *p = 0u;
}

__global__ void add_stats_kernel(const uint32_t *count, uint32_t *stats) {
    if (threadIdx.x == 0) atomicAdd(stats, *count);
}

// Merge of select_list_split_kernel's lists: one wave per entry, grid-stride.
// Also adds the list's length to *stats (when given), once.
__global__ __launch_bounds__(256) void select_list_merge_kernel(
    int nsplit, int k, int64_t q0, int64_t Ncap, const uint64_t *__restrict__ list,
    const uint32_t *__restrict__ list_count, int64_t cap, const double *__restrict__ pd,
    const int *__restrict__ pj, uint16_t *__restrict__ idx, uint32_t *__restrict__ stats) {
    const uint32_t cnt = *list_count;
    if (stats && blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(stats, cnt);
    const int64_t n = min((int64_t)cnt, cap);
    const int64_t wstep = (int64_t)gridDim.x * 4;
    for (int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); e < n; e += wstep) {
        const uint64_t ent = list[e];
        const int64_t unit = (int64_t)(ent >> 32);
        const int64_t q = q0 + (int64_t)(ent & 0xffffffffu);
        wave_merge_lists(nsplit, k, pd + e * nsplit * kMaxK, pj + e * nsplit * kMaxK,
                         idx + (unit * Ncap + q) * k);
    }
}

template <typename T, int D>
hipError_t launch_exact_t(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                          int64_t nq, const CacheArgs &c, const uint64_t *list,
                          const uint32_t *list_count, int64_t list_cap, void *scratch,
                          size_t scratch_bytes, uint32_t *stats, hipStream_t st) {
    if (list) {
        // grids sized for the usual few entries (the count is on the device);
        // the kernels walk longer lists grid-stride
        // the first entries with their references split over blocks (as many
        // as the scratch holds partial lists for), the rest one block each
        int64_t first = 0;
        if constexpr (sizeof(T) == 2) {
            int chunk, nsplit;
            list_split_plan(dm, t1, &chunk, &nsplit);
            const size_t per = (size_t)nsplit * kMaxK * (sizeof(double) + sizeof(int));
            const int64_t cap = std::min<int64_t>({list_cap, kListSplitCap,
                                                   scratch ? (int64_t)(scratch_bytes / per) : 0});
            if (cap > 0) {
                double *pd = (double *)scratch;
                int *pj = (int *)((char *)scratch + (size_t)cap * nsplit * kMaxK * sizeof(double));
                const unsigned g = (unsigned)std::min<int64_t>((cap * nsplit + 3) / 4, 256);
                hipLaunchKernelGGL((select_list_split_kernel<D>), dim3(g), dim3(256), 0, st,
                                   (const bf16_t *)x, t0, t1 - t0, dm.s, (const bf16_t *)c.refs,
                                   dm.R, q0, list, list_count, cap, nsplit, chunk, pd, pj);
                hipLaunchKernelGGL(select_list_merge_kernel,
                                   dim3((unsigned)std::min<int64_t>((cap + 3) / 4, 64)), dim3(256),
                                   0, st, nsplit, dm.k, q0, dm.N, list, list_count, cap, pd, pj,
                                   c.idx, stats);
                stats = nullptr;   // counted
                first = cap;
            }
        }
        if (stats) hipLaunchKernelGGL(add_stats_kernel, dim3(1), dim3(64), 0, st, list_count, stats);
        if (first < list_cap) {
            // entries past the split scan's share (rarely any): blocks of 256
            // threads, which find room on a CU that other streams' kernels
            // share (a 1024-thread block can wait long for one, and the
            // stream's later kernels with it)
            const unsigned g =
                (unsigned)std::max<int64_t>(1, std::min<int64_t>(list_cap - first, 256));
            hipLaunchKernelGGL((select_exact_block_kernel<T, D, 256>), dim3(g), dim3(256), 0,
                               st, (const T *)x, t0, t1 - t0, dm.s, (const T *)c.refs, dm.R, dm.N,
                               q0, dm.k, c.idx, list, list_count, (int64_t)dm.B * dm.H, nq, first);
        }
        return hipGetLastError();
    }
    if (nq <= kSmallRange) {
        // a few tokens (a streaming append): one block per token, the
        // references split over its threads
        const int64_t n = (int64_t)dm.B * dm.H * nq;
        const unsigned g = (unsigned)std::min<int64_t>(n, 1024);
        hipLaunchKernelGGL((select_exact_block_kernel<T, D>), dim3(g), dim3(kExactThreads), 0, st,
                           (const T *)x, t0, t1 - t0, dm.s, (const T *)c.refs, dm.R, dm.N, q0,
                           dm.k, c.idx, nullptr, nullptr, (int64_t)dm.B * dm.H, nq, (int64_t)0);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((nq + 3) / 4), (unsigned)(dm.B * dm.H));
    hipLaunchKernelGGL((select_exact_kernel<T, D>), grid, dim3(256), 0, st, (const T *)x, t0,
                       t1 - t0, dm.s, (const T *)c.refs, dm.R, dm.N, q0, nq, dm.k, c.idx, list,
                       list_count);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Matrix-core top-k (bf16 storage).
//
// The matrix cores give approximate squared distances directly: with the
// token operand scaled by -2 (exact in bf16), the accumulator seeded with
// the reference's fp32 norm |r|^2 and one 32x32x8 step that adds the token's
// fp32 norm |x|^2 (split into three bf16 pieces whose sum is that fp32 value
// exactly, times a column of ones), a chain of 32x32x16 bf16 MFMAs yields
// S = |r|^2 - 2 x.r + |x|^2 ~ |x - r|^2.  References are the M
// dimension, tokens the N dimension, so each lane holds 16 values of one
// token per 32-reference block.  A block takes 256 consecutive compressed
// tokens (4 waves x 2 N-tiles of 32) and streams the references they can see
// (j * s < p) and their norms through LDS in stages of 64, double-buffered,
// loaded straight from global memory with 16-byte chunks XOR-swizzled per row
// (row % 16 for head_dim 128, (row / 2) % 8 for 64: the 16 rows one pass of a
// 16-byte LDS read touches then fall in disjoint banks).
//
// Per lane, a descending list of the LK largest -S is kept as packed floats:
// the low `ibits` mantissa bits of each value are replaced by imask - ordinal
// (the order among values equal after truncation does not matter for the
// result, which the exact rescore and the certificate decide), which lets one
// insertion be LK v_med3 operations with the negation folded into their
// source modifiers and one packing be a single bitwise instruction.  After
// each 32 x 32 product the two lane halves exchange values (one
// v_permlane32_swap per register) so that every lane holds all 32 values of
// one token and keeps one list; at the end the LK candidates are rescored
// exactly (fp64, coordinate order, no fused multiply-add) and sorted by
// (distance, ordinal).  The result is written only when a certificate holds:
// every reference outside the list has an approximate S of at least minus
// the list's last entry (less its truncation), hence a true distance of at
// least -tau - delta, where delta bounds the fp32 accumulation error of the
// MFMA chain and of the two fp32 norms; this lower bound must exceed the k-th
// exact distance.  As S is of the size of the distances themselves (not of
// |x|^2), the truncation costs a relative 2^(ibits - 22) of the distance.
// Tokens that fail go to a list for the exact scan.

// the low bits of a packed score hold imask - j (one instruction to pack)
__device__ __forceinline__ float pack_score(float sc, uint32_t code, uint32_t nmask) {
    return __uint_as_float((__float_as_uint(sc) & nmask) | code);
}
__device__ __forceinline__ int unpack_ordinal(float v, uint32_t imask) {
    return (int)(imask - (__float_as_uint(v) & imask));
}

template <int LK>
__device__ __forceinline__ void list_insert(float (&a)[LK], float v) {
#pragma unroll
    for (int i = LK - 1; i > 0; --i) a[i] = __builtin_amdgcn_fmed3f(a[i - 1], a[i], v);
    // max(a[0], v) as one instruction: the list holds no NaN, so the
    // NaN-quieting operations the compiler adds around fmaxf are not needed
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(a[0]), "v"(v));
    a[0] = m;
}

// Insertion of -v (the negations are source modifiers of the same
// instructions).
template <int LK>
__device__ __forceinline__ void list_insert_neg(float (&a)[LK], float v) {
#pragma unroll
    for (int i = LK - 1; i > 0; --i) a[i] = __builtin_amdgcn_fmed3f(a[i - 1], a[i], -v);
    float m;
    asm("v_max_f32_e64 %0, %1, -%2" : "=v"(m) : "v"(a[0]), "v"(v));
    a[0] = m;
}

// Lower bound on the true squared distance of every reference the search
// excluded, from the list's last entry tp (a packed -S): S >= -tau with tau
// = tp + |tp| 2^(ibits - 22) (the packing moves a value by less than
// |value| 2^(ibits - 23)), and |S - |x - r|^2| <= delta: the chain sums
// D + 16 products and the two norms, each partial sum rounded within 2^-23
// of itself (round to nearest or toward zero), so its error is at most
// gam (2 |x||r| + |x|^2 + |r|^2) = gam (|x| + |r|)^2; the fp32 norms
// themselves are within gam of |x|^2 and |r|^2.  xn and rm bound |x| and
// every excluded |r|.
template <int D>
__device__ __forceinline__ double excluded_lower_bound(float tpf, int ibits, double xn,
                                                       double rm) {
    // every term and partial sum of the chain must stay finite in fp32
    if ((xn + rm) * (xn + rm) > 1e38) return -INFINITY;
    const double tp = (double)tpf;
    const double tau = tp + fabs(tp) * ldexp(1.0, ibits - 22);
    const double nu = (double)(D + 16) * ldexp(1.0, -23);
    const double gam = nu / (1.0 - nu);
    const double delta = 2.0 * gam * (xn + rm) * (xn + rm) + 1e-30 * (1.0 + rm * rm);
    // the bound itself is evaluated in fp64: keep a relative margin for it
    return -tau - delta - 1e-9 * (fabs(tau) + delta + xn * xn);
}

// The k result ordinals of a token (kIdxUnused past the kk found), as one
// 8- or 16-byte store for k = 4 or 8 (the index row is then aligned to its
// size), else one store per slot.
template <int LK>
__device__ __forceinline__ void store_idx(uint16_t *__restrict__ out, const int (&jj)[LK], int k,
                                          int kk) {
    auto at = [&](int r) -> uint32_t {
        return r < kk ? ((uint32_t)jj[r] & 0xffffu) : (uint32_t)kIdxUnused;
    };
    if (k == 4 && LK >= 4) {
        u32x2 v;
        v[0] = at(0) | (at(1) << 16);
        v[1] = at(2) | (at(3) << 16);
        *reinterpret_cast<u32x2 *>(out) = v;
    } else if (k == 8 && LK >= 8) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = at(2 * i) | (at(2 * i + 1) << 16);
        *reinterpret_cast<u32x4 *>(out) = v;
    } else {
#pragma unroll
        for (int r = 0; r < LK; ++r)
            if (r < k) out[r] = (uint16_t)at(r);
    }
}

// Exact rescore of one token's LK candidates in one lane: fp64 distances in
// coordinate order without fused multiply-add, sort by (distance, ordinal),
// certificate; the result or a fallback entry is written.  ncand is the
// token's reference count: a list that is not full must hold all of them.
// CU chunks of 16 bytes are requested per candidate at once (memory round
// trips: D / 8 / CU; registers: 4 LK CU).
template <int D, int LK>
__device__ __forceinline__ void rescore_finish(double (&dd)[LK], int (&jj)[LK], const float (&lst)[LK],
                                               double xsq, int ibits, int k, int ncand, float rmax2,
                                               uint16_t *__restrict__ out, uint64_t fentry,
                                               uint64_t *__restrict__ flist,
                                               uint32_t *__restrict__ fcount);

template <int D, int LK, int CU = 1>
__device__ void rescore_lane(const bf16_t *__restrict__ xrow, const bf16_t *__restrict__ urefs,
                             const float (&lst)[LK], uint32_t imask, int ibits, int k, int ncand,
                             float rmax2, bool write, uint16_t *__restrict__ out,
                             uint64_t fentry, uint64_t *__restrict__ flist,
                             uint32_t *__restrict__ fcount) {
#pragma clang fp contract(off)
    int jj[LK];
    bool cv[LK];
#pragma unroll
    for (int e = 0; e < LK; ++e) {
        cv[e] = lst[e] != -INFINITY;
        jj[e] = cv[e] ? unpack_ordinal(lst[e], imask) : 0;
    }
    double dd[LK];
#pragma unroll
    for (int e = 0; e < LK; ++e) dd[e] = 0.0;
    double xsq = 0.0;
#pragma unroll CU
    for (int c = 0; c < D / 8; ++c) {
        const u32x4 xv = ld16(xrow + 8 * c);
        double xd[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xd[2 * i] = (double)__uint_as_float(xv[i] << 16);
            xd[2 * i + 1] = (double)__uint_as_float(xv[i] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double sq = xd[i] * xd[i];
            xsq = xsq + sq;
        }
#pragma unroll
        for (int e = 0; e < LK; ++e) {
            const u32x4 rv = ld16(at_byte(urefs, ((uint32_t)jj[e] * D + 8u * c) * 2u));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double r0 = (double)__uint_as_float(rv[i] << 16);
                const double r1 = (double)__uint_as_float(rv[i] & 0xffff0000u);
                const double d0 = xd[2 * i] - r0;
                const double s0 = d0 * d0;
                dd[e] = dd[e] + s0;
                const double d1 = xd[2 * i + 1] - r1;
                const double s1 = d1 * d1;
                dd[e] = dd[e] + s1;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < LK; ++e) {
        dd[e] = cv[e] ? dd[e] : __builtin_inf();
        jj[e] = cv[e] ? jj[e] : INT_MAX;
    }
    if (!write) return;
    rescore_finish<D, LK>(dd, jj, lst, xsq, ibits, k, ncand, rmax2, out, fentry, flist, fcount);
}

// Sort of a token's exact candidate distances by (distance, ordinal)
// (unused candidates: +inf, INT_MAX), certificate, and the result or a
// fallback entry.
template <int D, int LK>
__device__ __forceinline__ void rescore_finish(double (&dd)[LK], int (&jj)[LK], const float (&lst)[LK],
                                               double xsq, int ibits, int k, int ncand, float rmax2,
                                               uint16_t *__restrict__ out, uint64_t fentry,
                                               uint64_t *__restrict__ flist,
                                               uint32_t *__restrict__ fcount) {
    // sort by (distance, ordinal): odd-even transposition network
#pragma unroll
    for (int pass = 0; pass < LK; ++pass) {
#pragma unroll
        for (int i = pass & 1; i + 1 < LK; i += 2) {
            const bool sw = (dd[i + 1] < dd[i]) | ((dd[i + 1] == dd[i]) & (jj[i + 1] < jj[i]));
            const double td = dd[i];
            const int tj = jj[i];
            dd[i] = sw ? dd[i + 1] : dd[i];
            jj[i] = sw ? jj[i + 1] : jj[i];
            dd[i + 1] = sw ? td : dd[i + 1];
            jj[i + 1] = sw ? tj : jj[i + 1];
        }
    }
    const bool full = lst[LK - 1] != -INFINITY;
    int nvalid = 0;
#pragma unroll
    for (int e = 0; e < LK; ++e) nvalid += jj[e] != INT_MAX;
    const int kk = min(k, nvalid);
    // the fp32 norms behind the approximate values must be finite (else a
    // reference may have dropped out of the list unseen)
    bool ok = xsq <= 3.0e38 && rmax2 <= 3.0e38f;
    if (full) {
        const double rm = sqrt((double)rmax2 * (1.0 + 1e-6));
        const double xn = sqrt(xsq) * (1.0 + 1e-12);
        double dk_ = dd[0];
#pragma unroll
        for (int e = 1; e < LK; ++e) dk_ = (e == kk - 1) ? dd[e] : dk_;
        ok = ok && excluded_lower_bound<D>(lst[LK - 1], ibits, xn, rm) > dk_;
    } else {
        ok = ok && nvalid == ncand;
    }
    if (ok) {
        store_idx<LK>(out, jj, k, kk);
    } else {
        const uint32_t slot = atomicAdd(fcount, 1u);
        flist[slot] = fentry;
    }
}

template <int D, int LK>
__global__ __launch_bounds__(256, 3) void dist_topk_kernel(
    const bf16_t *__restrict__ x, int64_t t0, int64_t nrows, int s, int k,
    const bf16_t *__restrict__ refs, const float *__restrict__ sqn, int64_t Rcap, int64_t Ncap,
    int64_t q0, int64_t nq, int U, int ntiles, uint32_t imask, int ibits,
    uint16_t *__restrict__ idx, uint64_t *__restrict__ flist, uint32_t *__restrict__ fcount,
    int nsplit, int chunk, float *__restrict__ lists, float *__restrict__ rmaxs) {
    constexpr int KSTEPS = D / 16;
    constexpr int CH = D / 8;
    constexpr int RB = 64;
    constexpr int DMA_IT = RB * CH / 256;
    // LDS chunk swizzle of reference row r (bank = 4 chunk + 32 (r % 2) for
    // 128-byte rows, 4 chunk for 256-byte rows)
    auto swz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    // reference tiles of two stages: two objects, so the compiler can tell
    // the DMA fill of one from the reads of the other (one array would make
    // every read wait for the fill just issued)
    __shared__ __attribute__((aligned(16))) bf16_t rtA[RB][D];
    __shared__ __attribute__((aligned(16))) bf16_t rtB[RB][D];
    __shared__ __attribute__((aligned(16))) float nsA[RB];
    __shared__ __attribute__((aligned(16))) float nsB[RB];
    __shared__ float red[4];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int unit = blockIdx.x % U;
    // heaviest tiles first; split sp of the tile's reference range
    const int rest = (int)(blockIdx.x / U);
    const int sp = rest % nsplit;
    const int tile = ntiles - 1 - rest / nsplit;
    const int64_t qb = q0 + (int64_t)tile * 256;
    const int64_t qend = q0 + nq;
    const bf16_t *urefs = refs + (int64_t)unit * Rcap * D;
    const float *usqn = sqn + (int64_t)unit * Rcap;

    const int64_t qlast = min(qb + 255, qend - 1);
    // reference counts stay below 2^16: 32-bit arithmetic in the loop
    const int ncand_max = (int)((tok_pos(qlast, s) + s - 1) / s);
    // this block's references [jbeg, jend) (the whole range unless split)
    const int jbeg = sp * chunk;
    const int jend = min(ncand_max, jbeg + chunk);

    // MFMA column operands: the wave's two N-tiles of 32 tokens, times -2
    // (exact: a power of two; an overflow to infinity makes the fp32 norm
    // infinite too, which the certificate rejects), and the fp32 norm of
    // each token from the same products (lane and lane ^ 32 hold the two
    // halves of a row)
    bf16x8 xb[2][KSTEPS];
    float xnorm[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int64_t qq = min(qb + 64 * w + 32 * nt + l32, qend - 1);
        const bf16_t *xr = x + ((int64_t)unit * nrows + (tok_pos(qq, s) - t0)) * D;
        float part[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) part[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const u32x4 v = ld16(xr + 16 * ks + 8 * hl);
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xffff0000u);
                part[2 * i] += lo * lo;
                part[2 * i + 1] += hi * hi;
                o[i] = (__float_as_uint(-2.f * lo) >> 16) | (__float_as_uint(-2.f * hi) & 0xffff0000u);
            }
            xb[nt][ks] = as_bf16x8(o);
        }
        const float half_sq = ((part[0] + part[1]) + (part[2] + part[3])) +
                              ((part[4] + part[5]) + (part[6] + part[7]));
        xnorm[nt] = half_sq + __shfl_xor(half_sq, 32, 64);
    }
    // extra K step (32x32x8: k 0-3 in the lower lane half): the token norm as
    // hi + mid + lo (bf16 pieces cut from the fp32 value, so their sum is
    // that value exactly) against ones
    s16x4 xext[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const uint32_t hb = __float_as_uint(xnorm[nt]) & 0xffff0000u;
        const float r1 = xnorm[nt] - __uint_as_float(hb);
        const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
        const uint32_t lb = __float_as_uint(r1 - __uint_as_float(mb));
        u32x2 e;
        e[0] = hl ? 0u : ((hb >> 16) | mb);
        e[1] = hl ? 0u : (lb >> 16);
        xext[nt] = __builtin_bit_cast(s16x4, e);
    }
    u32x2 ones_w;
    ones_w[0] = 0x3f803f80u;
    ones_w[1] = 0x00003f80u;
    const s16x4 ones = __builtin_bit_cast(s16x4, ones_w);
    // after the half swap below, lane L holds all 32 values of token
    // qb + 64 w + L: one candidate list per lane
    const int64_t qq = qb + 64 * w + lane;
    const bool valid = qq < qend;
    const int64_t qn = min(qq, qend - 1);
    const int64_t pos = tok_pos(qn, s);
    const int ncand = (int)((pos + s - 1) / s);
    const int ncand_lo =
        (int)((tok_pos(min(qb + 64 * w, qend - 1), s) + s - 1) / s);  // the wave's first token
    float lst[LK];
#pragma unroll
    for (int e = 0; e < LK; ++e) lst[e] = -INFINITY;
    // in a vector register, so a packing is one v_and_or_b32 with the
    // (scalar) code as its other operand
    uint32_t nmask = ~imask;
    asm volatile("" : "+v"(nmask));

    // largest fp32 reference norm among the rows the block reads (bounds the
    // error of S for every reference it excludes)
    float rmax2 = 0.f;
    // one stage's reference rows and their norms, all by DMA (no register
    // results, so nothing waits for them before the stage's barrier)
    // a DMA pass of the block moves 256 16-byte chunks = 256 / CH rows;
    // the thread's row within a pass and its (swizzled) chunk are the same
    // in every pass (the swizzle depends on row % 16 or (row / 2) % 8 only)
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int dma_row = tid / CH;
    const uint32_t dma_col = 16u * (uint32_t)((tid % CH) ^ swz(dma_row));
    auto stage_load = [&](int jbase, bf16_t (*dst)[D], float *ndst) {
#pragma unroll
        for (int m = 0; m < DMA_IT; ++m) {
            const uint32_t j = (uint32_t)min(jbase + (256 / CH) * m + dma_row, jend - 1);
            __builtin_amdgcn_global_load_lds(
                (const void *)at_byte(urefs, j * (2u * D) + dma_col),
                (__attribute__((address_space(3))) void *)&dst[(256 * m + 64 * wu) / CH][0], 16,
                0, 0);
        }
        if (wu == 0) {
            const uint32_t j = (uint32_t)min(jbase + lane, jend - 1);
            __builtin_amdgcn_global_load_lds((const void *)(usqn + j),
                                             (__attribute__((address_space(3))) void *)ndst, 4,
                                             0, 0);
        }
    };
    const int nstage = jend > jbeg ? (jend - jbeg + RB - 1) / RB : 0;
    if (nstage > 0) {
        stage_load(jbeg, rtA, nsA);
        wait_vm_all();
        __syncthreads();
    }

    // one stage: 64 references from cur (norms ncur) while the next stage is
    // gathered into nxt (nnxt)
    auto stage = [&](int st, bf16_t (*cur)[D], const float *ncur, bf16_t (*nxt)[D], float *nnxt) {
        const int jst = jbeg + st * RB;
        const bool more = st + 1 < nstage;
        if (more) stage_load(jst + RB, nxt, nnxt);
        rmax2 = fmaxf(rmax2, ncur[lane]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int j0 = jst + 32 * mb;
            if (j0 >= jend) break;
            const uint32_t cbase = imask - (uint32_t)j0;
            f32x16 init;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&ncur[32 * mb + 8 * g4 + 4 * hl]);
#pragma unroll
                for (int i = 0; i < 4; ++i) init[4 * g4 + i] = v[i];
            }
            f32x16 acc0 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ones, xext[0], init, 0, 0, 0);
            f32x16 acc1 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ones, xext[1], init, 0, 0, 0);
            const int r = 32 * mb + l32;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const int pc = (2 * ks + hl) ^ swz(r);
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(&cur[r][8 * pc]));
                acc0 = mfma32_bf16(a, xb[0][ks], acc0);
                acc1 = mfma32_bf16(a, xb[1][ks], acc1);
            }
            // swap the upper half of acc0 with the lower half of acc1: lane L
            // then holds rows 8 (i / 4) + (i % 4) (acc0) and + 4 (acc1) of
            // token qb + 64 w + L
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[i]),
                                                                 __float_as_uint(acc1[i]), false,
                                                                 false);
                acc0[i] = __uint_as_float(sw[0]);
                acc1[i] = __uint_as_float(sw[1]);
            }
            if (j0 + 32 > ncand_lo) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = j0 + 8 * (i / 4) + (i % 4);
                    acc0[i] = j < ncand ? acc0[i] : INFINITY;
                    acc1[i] = j + 4 < ncand ? acc1[i] : INFINITY;
                }
            }
            // slots in pairs: one wave-wide test per pair, then each slot's
            // insertion under the mask of the lanes it passes in (a second
            // slot that no longer beats the list after the first went in
            // leaves the list unchanged)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float thr = lst[LK - 1];
                const bool p0 = -acc0[i] > thr, p1 = -acc1[i] > thr;
                if (__builtin_amdgcn_ballot_w64(p0 || p1)) {
                    const uint32_t code = cbase - (uint32_t)(8 * (i / 4) + (i % 4));
                    if (p0) list_insert_neg<LK>(lst, pack_score(acc0[i], code, nmask));
                    if (p1) list_insert_neg<LK>(lst, pack_score(acc1[i], code - 4u, nmask));
                }
            }
        }
        wait_vm_all();
        __syncthreads();
    };
    for (int st = 0; st < nstage; st += 2) {
        stage(st, rtA, nsA, rtB, nsB);
        if (st + 1 < nstage) stage(st + 1, rtB, nsB, rtA, nsA);
    }
    rmax2 = wave_max(rmax2);
    if (lane == 0) red[w] = rmax2;
    __syncthreads();
    rmax2 = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    if (nsplit > 1) {
        // a split of the reference range: its lists and largest norm go to
        // the workspace; the merge kernel rescores
        if (valid) {
            float *dst = lists + (((int64_t)sp * U + unit) * nq + (qq - q0)) * LK;
#pragma unroll
            for (int e = 0; e < LK; ++e) dst[e] = lst[e];
        }
        if (tid == 0) rmaxs[((int64_t)sp * U + unit) * ntiles + tile] = rmax2;
        return;
    }

    const bf16_t *xr = x + ((int64_t)unit * nrows + (pos - t0)) * D;
    uint16_t *out = idx + ((int64_t)unit * Ncap + qn) * k;
    // First pass of the rescore, in fp32: d'_e = |r_e|^2 - 2 x.r_e (the
    // distance minus |x|^2, which every candidate of the token shares) from
    // bf16 dot products with the -2 x operand (the products are exact; eight
    // partial sums per dot product) with a rigorous bound on the error of
    // each d'_e.  When the
    // bounds order the candidates the result needs (the first min(k, n)
    // positions and the one after them) and the certificate holds with the
    // k-th candidate's upper bound, the result is written from this pass and
    // true is returned; false sends the lane to the exact fp64 rescore.  Each
    // dot-product step's rounding is bounded by 2^-23 relative
    // (round-to-nearest or toward zero).
    //
    // The token's row is the lane's MFMA operand, made whole by the half
    // swap; the candidate rows are gathered through this wave's quarter of
    // the (now idle) reference-tile buffer: a round brings one 128-byte half
    // row of candidate e for LPR lanes' tokens, 8 lanes per half row
    // (coalesced), slots XOR-swizzled so that each lane then reads its own
    // half row without bank conflicts.
    auto rescore_fast = [&](const bf16_t *xrow_unused, uint16_t *o) -> bool {
        (void)xrow_unused;
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        constexpr int NA = 8;             // partial sums per dot product
        constexpr int LPR = D / 2;        // lanes per round
        constexpr int NDM = LPR / 8;      // gather instructions per round
        constexpr int HR = D / 64;        // half rows per row
        constexpr int NG = 64 / LPR;      // lane groups
        u32x4 xs0[KSTEPS], xs1[KSTEPS];   // chunk c: xs0[c / 2] (even), xs1[c / 2] (odd)
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const u32x4 a = __builtin_bit_cast(u32x4, xb[0][ks]);
            const u32x4 b = __builtin_bit_cast(u32x4, xb[1][ks]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t aq = a[q], bq = b[q];
                const auto sw = __builtin_amdgcn_permlane32_swap(aq, bq, false, false);
                xs0[ks][q] = sw[0];
                xs1[ks][q] = sw[1];
            }
        }
        auto xw = [&](int c, int i) -> uint32_t {
            const uint32_t v = (c & 1) ? xs1[c >> 1][i] : xs0[c >> 1][i];
            return v;
        };
        auto dot = [](uint32_t a, uint32_t b, float acc) {
            return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                                   __builtin_bit_cast(bf16x2_t, b), acc, false);
        };
        auto tree = [](const float (&v)[NA]) {
            return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        };
        int jj[LK];
        bool cv[LK];
#pragma unroll
        for (int e = 0; e < LK; ++e) {
            cv[e] = lst[e] != -INFINITY;
            jj[e] = cv[e] ? unpack_ordinal(lst[e], imask) : 0;
        }
        float xa[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) xa[a] = 0.f;
#pragma unroll
        for (int c = 0; c < 2 * KSTEPS; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[4 * (c & 1) + i] = dot(xw(c, i), xw(c, i), xa[4 * (c & 1) + i]);
        const float xsq = 0.25f * tree(xa);  // the operand is -2 x
        // error of a partial-sum dot product of D terms over NA sums: at most
        // D / NA + 3 roundings on any path, each within 2^-23 of the running
        // sum, hence <= g * sum |terms|
        constexpr float u = 1.1920929e-07f;  // 2^-23
        constexpr float g = (float)(D / NA + 4) * u * 1.01f;
        const float xsq_hi = xsq * (1.f + 4.f * g);
        char *wst = reinterpret_cast<char *>(w < 2 ? &rtA[0][0] : &rtB[0][0]) + (w & 1) * (64 * D);
        float dp[LK], er[LK];
#pragma unroll
        for (int e = 0; e < LK; ++e) {
            dp[e] = INFINITY;
            er[e] = 0.f;
        }
        // one candidate at a time (a run-time loop: the registers of one
        // candidate's rounds only)
#pragma unroll 1
        for (int e = 0; e < LK; ++e) {
            int je = jj[0];
            bool ce = cv[0];
#pragma unroll
            for (int q = 1; q < LK; ++q) {
                je = q == e ? jj[q] : je;
                ce = q == e ? cv[q] : ce;
            }
            float ra[NA];
#pragma unroll
            for (int a = 0; a < NA; ++a) ra[a] = 0.f;
#pragma unroll
            for (int hh = 0; hh < HR; ++hh) {
#pragma unroll
                for (int gq = 0; gq < NG; ++gq) {
                    // the previous round's reads are done before its slots
                    // are filled again
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
                    for (int m = 0; m < NDM; ++m) {
                        const int tl = 8 * m + (lane >> 3);
                        const int src = __shfl(je, gq * LPR + tl);
                        const int cc = (lane & 7) ^ ((tl >> 1) & 7);
                        __builtin_amdgcn_global_load_lds(
                            (const void *)at_byte(urefs, ((uint32_t)src * D + 64u * hh + 8u * cc) * 2u),
                            (__attribute__((address_space(3))) void *)(wst + 1024 * m), 16, 0, 0);
                    }
                    wait_vm_all();
                    if (NG == 1 || lane / LPR == gq) {
                        const int tl = lane - gq * LPR;
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc) {
                            const int pp = cc ^ ((tl >> 1) & 7);
                            const u32x4 rv = *reinterpret_cast<const u32x4 *>(wst + 128 * tl + 16 * pp);
                            const int c = 8 * hh + cc;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const uint32_t rw = rv[i];
                                ra[4 * (c & 1) + i] = dot(xw(c, i), rw, ra[4 * (c & 1) + i]);
                            }
                        }
                    }
                }
            }
            const float rsq = usqn[je];  // fp32 norm: within 8 u rsq
            const float xr2 = tree(ra);    // ~ -2 x.r
            // |xr2 + 2 x.r| <= 2 g |x||r| <= g (|x|^2 + |r|^2); evaluating
            // rsq + xr2 adds <= u (rsq + |xr2|); a denormal product flushed
            // to zero is within 2^-125 max(|x|, |r|) each
            const float dpe = ce ? rsq + xr2 : INFINITY;
            const float ere = ce ? 8.f * u * rsq + g * (xsq_hi + rsq) + u * (rsq + fabsf(xr2)) +
                                       1e-30f * (1.f + xsq_hi + rsq)
                                 : 0.f;
#pragma unroll
            for (int q = 0; q < LK; ++q) {
                dp[q] = q == e ? dpe : dp[q];
                er[q] = q == e ? ere : er[q];
            }
        }
        if (!valid) return true;
        // sort by d' (ordinals break exact ties; a tie cannot be certified)
#pragma unroll
        for (int pass = 0; pass < LK; ++pass) {
#pragma unroll
            for (int i = pass & 1; i + 1 < LK; i += 2) {
                const bool sw = (dp[i + 1] < dp[i]) | ((dp[i + 1] == dp[i]) & (jj[i + 1] < jj[i]));
                const float td = dp[i], te = er[i];
                const int tj = jj[i];
                dp[i] = sw ? dp[i + 1] : dp[i];
                er[i] = sw ? er[i + 1] : er[i];
                jj[i] = sw ? jj[i + 1] : jj[i];
                dp[i + 1] = sw ? td : dp[i + 1];
                er[i + 1] = sw ? te : er[i + 1];
                jj[i + 1] = sw ? tj : jj[i + 1];
            }
        }
        int nvalid = 0;
#pragma unroll
        for (int e = 0; e < LK; ++e) nvalid += cv[e] ? 1 : 0;
        const int kk = min(k, nvalid);
        // a certified gap must also clear the fp64 rounding of the exact values
        const float slack = 1e-9f * (xsq_hi + rmax2);
        bool ok = xsq_hi <= 3.0e38f && rmax2 <= 3.0e38f;
#pragma unroll
        for (int i = 0; i + 1 < LK; ++i)
            if (i < kk && i + 1 < nvalid) ok = ok && (dp[i + 1] - er[i + 1]) - (dp[i] + er[i]) > slack;
        if (lst[LK - 1] != -INFINITY) {
            // certificate: an excluded reference is at distance >= lb; the
            // k-th candidate at most dp + er + |x|^2
            const double rm = sqrt((double)rmax2 * (1.0 + 1e-6));
            const double xn = sqrt((double)xsq_hi);
            double dk_ = (double)dp[0] + (double)er[0];
#pragma unroll
            for (int e = 1; e < LK; ++e) dk_ = (e == kk - 1) ? (double)dp[e] + (double)er[e] : dk_;
            ok = ok && excluded_lower_bound<D>(lst[LK - 1], ibits, xn, rm) > dk_ + (double)xsq_hi;
        } else {
            ok = ok && nvalid == ncand;
        }
        if (!ok) return false;
        store_idx<LK>(o, jj, k, kk);
        return true;
    };

    // fp32 pass with error bounds (lists of up to 8: its partial sums for
    // longer ones would not fit the registers); the lanes it cannot settle
    // take the exact fp64 rescore
    bool settled = false;
    if constexpr (LK <= 8) settled = rescore_fast(xr, out);
    if (!settled)
        rescore_lane<D, LK>(xr, urefs, lst, imask, ibits, k, ncand, rmax2, valid, out,
                            ((uint64_t)unit << 32) | (uint64_t)(qn - q0), flist, fcount);
}

// Merge of the split top-k searches: per token, the LK best of the splits'
// lists (each split excluded only references below its own last entry, which
// is at most the merged last entry, so the certificate holds with it), then
// the exact fp64 rescore and certificate.  Four lanes per token: each merges
// the lists, computes the exact distances of every fourth candidate (the
// whole row requested at once) and the token norm, the distances are shared
// within the four lanes, and the first lane sorts, certifies and writes.
template <int D, int LK>
__global__ __launch_bounds__(256) void topk_merge_kernel(
    const bf16_t *__restrict__ x, int64_t t0, int64_t nrows, int s, int k,
    const bf16_t *__restrict__ refs, int64_t Rcap, int64_t Ncap, int64_t q0, int64_t nq, int U,
    int nsplit, uint32_t imask, int ibits, const float *__restrict__ lists,
    const float *__restrict__ rmaxs, int ntiles, uint16_t *__restrict__ idx,
    uint64_t *__restrict__ flist, uint32_t *__restrict__ fcount) {
#pragma clang fp contract(off)
    constexpr int NE = (LK + 3) / 4;  // candidates per lane
    const int lane = threadIdx.x & 63, sub = lane & 3;
    const int64_t gid = (int64_t)blockIdx.x * 64 + threadIdx.x / 4;
    // the four lanes of a token share gid, so they leave together
    if (gid >= (int64_t)U * nq) return;
    const int unit = (int)(gid / nq);
    const int64_t qi = gid % nq;
    float lst[LK];
#pragma unroll
    for (int e = 0; e < LK; ++e) lst[e] = -INFINITY;
    float rmax2 = 0.f;
    const int tile = (int)(qi / 256);
    // four splits' lists requested at a time, then merged
    for (int sp0 = 0; sp0 < nsplit; sp0 += 4) {
        float v[4][LK];
        float rm[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sp = min(sp0 + u, nsplit - 1);  // a repeated list merges to no change
            const float *src = lists + (((int64_t)sp * U + unit) * nq + qi) * LK;
#pragma unroll
            for (int e = 0; e < LK; ++e) v[u][e] = src[e];
            rm[u] = rmaxs[((int64_t)sp * U + unit) * ntiles + tile];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (sp0 + u < nsplit) {
#pragma unroll
                for (int e = 0; e < LK; ++e) list_insert<LK>(lst, v[u][e]);
                rmax2 = fmaxf(rmax2, rm[u]);
            }
        }
    }
    const int64_t q = q0 + qi;
    const bf16_t *xr = x + ((int64_t)unit * nrows + (tok_pos(q, s) - t0)) * D;
    const bf16_t *urefs = refs + (int64_t)unit * Rcap * D;
    const int ncand = (int)((tok_pos(q, s) + s - 1) / s);
    int jj[LK];
    bool cv[LK];
#pragma unroll
    for (int e = 0; e < LK; ++e) {
        cv[e] = lst[e] != -INFINITY;
        jj[e] = cv[e] ? unpack_ordinal(lst[e], imask) : 0;
    }
    // the token row in fp64-ready form and its norm (coordinate order)
    u32x4 xv[D / 8];
#pragma unroll
    for (int c = 0; c < D / 8; ++c) xv[c] = ld16(xr + 8 * c);
    double xsq = 0.0;
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double a0 = (double)__uint_as_float(xv[c][i] << 16);
            const double a1 = (double)__uint_as_float(xv[c][i] & 0xffff0000u);
            const double s0 = a0 * a0;
            xsq = xsq + s0;
            const double s1 = a1 * a1;
            xsq = xsq + s1;
        }
    // this lane's candidates sub, sub + 4, ...: each row requested whole
    double mine[NE];
#pragma unroll
    for (int u = 0; u < NE; ++u) mine[u] = 0.0;
#pragma unroll 1
    for (int u = 0; u < NE; ++u) {
        const int e = sub + 4 * u;
        int je = jj[0];
#pragma unroll
        for (int q2 = 1; q2 < LK; ++q2) je = q2 == e ? jj[q2] : je;
        u32x4 rv[D / 8];
#pragma unroll
        for (int c = 0; c < D / 8; ++c) rv[c] = ld16(at_byte(urefs, ((uint32_t)je * D + 8u * c) * 2u));
        // (the token row's fp64 conversions stay in the loop: hoisted, they
        // would take 2 D registers)
#pragma unroll
        for (int c = 0; c < D / 8; ++c) asm volatile("" : "+v"(xv[c]));
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < D / 8; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double d0 = (double)__uint_as_float(xv[c][i] << 16) -
                                  (double)__uint_as_float(rv[c][i] << 16);
                const double s0 = d0 * d0;
                acc = acc + s0;
                const double d1 = (double)__uint_as_float(xv[c][i] & 0xffff0000u) -
                                  (double)__uint_as_float(rv[c][i] & 0xffff0000u);
                const double s1 = d1 * d1;
                acc = acc + s1;
            }
#pragma unroll
        for (int u2 = 0; u2 < NE; ++u2) mine[u2] = u2 == u ? acc : mine[u2];
    }
    // gather the distances of all candidates (candidate e from lane e % 4)
    double dd[LK];
    const int gbase = lane & ~3;
#pragma unroll
    for (int e = 0; e < LK; ++e) {
        const double d = __shfl(mine[e / 4], gbase + (e % 4), 64);
        dd[e] = cv[e] ? d : __builtin_inf();
        jj[e] = cv[e] ? jj[e] : INT_MAX;
    }
    if (sub == 0)
        rescore_finish<D, LK>(dd, jj, lst, xsq, ibits, k, ncand, rmax2,
                              idx + ((int64_t)unit * Ncap + q) * k,
                              ((uint64_t)unit << 32) | (uint64_t)qi, flist, fcount);
}


template <int D, int LK>
void launch_topk_t(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0, int64_t nq,
                   const CacheArgs &c, uint64_t *flist, uint32_t *fcount, void *tail,
                   hipStream_t st) {
    const int U = dm.B * dm.H;
    const int ntiles = (int)((nq + 255) / 256);
    // ordinal bits of the packed scores: enough for the references this call
    // can see (those before t1), not for the cache's capacity, so that a
    // chunk early in a prompt keeps more of each score's mantissa and fewer
    // of its tokens fail the certificate
    int ibits = 1;
    while (((int64_t)1 << ibits) < refs_upto(t1, dm.s)) ++ibits;
    const uint32_t imask = (1u << ibits) - 1u;
    int nsplit, chunk;
    topk_split_plan(dm, t1, nq, &nsplit, &chunk);
    float *lists = nullptr, *rmaxs = nullptr;
    if (nsplit > 1) {
        lists = (float *)tail;
        rmaxs = (float *)((char *)tail + align256((size_t)nsplit * U * nq * LK * sizeof(float)));
    }
    hipLaunchKernelGGL((dist_topk_kernel<D, LK>), dim3((unsigned)(ntiles * U * nsplit)), dim3(256),
                       0, st, (const bf16_t *)x, t0, t1 - t0, dm.s, dm.k, (const bf16_t *)c.refs,
                       c.sqn, dm.R, dm.N, q0, nq, U, ntiles, imask, ibits, c.idx, flist, fcount,
                       nsplit, chunk, lists, rmaxs);
    if (nsplit > 1)
        hipLaunchKernelGGL((topk_merge_kernel<D, LK>), dim3((unsigned)((U * nq + 63) / 64)),
                           dim3(256), 0, st, (const bf16_t *)x, t0, t1 - t0, dm.s, dm.k,
                           (const bf16_t *)c.refs, dm.R, dm.N, q0, nq, U, nsplit, imask, ibits,
                           lists, rmaxs, ntiles, c.idx, flist, fcount);
}

}  // namespace

size_t select_split_ws_bytes(const Dims &dm, int64_t t0, int64_t t1) {
    const int64_t nq = toks_upto(t1, dm.s) - toks_upto(t0, dm.s);
    if (nq <= 0 || nq > kSmallRange) return 0;
    // split_plan's chunk is at least 256 and at least rmax / kSplitMax
    const int64_t rmax = std::max<int64_t>(1, refs_upto(t1, dm.s));
    const int64_t nsplit = std::min<int64_t>((rmax + 255) / 256, kSplitMax);
    const size_t n = (size_t)dm.B * dm.H * nq * nsplit * kMaxK;
    return n * sizeof(double) + n * sizeof(int) + 256;
}

// Splits of a batched append: enough blocks to fill the GPU (about 4096 over
// the set), whole 256-reference chunks.
static int64_t append_split_bound(const Dims &dm, int64_t t, int n) {
    const int64_t R = std::max<int64_t>(1, refs_upto(t, dm.s));
    const int64_t items = std::max<int64_t>(1, (int64_t)n * dm.B * dm.H);
    return std::max<int64_t>(1, std::min<int64_t>((4096 + items - 1) / items, (R + 255) / 256));
}

static void append_split_plan(const Dims &dm, int64_t t, int n, int *chunk, int *nsplit) {
    const int64_t R = std::max<int64_t>(1, refs_upto(t, dm.s));
    const int64_t ns = append_split_bound(dm, t, n);
    int64_t c = (R + ns - 1) / ns;
    c = (c + 63) / 64 * 64;
    *chunk = (int)c;
    *nsplit = (int)((R + c - 1) / c);   // <= ns
}

size_t append_select_ws_bytes(const Dims &dm, int64_t t, int n) {
    const size_t m = (size_t)n * dm.B * dm.H * append_split_bound(dm, t, n) * kMaxK;
    return m * sizeof(double) + m * sizeof(int) + 256;
}

hipError_t launch_append_select(const Dims &dm, int64_t t, int n, const AppendSet &set, void *ws,
                                hipStream_t st) {
    int chunk, nsplit;
    append_split_plan(dm, t, n, &chunk, &nsplit);
    const int U = dm.B * dm.H;
    const size_t m = (size_t)n * U * nsplit * kMaxK;
    double *pd = (double *)ws;
    int *pj = (int *)((char *)ws + m * sizeof(double));
    const dim3 grid((unsigned)nsplit, (unsigned)U, (unsigned)n);
    const PageMap pg = set_pages(dm);
    if (dm.d == 128)
        hipLaunchKernelGGL(append_split_kernel<128>, grid, dim3(256), 0, st, set, t, dm.s, dm.R,
                           chunk, pd, pj, pg);
    else
        hipLaunchKernelGGL(append_split_kernel<64>, grid, dim3(256), 0, st, set, t, dm.s, dm.R,
                           chunk, pd, pj, pg);
    const int64_t q = t - refs_upto(t + 1, dm.s);   // token ordinal of position t
    hipLaunchKernelGGL(append_merge_kernel, dim3((unsigned)U, (unsigned)n), dim3(64), 0, st, set,
                       nsplit, dm.k, q, dm.N, pd, pj, pg);
    return hipGetLastError();
}

hipError_t launch_select_split(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                               int64_t nq, const CacheArgs &c, void *ws, hipStream_t st) {
    int chunk, nsplit;
    split_plan(dm, t1, &chunk, &nsplit);
    const int64_t items = (int64_t)dm.B * dm.H * nq;
    double *pd = (double *)ws;
    int *pj = (int *)((char *)ws + (size_t)items * nsplit * kMaxK * sizeof(double));
    dim3 grid((unsigned)nsplit, (unsigned)items);
    if (dm.d == 128)
        hipLaunchKernelGGL((select_split_kernel<bf16_t, 128>), grid, dim3(256), 0, st,
                           (const bf16_t *)x, t0, t1 - t0, dm.s, (const bf16_t *)c.refs, dm.R,
                           q0, nq, chunk, pd, pj);
    else
        hipLaunchKernelGGL((select_split_kernel<bf16_t, 64>), grid, dim3(256), 0, st,
                           (const bf16_t *)x, t0, t1 - t0, dm.s, (const bf16_t *)c.refs, dm.R,
                           q0, nq, chunk, pd, pj);
    hipLaunchKernelGGL(select_merge_kernel, dim3((unsigned)items), dim3(64), 0, st, nsplit, dm.k,
                       q0, nq, dm.N, pd, pj, c.idx);
    return hipGetLastError();
}

hipError_t launch_select_exact(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                               int64_t q0, int64_t nq, const CacheArgs &c,
                               const uint64_t *list, const uint32_t *list_count,
                               int64_t list_cap, void *scratch, size_t scratch_bytes,
                               hipStream_t st, uint32_t *stats) {
    if (dm.dtype == 0)
        return dm.d == 64 ? launch_exact_t<float, 64>(dm, x, t0, t1, q0, nq, c, list, list_count,
                                                      list_cap, scratch, scratch_bytes, stats, st)
                          : launch_exact_t<float, 128>(dm, x, t0, t1, q0, nq, c, list, list_count,
                                                       list_cap, scratch, scratch_bytes, stats, st);
    return dm.d == 64 ? launch_exact_t<bf16_t, 64>(dm, x, t0, t1, q0, nq, c, list, list_count,
                                                   list_cap, scratch, scratch_bytes, stats, st)
                      : launch_exact_t<bf16_t, 128>(dm, x, t0, t1, q0, nq, c, list, list_count,
                                                    list_cap, scratch, scratch_bytes, stats, st);
}

}  // namespace dk

namespace dk {

// Matrix-core candidate search with certificate; tokens it cannot certify are
// appended to `flist` and rescanned exactly.  fcount must point to a device
// counter; it is cleared here.
hipError_t launch_select_mfma(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                              int64_t nq, const CacheArgs &c, uint64_t *flist, uint32_t *fcount,
                              uint32_t *stats, hipStream_t st) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, fcount);
    // split lists after the fallback list (one entry per unit and token)
    void *tail = (char *)flist + align256((size_t)nq * dm.B * dm.H * sizeof(uint64_t));
    if (dm.d == 128) {
        if (dm.k <= 4) launch_topk_t<128, kListLen4>(dm, x, t0, t1, q0, nq, c, flist, fcount, tail, st);
        else launch_topk_t<128, kListLen8>(dm, x, t0, t1, q0, nq, c, flist, fcount, tail, st);
    } else {
        if (dm.k <= 4) launch_topk_t<64, kListLen4>(dm, x, t0, t1, q0, nq, c, flist, fcount, tail, st);
        else launch_topk_t<64, kListLen8>(dm, x, t0, t1, q0, nq, c, flist, fcount, tail, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the split lists of the search are consumed: their space holds the
    // partial lists of the split exact scan
    e = launch_select_exact(dm, x, t0, t1, q0, nq, c, flist, fcount, (int64_t)nq * dm.B * dm.H,
                            tail, exact_list_ws_bytes(dm, t1, (int64_t)nq * dm.B * dm.H), st,
                            stats);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace dk
