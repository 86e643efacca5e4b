// dk_launch.h -- host-side launchers of libdeltakv's kernels.  Every launcher
// enqueues on `stream` and returns hipSuccess or the launch error.  Arguments
// have been validated by the C ABI layer (api.cpp) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dk_common.h"

namespace dk {

// Sizes of one (layer, stream) cache, derived from deltakv_shape.
struct Dims {
    int B, H, d, s, k, dc;
    int dtype;          // 0 fp32, 1 bf16
    int lat_fmt;        // 0: latents in dtype, 1: 4-bit codes + per-row bf16 shift / scale
    int64_t cap;        // capacity (positions)
    int64_t R;          // reference rows per unit = ceil(cap / s)
    int64_t N;          // compressed-token rows per unit = cap - R
    int pr = 0;         // paged layout: reference rows per page (0: unit-contiguous arrays)
};

struct MlpArgs {
    const void *w1;
    const float *b1;
    const void *w2;
    const float *b2;
    int in_dim, hidden, out_dim, act;
};

struct CacheArgs {
    void *refs;
    float *sqn;
    void *lat;
    uint16_t *idx;
    const int32_t *tbl = nullptr;  // paged layout: block table [B][H][max_pages]
    int64_t npages = 0;            // paged layout: pages in each pool
};

// Paged layout: logical pages per unit, and the device-side page map of a
// cache (dm.pr != 0).
inline int64_t pages_per_unit(const Dims &dm) {
    const int64_t pp = (int64_t)dm.pr * dm.s;
    return (dm.cap + pp - 1) / pp;
}
inline PageMap page_map(const Dims &dm, const CacheArgs &c) {
    PageMap pm;
    pm.tbl = c.tbl;
    pm.maxp = pages_per_unit(dm);
    int lg = 0;
    while ((1 << lg) < dm.pr) ++lg;
    pm.lg = lg;
    pm.npp = dm.pr * (dm.s - 1);
    pm.npages = (int32_t)c.npages;
    // ceil(2^40 / npp): exact quotients while t npp < 2^40
    pm.mag = (((uint64_t)1 << 40) + (uint64_t)pm.npp - 1) / (uint64_t)pm.npp;
    return pm;
}

// reference-set build
hipError_t launch_build_refs(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                             const CacheArgs &c, hipStream_t st);

// compression: workspace layout and size
size_t compress_ws_bytes(const Dims &dm, int64_t t0, int64_t t1);
hipError_t launch_compress(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                           const MlpArgs &comp, const CacheArgs &c, void *ws, size_t ws_bytes,
                           uint32_t *stats, hipStream_t st);

// compression into a paged cache (k_paged.hip): the unit's reference pages
// staged contiguously, the unit-contiguous kernels, the range's rows copied
// into their pages
size_t paged_compress_ws_bytes(const Dims &dm, int64_t t0, int64_t t1);
hipError_t launch_compress_paged(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                                 const MlpArgs &comp, const CacheArgs &c, void *ws,
                                 size_t ws_bytes, uint32_t *stats, hipStream_t st);

// decode attention
size_t decode_ws_bytes(const Dims &dm, int Hq, int64_t T);
hipError_t launch_decode(const Dims &dm, int Hq, int64_t T, const void *q, const CacheArgs &kc,
                         const MlpArgs &kdec, const CacheArgs &vc, const MlpArgs &vdec,
                         float scale, float *out, void *ws, size_t ws_bytes, hipStream_t st);
// dense decode attention that also selects, per (sequence, KV head), the
// n_keep positions of largest attention probability summed over the group
size_t decode_select_ws_bytes(const Dims &dm, int Hq, int64_t T);
hipError_t launch_decode_select(const Dims &dm, int Hq, int64_t T, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, float scale, float *out, int n_keep,
                                int32_t *positions, float *scores, void *ws, size_t ws_bytes,
                                hipStream_t st);
// dense decode attention over the compressed cache plus n_win exact rows
// kwin / vwin [B][H][n_win][d] (a recent window or attention sinks)
size_t decode_window_ws_bytes(const Dims &dm, int Hq, int64_t T, int64_t n_win);
hipError_t launch_decode_window(const Dims &dm, int Hq, int64_t T, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, const void *kwin, const void *vwin,
                                int64_t n_win, float scale, float *out, void *ws, size_t ws_bytes,
                                hipStream_t st);
// decode attention over a batch of sequences of different lengths
// (lens[b] tokens of sequence b, a device array, clamped into [1, nmax])
size_t decode_varlen_ws_bytes(const Dims &dm, int Hq, int64_t nmax);
hipError_t launch_decode_varlen(const Dims &dm, int Hq, const int64_t *lens, int64_t nmax,
                                const void *q, const CacheArgs &kc, const MlpArgs &kdec,
                                const CacheArgs &vc, const MlpArgs &vdec, float scale, float *out,
                                void *ws, size_t ws_bytes, hipStream_t st);
// mixed lengths on the dense kernels: per-unit (compressed, reference) counts
bool decode_counts_supported(const Dims &dm, const MlpArgs &kdec, const MlpArgs &vdec);
size_t decode_counts_ws_bytes(const Dims &dm, int Hq, int64_t nmax);
hipError_t launch_decode_counts(const Dims &dm, int Hq, int64_t nmax, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, const int32_t *counts, float scale,
                                float *out, void *ws, hipStream_t st);
// whether a call on a 4-bit latent cache has a kernel (compress / decode)
bool compress_q4_supported(const Dims &dm, const MlpArgs &comp);
bool decode_q4_supported(const Dims &dm, const MlpArgs &kdec, const MlpArgs &vdec);
// bytes of one unit's latent array
inline int64_t lat_unit_bytes(const Dims &dm) {
    return dm.lat_fmt ? dm.N * (dm.dc / 2 + 4) : dm.N * dm.dc * (dm.dtype == 0 ? 4 : 2);
}
// sparse decode attention over listed positions pos[B][H][nsel]
size_t decode_sparse_ws_bytes(const Dims &dm, int Hq, int64_t T, int nsel);
hipError_t launch_decode_sparse(const Dims &dm, int Hq, int64_t T, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, const int32_t *pos, int nsel, float scale,
                                float *out, void *ws, size_t ws_bytes, hipStream_t st);

}  // namespace dk

namespace dk {
// exact fp64 top-k scan (k_select.hip); list mode when `list` is non-null
// (bf16: the first listed tokens split over blocks, with partial lists in
// `scratch`, up to exact_list_ws_bytes)
hipError_t launch_select_exact(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                               int64_t q0, int64_t nq, const CacheArgs &c,
                               const uint64_t *list, const uint32_t *list_count,
                               int64_t list_cap, void *scratch, size_t scratch_bytes,
                               hipStream_t st, uint32_t *stats = nullptr);
size_t exact_list_ws_bytes(const Dims &dm, int64_t t1, int64_t nitems);
// exact selection of a few tokens (bf16) with the references split over
// blocks; workspace of select_split_ws_bytes
size_t select_split_ws_bytes(const Dims &dm, int64_t t0, int64_t t1);
// Reference-range splits of the matrix-core top-k search of nq tokens ending
// before t1, and the workspace their lists take beyond the fallback list
void topk_split_plan(const Dims &dm, int64_t t1, int64_t nq, int *nsplit, int *chunk);
size_t topk_split_ws_bytes(const Dims &dm, int64_t t1, int64_t nq);
hipError_t launch_select_split(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                               int64_t nq, const CacheArgs &c, void *ws, hipStream_t st);
}  // namespace dk

namespace dk {
// matrix-core top-k with certificate and exact fallback (k_select.hip, bf16)
hipError_t launch_select_mfma(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                              int64_t nq, const CacheArgs &c, uint64_t *flist, uint32_t *fcount,
                              uint32_t *stats, hipStream_t st);
// measured denominators (k_peaks.hip): `blocks` blocks of 256 threads
hipError_t launch_peak_mfma(int blocks, int iters, float *sink, hipStream_t st);
hipError_t launch_peak_gelu(int blocks, int iters, float *sink, hipStream_t st);

// ---- batched one-token appends -----------------------------------------------
// One position t appended to up to kAppendMax caches of the same shape in one
// set of launches (a decode step appends one token to every layer and stream).
// Passed to kernels by value.
constexpr int kAppendMax = 32;
struct AppendSet {
    const void *x[kAppendMax];      // [B][H][1][d]: the row of position t of every unit
    void *refs[kAppendMax];
    float *sqn[kAppendMax];
    void *lat[kAppendMax];
    uint16_t *idx[kAppendMax];
    const void *w1[kAppendMax];
    const float *b1[kAppendMax];
    const void *w2[kAppendMax];
    const float *b2[kAppendMax];
    // paged caches: each cache's block table and pool size (the page geometry,
    // common to the set, travels in a PageMap beside the set)
    const int32_t *tbl[kAppendMax];
    int32_t npages[kAppendMax];
};
// the page map of cache `item` of a set (pg: the set's common page geometry)
__host__ __device__ inline PageMap item_pages(const PageMap &pg, const AppendSet &set, int item) {
    PageMap pm = pg;
    pm.tbl = set.tbl[item];
    pm.npages = set.npages[item];
    return pm;
}
// the batched kernels serve bf16 caches with the matrix-core Compressor's
// shapes; other shapes run the per-cache calls
bool append_batched_supported(const Dims &dm, const MlpArgs &comp);
size_t append_ws_bytes(const Dims &dm, int64_t t, int n);
size_t append_select_ws_bytes(const Dims &dm, int64_t t, int n);
hipError_t launch_append_refs(const Dims &dm, int64_t t, int n, const AppendSet &set,
                              hipStream_t st);
// the set's common page geometry (dm.pr != 0), tables left to the items
inline PageMap set_pages(const Dims &dm) {
    if (!dm.pr) return PageMap{};
    CacheArgs none{};
    return page_map(dm, none);
}
hipError_t launch_append_select(const Dims &dm, int64_t t, int n, const AppendSet &set, void *ws,
                                hipStream_t st);
hipError_t launch_append_compress(const Dims &dm, int64_t t, int n, const AppendSet &set,
                                  int hidden, int act, hipStream_t st);

// ---- residual rows and Compressor / Decompressor training (k_train.hip) -------
// residual rows of the compressed tokens of [t0, t1): out [B][H][nq][d] fp32
hipError_t launch_residuals(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                            const CacheArgs &c, float *out, hipStream_t st);
struct MlpF32 {
    float *w1, *b1, *w2, *b2;   // [hidden][in], [hidden], [out][hidden], [out]
    int in, hidden, out, act;
};
struct TrainArgs {
    int64_t n;            // residual rows
    const float *delta;   // [n][comp.in]
    MlpF32 comp, dec;     // comp: d -> d_c, dec: d_c -> d
    float lr, momentum;
    float *velocity;      // packed parameters, or null (momentum 0)
    float *grad;          // packed parameters, or null
    float *loss;          // [1], or null
    void *wexp[4];        // bf16 copies of W1c, W2c, W1d, W2d written after the update, or null
    void *ws;
};
size_t train_ws_bytes(int d, int h1, int dc, int h2, int64_t n);
hipError_t launch_train_step(const TrainArgs &a, hipStream_t st);

}  // namespace dk
