// dk_launch.h -- host-side launchers of libdeltakv's kernels.  Every launcher
// enqueues on `stream` and returns hipSuccess or the launch error.  Arguments
// have been validated by the C ABI layer (api.cpp) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dk {

// Sizes of one (layer, stream) cache, derived from deltakv_shape.
struct Dims {
    int B, H, d, s, k, dc;
    int dtype;          // 0 fp32, 1 bf16
    int lat_fmt;        // 0: latents in dtype, 1: 4-bit codes + per-row bf16 shift / scale
    int64_t cap;        // capacity (positions)
    int64_t R;          // reference rows per unit = ceil(cap / s)
    int64_t N;          // compressed-token rows per unit = cap - R
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
};

// reference-set build
hipError_t launch_build_refs(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                             const CacheArgs &c, hipStream_t st);

// compression: workspace layout and size
size_t compress_ws_bytes(const Dims &dm, int64_t t0, int64_t t1);
hipError_t launch_compress(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                           const MlpArgs &comp, const CacheArgs &c, void *ws, size_t ws_bytes,
                           uint32_t *stats, hipStream_t st);

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
// (lens_host[b] tokens of sequence b, at most nmax), through the sparse decode
size_t decode_varlen_ws_bytes(const Dims &dm, int Hq, int64_t nmax);
hipError_t launch_decode_varlen(const Dims &dm, int Hq, const int64_t *lens_host, int64_t nmax,
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
                               hipStream_t st);
size_t exact_list_ws_bytes(const Dims &dm, int64_t t1);
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
}  // namespace dk
