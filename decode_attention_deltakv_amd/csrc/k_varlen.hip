// k_varlen.hip -- decode attention over a batch whose sequences hold different
// numbers of tokens (serving batches mix lengths).  Sequence b attends its
// positions 0 .. len[b] - 1, the lengths read on the device (each clamped
// into [1, nmax], the bound the launch plan is sized for).  Where the
// wave-specialised decode kernel serves the shape, it runs with per-unit
// token counts written here; otherwise the
// call runs as the sparse decode over position lists written here (every
// position below the sequence's length, then -1 padding), which over a full
// list gives the dense result.
#include <algorithm>

#include "dk_common.h"
#include "dk_launch.h"

namespace dk {
namespace {

__device__ __forceinline__ int64_t clamp_len(int64_t len, int64_t nmax) {
    return len < 1 ? 1 : (len > nmax ? nmax : len);
}

// pos[b][h][i] = i < len_b ? i : -1, for i < nmax.  grid (ceil(nmax / 256), H, B).
__global__ __launch_bounds__(256) void varlen_lists_kernel(const int64_t *__restrict__ lens,
                                                           int nmax, int32_t *__restrict__ pos) {
    const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nmax) return;
    const int64_t len = clamp_len(lens[b], nmax);
    pos[((int64_t)b * H + h) * nmax + i] = i < len ? (int32_t)i : -1;
}

// counts[b][h] = (compressed tokens, references) among positions 0 .. len_b - 1.
// grid B, H threads (at most 1024 KV heads).
__global__ void varlen_counts_kernel(const int64_t *__restrict__ lens, int64_t nmax, int s,
                                     int32_t *__restrict__ counts) {
    const int b = blockIdx.x, h = threadIdx.x, H = blockDim.x;
    const int64_t len = clamp_len(lens[b], nmax);
    const int64_t r = (len + s - 1) / s;
    counts[2 * ((int64_t)b * H + h)] = (int32_t)(len - r);
    counts[2 * ((int64_t)b * H + h) + 1] = (int32_t)r;
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

// Workspace: the lists, then the sparse call's, or the counts, then the
// counts-mode call's (the larger of the two ways, so the size does not depend
// on the MLPs).
size_t decode_varlen_ws_bytes(const Dims &dm, int Hq, int64_t nmax) {
    const size_t lists = align256((size_t)dm.B * dm.H * nmax * 4) +
                         decode_sparse_ws_bytes(dm, Hq, nmax, (int)nmax);
    const size_t counts = align256((size_t)dm.B * dm.H * 8) + decode_counts_ws_bytes(dm, Hq, nmax);
    return std::max(lists, counts);
}

hipError_t launch_decode_varlen(const Dims &dm, int Hq, const int64_t *lens, int64_t nmax,
                                const void *q, const CacheArgs &kc, const MlpArgs &kdec,
                                const CacheArgs &vc, const MlpArgs &vdec, float scale, float *out,
                                void *ws, size_t ws_bytes, hipStream_t st) {
    char *w = (char *)ws;
    int32_t *pos = (int32_t *)w;
    char *sws = w + align256((size_t)dm.B * dm.H * nmax * 4);
    hipError_t e;
    if (dm.H <= 1024 && decode_counts_supported(dm, kdec, vdec)) {
        int32_t *counts = (int32_t *)w;
        char *dws = w + align256((size_t)dm.B * dm.H * 8);
        hipLaunchKernelGGL(varlen_counts_kernel, dim3((unsigned)dm.B), dim3((unsigned)dm.H), 0, st,
                           lens, nmax, dm.s, counts);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_decode_counts(dm, Hq, nmax, q, kc, kdec, vc, vdec, counts, scale, out, dws,
                                    st);
    }
    if (dm.pr) return hipErrorInvalidValue;  // paged caches take the counts path only
    hipLaunchKernelGGL(varlen_lists_kernel, dim3((unsigned)((nmax + 255) / 256), dm.H, dm.B),
                       dim3(256), 0, st, lens, (int)nmax, pos);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_sparse(dm, Hq, nmax, q, kc, kdec, vc, vdec, pos, (int)nmax, scale, out,
                                sws, ws_bytes - (size_t)(sws - w), st);
}

}  // namespace dk
