// k_paged.hip -- compression into a paged cache.
//
// The DeltaKV page ("DeltaKV: Residual-Based KV Cache Compression via
// Long-Range Similarity", section 4, "Implementazione") pairs the method with
// a cache manager for irregular compressed layouts; a serving engine keeps such
// caches in pages of a shared pool, indexed by a block table per (sequence,
// head), as a paged KV cache does.  The decode kernels read the pages through
// the table directly.  Compression instead stages: the search for the k
// nearest references reads every earlier reference of a unit once per tile of
// 256 tokens (and the exact scans read them again), so one copy of the unit's
// reference pages into a contiguous staging area per call costs at most one
// more pass over them, and the search and Compressor kernels then run
// unchanged on the staging area.  The index and latent rows of the call's
// range are written to staging rows too and then copied into their pages.
//
// Workspace of a paged compress call over [t0, t1) (U = B H units, Rl =
// ceil(t1 / s) references, nq compressed tokens in the range):
//   refs [U][Rl][d] bf16, sqnorm [U][Rl] fp32, idx [U][nq][k] uint16,
//   latents [U][nq][d_c] bf16 (each 256-byte aligned), then the workspace of
//   the unit-contiguous call.
#include <algorithm>

#include "dk_common.h"
#include "dk_launch.h"

namespace dk {

namespace {

static inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

struct StagePlan {
    int64_t Rl, q0, nq;
    size_t off_refs, off_sqn, off_idx, off_lat, off_ws, total;
};

StagePlan stage_plan(const Dims &dm, int64_t t0, int64_t t1) {
    StagePlan p;
    const size_t U = (size_t)dm.B * dm.H;
    p.Rl = std::max<int64_t>(1, refs_upto(t1, dm.s));
    p.q0 = toks_upto(t0, dm.s);
    p.nq = toks_upto(t1, dm.s) - p.q0;
    const int64_t nqs = std::max<int64_t>(1, p.nq);
    size_t off = 0;
    p.off_refs = off;
    off += al256(U * p.Rl * dm.d * 2);
    p.off_sqn = off;
    off += al256(U * p.Rl * 4);
    p.off_idx = off;
    off += al256(U * nqs * dm.k * 2);
    p.off_lat = off;
    off += al256(U * nqs * dm.dc * 2);
    p.off_ws = off;
    p.total = off;
    return p;
}

// Dims of the staging area seen as a unit-contiguous cache: Rl reference rows
// and nq token rows per unit.
Dims staged_dims(const Dims &dm, const StagePlan &p) {
    Dims d2 = dm;
    d2.pr = 0;
    d2.R = p.Rl;
    d2.N = std::max<int64_t>(1, p.nq);
    return d2;
}

// Reference rows [0, Rl) of every unit from their pages into the staging
// area, with their squared norms: one thread per 16-byte chunk, grid
// (ceil(Rl CH / 256), U).
template <int D>
__global__ __launch_bounds__(256) void gather_refs_kernel(const bf16_t *__restrict__ pool,
                                                          const float *__restrict__ pool_sqn,
                                                          PageMap pm, int64_t Rl,
                                                          bf16_t *__restrict__ srefs,
                                                          float *__restrict__ ssqn) {
    constexpr int CH = D / 8;
    const int64_t unit = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t j = i / CH;
    const int c = (int)(i % CH);
    if (j >= Rl) return;
    const int64_t row = pg_ref_row(pm, unit, j);
    const uint4 v = reinterpret_cast<const uint4 *>(pool + row * D)[c];
    reinterpret_cast<uint4 *>(srefs + (unit * Rl + j) * D)[c] = v;
    if (c == 0) ssqn[unit * Rl + j] = pool_sqn[row];
}

// Index and latent rows of token ordinals [q0, q0 + nq) of every unit from
// the staging area into their pages: one thread per token, grid
// (ceil(nq / 256), U).
__global__ __launch_bounds__(256) void scatter_tokens_kernel(const uint16_t *__restrict__ sidx,
                                                             const bf16_t *__restrict__ slat,
                                                             int64_t q0, int64_t nq, int k,
                                                             int dc, PageMap pm,
                                                             uint16_t *__restrict__ idx,
                                                             bf16_t *__restrict__ lat) {
    const int64_t unit = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nq) return;
    const int64_t row = pg_tok_row(pm, unit, q0 + i);
    const uint16_t *si = sidx + (unit * nq + i) * k;
    if (k == 4) {
        *reinterpret_cast<uint2 *>(idx + row * 4) = *reinterpret_cast<const uint2 *>(si);
    } else if (k == 8) {
        *reinterpret_cast<uint4 *>(idx + row * 8) = *reinterpret_cast<const uint4 *>(si);
    } else {
        for (int r = 0; r < k; ++r) idx[row * k + r] = si[r];
    }
    const uint4 *sl = reinterpret_cast<const uint4 *>(slat + (unit * nq + i) * dc);
    uint4 *dl = reinterpret_cast<uint4 *>(lat + row * dc);
    for (int c = 0; c < dc / 8; ++c) dl[c] = sl[c];
}

}  // namespace

size_t paged_compress_ws_bytes(const Dims &dm, int64_t t0, int64_t t1) {
    const StagePlan p = stage_plan(dm, t0, t1);
    return p.off_ws + compress_ws_bytes(staged_dims(dm, p), t0, t1);
}

hipError_t launch_compress_paged(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                                 const MlpArgs &comp, const CacheArgs &c, void *ws,
                                 size_t ws_bytes, uint32_t *stats, hipStream_t st) {
    const StagePlan p = stage_plan(dm, t0, t1);
    if (p.nq <= 0) return hipSuccess;
    const Dims d2 = staged_dims(dm, p);
    const PageMap pm = page_map(dm, c);
    const unsigned U = (unsigned)(dm.B * dm.H);
    char *w = (char *)ws;
    bf16_t *srefs = (bf16_t *)(w + p.off_refs);
    float *ssqn = (float *)(w + p.off_sqn);
    uint16_t *sidx = (uint16_t *)(w + p.off_idx);
    bf16_t *slat = (bf16_t *)(w + p.off_lat);
    const int CH = dm.d / 8;
    const dim3 gg((unsigned)((p.Rl * CH + 255) / 256), U);
    if (dm.d == 128)
        hipLaunchKernelGGL(gather_refs_kernel<128>, gg, dim3(256), 0, st,
                           (const bf16_t *)c.refs, c.sqn, pm, p.Rl, srefs, ssqn);
    else
        hipLaunchKernelGGL(gather_refs_kernel<64>, gg, dim3(256), 0, st,
                           (const bf16_t *)c.refs, c.sqn, pm, p.Rl, srefs, ssqn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the staging rows as a unit-contiguous cache whose token rows start at
    // ordinal q0: row (unit, q) of the kernels' (unit N + q) addressing is
    // staging row unit nq + (q - q0)
    CacheArgs c2{};
    c2.refs = srefs;
    c2.sqn = ssqn;
    c2.idx = sidx - p.q0 * dm.k;
    c2.lat = slat - p.q0 * dm.dc;
    e = launch_compress(d2, x, t0, t1, comp, c2, w + p.off_ws, ws_bytes - p.off_ws, stats, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scatter_tokens_kernel, dim3((unsigned)((p.nq + 255) / 256), U), dim3(256),
                       0, st, sidx, slat, p.q0, p.nq, dm.k, dm.dc, pm, c.idx, (bf16_t *)c.lat);
    return hipGetLastError();
}

}  // namespace dk
