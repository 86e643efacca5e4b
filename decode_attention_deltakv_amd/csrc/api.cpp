// api.cpp -- the C ABI of libdeltakv.so (declared in include/deltakv.h):
// argument validation, cache / workspace sizing and dispatch to the kernel
// launchers.  Validation happens before any HIP call, so every error that an
// argument can cause is returned synchronously and without a device.
#include "deltakv.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "dk_common.h"
#include "dk_launch.h"

namespace {

thread_local std::string g_last_error;

constexpr int32_t kMaxAppendItems = 4096;

deltakv_status fail(deltakv_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

deltakv_status ok() {
    g_last_error.clear();
    return DELTAKV_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

deltakv_status check_shape(const deltakv_shape *sh, dk::Dims *dm) {
    if (!sh) return fail(DELTAKV_ERR_INVALID_ARG, "shape is NULL");
    if (sh->batch < 1 || sh->num_kv_heads < 1)
        return fail(DELTAKV_ERR_INVALID_ARG, "batch (%d) and num_kv_heads (%d) must be >= 1",
                    sh->batch, sh->num_kv_heads);
    if (sh->head_dim != 64 && sh->head_dim != 128)
        return fail(DELTAKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", sh->head_dim);
    if (sh->stride < 1) return fail(DELTAKV_ERR_INVALID_ARG, "stride %d < 1", sh->stride);
    if (sh->k < 1 || sh->k > 8) return fail(DELTAKV_ERR_UNSUPPORTED, "k %d not in [1, 8]", sh->k);
    if (sh->d_c != 16 && sh->d_c != 32 && sh->d_c != 64 && sh->d_c != 128)
        return fail(DELTAKV_ERR_UNSUPPORTED, "d_c %d not in {16, 32, 64, 128}", sh->d_c);
    if (sh->capacity < 1) return fail(DELTAKV_ERR_INVALID_ARG, "capacity %lld < 1",
                                      (long long)sh->capacity);
    if (sh->dtype != DELTAKV_F32 && sh->dtype != DELTAKV_BF16)
        return fail(DELTAKV_ERR_UNSUPPORTED, "dtype %d unknown", sh->dtype);
    if (sh->latent_format != DELTAKV_LATENT_DTYPE && sh->latent_format != DELTAKV_LATENT_Q4)
        return fail(DELTAKV_ERR_INVALID_ARG, "latent_format %d unknown", sh->latent_format);
    if (sh->latent_format == DELTAKV_LATENT_Q4 &&
        (sh->dtype != DELTAKV_BF16 || (sh->d_c != 16 && sh->d_c != 32)))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents need bf16 and d_c 16 or 32");
    const int64_t R = dk::refs_upto(sh->capacity, sh->stride);
    if (R > 65535)
        return fail(DELTAKV_ERR_CAPACITY,
                    "capacity %lld at stride %d needs %lld reference rows; 16-bit indices "
                    "hold at most 65535", (long long)sh->capacity, sh->stride, (long long)R);
    // keep every array's element count far inside int64
    const double elems = (double)sh->batch * sh->num_kv_heads * (double)sh->capacity * 128.0;
    if (elems > 9.0e15) return fail(DELTAKV_ERR_CAPACITY, "cache too large");
    if (sh->page_refs != 0) {
        const int pr = sh->page_refs;
        if (pr < 128 || pr > 4096 || (pr & (pr - 1)) != 0)
            return fail(DELTAKV_ERR_UNSUPPORTED,
                        "page_refs %d: a paged cache needs a power of two in [128, 4096]", pr);
        if (sh->stride < 2 || sh->dtype != DELTAKV_BF16 ||
            sh->latent_format != DELTAKV_LATENT_DTYPE)
            return fail(DELTAKV_ERR_UNSUPPORTED,
                        "a paged cache needs stride >= 2, bf16 storage and latents in bf16");
        // token ordinals are split into pages by a multiply-shift that is
        // exact while (tokens per unit) x (tokens per page) < 2^40
        if ((double)sh->capacity * (double)pr * (double)(sh->stride - 1) >= 1099511627776.0)
            return fail(DELTAKV_ERR_UNSUPPORTED,
                        "paged cache: capacity x page_refs x (stride - 1) must stay below 2^40");
    }
    if (dm) {
        dm->B = sh->batch;
        dm->H = sh->num_kv_heads;
        dm->d = sh->head_dim;
        dm->s = sh->stride;
        dm->k = sh->k;
        dm->dc = sh->d_c;
        dm->dtype = sh->dtype;
        dm->lat_fmt = sh->latent_format;
        dm->cap = sh->capacity;
        dm->R = R;
        dm->N = sh->capacity - R;
        dm->pr = sh->page_refs;
    }
    return DELTAKV_OK;
}

deltakv_status check_mlp(const deltakv_mlp *m, const char *name, int in_dim, int out_dim,
                         dk::MlpArgs *a) {
    if (!m) return fail(DELTAKV_ERR_INVALID_ARG, "%s is NULL", name);
    if (!m->w1 || !m->w2) return fail(DELTAKV_ERR_INVALID_ARG, "%s weights are NULL", name);
    if (!aligned16(m->w1) || !aligned16(m->w2))
        return fail(DELTAKV_ERR_INVALID_ARG, "%s weights must be 16-byte aligned", name);
    if ((m->b1 && !aligned16(m->b1)) || (m->b2 && !aligned16(m->b2)))
        return fail(DELTAKV_ERR_INVALID_ARG, "%s biases must be 16-byte aligned", name);
    if (m->in_dim != in_dim || m->out_dim != out_dim)
        return fail(DELTAKV_ERR_INVALID_ARG, "%s maps %d -> %d, expected %d -> %d", name,
                    m->in_dim, m->out_dim, in_dim, out_dim);
    if (m->hidden != 64 && m->hidden != 128 && m->hidden != 256)
        return fail(DELTAKV_ERR_UNSUPPORTED, "%s hidden width %d not in {64, 128, 256}", name,
                    m->hidden);
    if (m->act != DELTAKV_ACT_GELU && m->act != DELTAKV_ACT_IDENTITY)
        return fail(DELTAKV_ERR_INVALID_ARG, "%s activation %d unknown", name, m->act);
    a->w1 = m->w1;
    a->b1 = m->b1;
    a->w2 = m->w2;
    a->b2 = m->b2;
    a->in_dim = m->in_dim;
    a->hidden = m->hidden;
    a->out_dim = m->out_dim;
    a->act = m->act;
    return DELTAKV_OK;
}

// reads_upto > 0: the call reads positions [0, reads_upto), which must have
// been compressed (the struct's host-side filled length).
deltakv_status check_cache(const deltakv_cache *c, const dk::Dims &dm, const char *name,
                           bool need_tokens, dk::CacheArgs *a, int64_t reads_upto = 0) {
    if (!c) return fail(DELTAKV_ERR_INVALID_ARG, "%s is NULL", name);
    if (c->n_compressed < 0 || c->n_compressed > c->n_built || c->n_built > dm.cap)
        return fail(DELTAKV_ERR_INVALID_ARG,
                    "%s: filled lengths need 0 <= n_compressed (%lld) <= n_built (%lld) <= "
                    "capacity (%lld)", name, (long long)c->n_compressed, (long long)c->n_built,
                    (long long)dm.cap);
    if (reads_upto > c->n_compressed)
        return fail(DELTAKV_ERR_INVALID_ARG,
                    "%s: the call reads %lld positions but only %lld are compressed", name,
                    (long long)reads_upto, (long long)c->n_compressed);
    if (!c->refs || !c->ref_sqnorm)
        return fail(DELTAKV_ERR_INVALID_ARG, "%s: refs / ref_sqnorm are NULL", name);
    if (need_tokens && dm.N > 0 && (!c->latents || !c->idx))
        return fail(DELTAKV_ERR_INVALID_ARG, "%s: latents / idx are NULL", name);
    if (!aligned16(c->refs) || !aligned16(c->ref_sqnorm) ||
        (c->latents && !aligned16(c->latents)) || (c->idx && !aligned16(c->idx)))
        return fail(DELTAKV_ERR_INVALID_ARG, "%s: arrays must be 16-byte aligned", name);
    a->refs = c->refs;
    a->sqn = c->ref_sqnorm;
    a->lat = c->latents;
    a->idx = c->idx;
    a->tbl = nullptr;
    a->npages = 0;
    if (dm.pr) {
        if (!c->block_table || (reinterpret_cast<uintptr_t>(c->block_table) & 3u))
            return fail(DELTAKV_ERR_INVALID_ARG,
                        "%s: a paged cache needs a 4-byte aligned block_table", name);
        if (c->n_pages < 1 || c->n_pages > INT32_MAX)
            return fail(DELTAKV_ERR_INVALID_ARG, "%s: n_pages %lld not in [1, 2^31)", name,
                        (long long)c->n_pages);
        // the decode addresses reference rows by 32-bit byte offsets into the pool
        if ((double)c->n_pages * dm.pr * dm.d * 2.0 > 2147483648.0)
            return fail(DELTAKV_ERR_UNSUPPORTED, "%s: a reference pool above 2 GiB", name);
        a->tbl = c->block_table;
        a->npages = c->n_pages;
    }
    return DELTAKV_OK;
}

deltakv_status check_range(const dk::Dims &dm, int64_t t0, int64_t t1) {
    if (t0 < 0 || t1 <= t0)
        return fail(DELTAKV_ERR_INVALID_ARG, "need 0 <= t0 < t1 (t0 %lld, t1 %lld)",
                    (long long)t0, (long long)t1);
    if (t1 > dm.cap)
        return fail(DELTAKV_ERR_CAPACITY, "t1 %lld exceeds capacity %lld", (long long)t1,
                    (long long)dm.cap);
    return DELTAKV_OK;
}

deltakv_status check_heads_tokens(const dk::Dims &dm, int32_t num_q_heads, int64_t n_tokens) {
    if (num_q_heads < 1 || num_q_heads % dm.H != 0 || num_q_heads / dm.H > 8)
        return fail(DELTAKV_ERR_UNSUPPORTED,
                    "num_q_heads %d must be a multiple of num_kv_heads %d, at most 8x",
                    num_q_heads, dm.H);
    if (n_tokens < 1 || n_tokens > dm.cap)
        return fail(n_tokens > dm.cap ? DELTAKV_ERR_CAPACITY : DELTAKV_ERR_INVALID_ARG,
                    "n_tokens %lld not in [1, capacity %lld]", (long long)n_tokens,
                    (long long)dm.cap);
    return DELTAKV_OK;
}

deltakv_status from_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(DELTAKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elt_bytes(const dk::Dims &dm) { return dm.dtype == DELTAKV_F32 ? 4 : 2; }

}  // namespace

extern "C" {

deltakv_status deltakv_cache_bytes(const deltakv_shape *shape, size_t *refs_bytes,
                                   size_t *ref_sqnorm_bytes, size_t *latents_bytes,
                                   size_t *idx_bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    const size_t units = (size_t)dm.B * dm.H;
    if (dm.pr) {
        // pools with every logical page of every unit backed
        const size_t pages = units * (size_t)dk::pages_per_unit(dm);
        const size_t pr = (size_t)dm.pr, npp = pr * (size_t)(dm.s - 1);
        if (refs_bytes) *refs_bytes = pages * pr * dm.d * elt_bytes(dm);
        if (ref_sqnorm_bytes) *ref_sqnorm_bytes = pages * pr * sizeof(float);
        if (latents_bytes) *latents_bytes = pages * npp * dm.dc * elt_bytes(dm);
        if (idx_bytes) *idx_bytes = pages * npp * dm.k * sizeof(uint16_t);
        return ok();
    }
    if (refs_bytes) *refs_bytes = units * dm.R * dm.d * elt_bytes(dm);
    if (ref_sqnorm_bytes) *ref_sqnorm_bytes = units * dm.R * sizeof(float);
    if (latents_bytes) *latents_bytes = units * (size_t)dk::lat_unit_bytes(dm);
    if (idx_bytes) *idx_bytes = units * dm.N * dm.k * sizeof(uint16_t);
    return ok();
}

deltakv_status deltakv_page_bytes(const deltakv_shape *shape, size_t *refs_bytes,
                                  size_t *ref_sqnorm_bytes, size_t *latents_bytes,
                                  size_t *idx_bytes, int32_t *max_pages) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if (!dm.pr) return fail(DELTAKV_ERR_INVALID_ARG, "page_refs is 0: the shape is not paged");
    const size_t pr = (size_t)dm.pr, npp = pr * (size_t)(dm.s - 1);
    if (refs_bytes) *refs_bytes = pr * dm.d * elt_bytes(dm);
    if (ref_sqnorm_bytes) *ref_sqnorm_bytes = pr * sizeof(float);
    if (latents_bytes) *latents_bytes = npp * dm.dc * elt_bytes(dm);
    if (idx_bytes) *idx_bytes = npp * dm.k * sizeof(uint16_t);
    if (max_pages) *max_pages = (int32_t)dk::pages_per_unit(dm);
    return ok();
}

deltakv_status deltakv_compress_workspace_bytes(const deltakv_shape *shape, int64_t t0,
                                                int64_t t1, size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t0, t1)) != DELTAKV_OK) return st;
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::compress_ws_bytes(dm, t0, t1);
    return ok();
}

deltakv_status deltakv_decode_workspace_bytes(const deltakv_shape *shape, int32_t num_q_heads,
                                              int64_t n_tokens, size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if (num_q_heads < 1 || num_q_heads % dm.H != 0 || num_q_heads / dm.H > 8)
        return fail(DELTAKV_ERR_UNSUPPORTED,
                    "num_q_heads %d must be a multiple of num_kv_heads %d, at most 8x",
                    num_q_heads, dm.H);
    if (n_tokens < 1 || n_tokens > dm.cap)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_tokens %lld not in [1, capacity]",
                    (long long)n_tokens);
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::decode_ws_bytes(dm, num_q_heads, n_tokens);
    return ok();
}

deltakv_status deltakv_decode_sparse_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t n_tokens,
                                                     int32_t n_sel, size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, n_tokens)) != DELTAKV_OK) return st;
    if (n_sel < 1 || n_sel > DELTAKV_MAX_SPARSE_SELECT)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_sel %d not in [1, %d]", n_sel,
                    DELTAKV_MAX_SPARSE_SELECT);
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::decode_sparse_ws_bytes(dm, num_q_heads, n_tokens, n_sel);
    return ok();
}

deltakv_status deltakv_decode_select_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t n_tokens,
                                                     size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, n_tokens)) != DELTAKV_OK) return st;
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::decode_select_ws_bytes(dm, num_q_heads, n_tokens);
    return ok();
}

deltakv_status deltakv_decode_window_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t n_tokens,
                                                     int64_t n_win, size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, n_tokens)) != DELTAKV_OK) return st;
    if (n_win < 1 || n_win > 65535)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_win %lld not in [1, 65535]", (long long)n_win);
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::decode_window_ws_bytes(dm, num_q_heads, n_tokens, n_win);
    return ok();
}

deltakv_status deltakv_decode_varlen_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t max_tokens,
                                                     size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, max_tokens)) != DELTAKV_OK) return st;
    if (max_tokens > DELTAKV_MAX_SPARSE_SELECT)
        return fail(DELTAKV_ERR_UNSUPPORTED, "max_tokens %lld above %d", (long long)max_tokens,
                    DELTAKV_MAX_SPARSE_SELECT);
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::decode_varlen_ws_bytes(dm, num_q_heads, max_tokens);
    return ok();
}

deltakv_status deltakv_build_refs(const deltakv_shape *shape, const void *x, int64_t t0,
                                  int64_t t1, deltakv_cache *cache, void *stream) {
    dk::Dims dm;
    dk::CacheArgs ca;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t0, t1)) != DELTAKV_OK) return st;
    if (!x) return fail(DELTAKV_ERR_INVALID_ARG, "x is NULL");
    if (!aligned16(x)) return fail(DELTAKV_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if ((st = check_cache(cache, dm, "cache", false, &ca)) != DELTAKV_OK) return st;
    if (t0 != cache->n_built)
        return fail(DELTAKV_ERR_INVALID_ARG,
                    "references are built in order: t0 (%lld) must equal n_built (%lld)",
                    (long long)t0, (long long)cache->n_built);
    st = from_hip(dk::launch_build_refs(dm, x, t0, t1, ca, (hipStream_t)stream),
                  "deltakv_build_refs");
    if (st == DELTAKV_OK) cache->n_built = t1;
    return st;
}

deltakv_status deltakv_compress(const deltakv_shape *shape, const void *x, int64_t t0,
                                int64_t t1, const deltakv_mlp *compressor,
                                deltakv_cache *cache, void *workspace,
                                size_t workspace_bytes, uint32_t *stats, void *stream) {
    dk::Dims dm;
    dk::CacheArgs ca;
    dk::MlpArgs ma;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t0, t1)) != DELTAKV_OK) return st;
    if (!x) return fail(DELTAKV_ERR_INVALID_ARG, "x is NULL");
    if (!aligned16(x)) return fail(DELTAKV_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if ((st = check_mlp(compressor, "compressor", dm.d, dm.dc, &ma)) != DELTAKV_OK) return st;
    if (dm.lat_fmt && !dk::compress_q4_supported(dm, ma))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: compressor must have hidden width "
                    "128 or 256");
    if ((st = check_cache(cache, dm, "cache", true, &ca)) != DELTAKV_OK) return st;
    if (t0 != cache->n_compressed)
        return fail(DELTAKV_ERR_INVALID_ARG,
                    "tokens are compressed in order: t0 (%lld) must equal n_compressed (%lld)",
                    (long long)t0, (long long)cache->n_compressed);
    if (t1 > cache->n_built)
        return fail(DELTAKV_ERR_INVALID_ARG,
                    "compressing up to %lld needs the references built that far (n_built %lld)",
                    (long long)t1, (long long)cache->n_built);
    const size_t need = dk::compress_ws_bytes(dm, t0, t1);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(DELTAKV_ERR_WORKSPACE, "compress needs %zu workspace bytes, got %zu", need,
                    workspace_bytes);
    if (workspace && !aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (dk::toks_upto(t1, dm.s) == dk::toks_upto(t0, dm.s)) {  // only references
        cache->n_compressed = t1;
        return ok();
    }
    st = from_hip(dk::launch_compress(dm, x, t0, t1, ma, ca, workspace, workspace_bytes, stats,
                                      (hipStream_t)stream),
                  "deltakv_compress");
    if (st == DELTAKV_OK) cache->n_compressed = t1;
    return st;
}

deltakv_status deltakv_residuals(const deltakv_shape *shape, const void *x, int64_t t0,
                                 int64_t t1, const deltakv_cache *cache, float *out,
                                 void *stream) {
    dk::Dims dm;
    dk::CacheArgs ca;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t0, t1)) != DELTAKV_OK) return st;
    if (!x) return fail(DELTAKV_ERR_INVALID_ARG, "x is NULL");
    if (!aligned16(x)) return fail(DELTAKV_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if ((st = check_cache(cache, dm, "cache", true, &ca, t1)) != DELTAKV_OK) return st;
    if (dm.pr) return fail(DELTAKV_ERR_UNSUPPORTED, "residual rows of a paged cache");
    const int64_t nq = dk::toks_upto(t1, dm.s) - dk::toks_upto(t0, dm.s);
    if (nq == 0) return ok();
    if (!out) return fail(DELTAKV_ERR_INVALID_ARG, "out is NULL");
    if (!aligned16(out)) return fail(DELTAKV_ERR_INVALID_ARG, "out must be 16-byte aligned");
    return from_hip(dk::launch_residuals(dm, x, t0, t1, ca, out, (hipStream_t)stream),
                    "deltakv_residuals");
}

deltakv_status deltakv_append_workspace_bytes(const deltakv_shape *shape, int64_t t,
                                              int32_t n_items, size_t *bytes) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t, t + 1)) != DELTAKV_OK) return st;
    if (n_items < 1 || n_items > kMaxAppendItems)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_items %d not in [1, %d]", n_items,
                    kMaxAppendItems);
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::append_ws_bytes(dm, t, n_items);
    return ok();
}

deltakv_status deltakv_append(const deltakv_shape *shape, int64_t t, int32_t n_items,
                              const deltakv_append_item *items, void *workspace,
                              size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t, t + 1)) != DELTAKV_OK) return st;
    if (n_items < 1 || n_items > kMaxAppendItems)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_items %d not in [1, %d]", n_items,
                    kMaxAppendItems);
    if (!items) return fail(DELTAKV_ERR_INVALID_ARG, "items is NULL");
    // every check before anything is enqueued
    std::vector<dk::CacheArgs> ca((size_t)n_items);
    std::vector<dk::MlpArgs> ma((size_t)n_items);
    bool batched = true;
    for (int i = 0; i < n_items; ++i) {
        const deltakv_append_item &it = items[i];
        char name[48];
        snprintf(name, sizeof(name), "items[%d].cache", i);
        if (!it.x) return fail(DELTAKV_ERR_INVALID_ARG, "items[%d].x is NULL", i);
        if (!aligned16(it.x))
            return fail(DELTAKV_ERR_INVALID_ARG, "items[%d].x must be 16-byte aligned", i);
        if ((st = check_mlp(it.compressor, "compressor", dm.d, dm.dc, &ma[i])) != DELTAKV_OK)
            return st;
        if (dm.lat_fmt && !dk::compress_q4_supported(dm, ma[i]))
            return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: items[%d].compressor must "
                        "have hidden width 128 or 256", i);
        if ((st = check_cache(it.cache, dm, name, true, &ca[i])) != DELTAKV_OK) return st;
        if (it.cache->n_built != t || it.cache->n_compressed != t)
            return fail(DELTAKV_ERR_INVALID_ARG,
                        "%s: appending position %lld needs n_built == n_compressed == %lld "
                        "(have %lld, %lld)", name, (long long)t, (long long)t,
                        (long long)it.cache->n_built, (long long)it.cache->n_compressed);
        // (paged caches may share a pool: then their block tables tell them apart)
        for (int j = 0; j < i; ++j)
            if (items[j].cache == it.cache ||
                (items[j].cache->refs == it.cache->refs &&
                 (!dm.pr || items[j].cache->block_table == it.cache->block_table)))
                return fail(DELTAKV_ERR_INVALID_ARG, "items %d and %d name the same cache", j,
                            i);
        batched = batched && dk::append_batched_supported(dm, ma[i]) &&
                  ma[i].hidden == ma[0].hidden && ma[i].act == ma[0].act;
    }
    const size_t need = dk::append_ws_bytes(dm, t, n_items);
    const bool is_ref = t % dm.s == 0;
    if (!is_ref && (workspace_bytes < need || !workspace))
        return fail(DELTAKV_ERR_WORKSPACE, "append needs %zu workspace bytes, got %zu", need,
                    workspace_bytes);
    if (workspace && !aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (batched) {
        for (int i0 = 0; i0 < n_items && e == hipSuccess; i0 += dk::kAppendMax) {
            const int n = std::min(dk::kAppendMax, n_items - i0);
            dk::AppendSet set{};
            for (int i = 0; i < n; ++i) {
                const int j = i0 + i;
                set.x[i] = items[j].x;
                set.refs[i] = ca[j].refs;
                set.sqn[i] = ca[j].sqn;
                set.lat[i] = ca[j].lat;
                set.idx[i] = ca[j].idx;
                set.w1[i] = ma[j].w1;
                set.b1[i] = ma[j].b1;
                set.w2[i] = ma[j].w2;
                set.b2[i] = ma[j].b2;
                set.tbl[i] = ca[j].tbl;
                set.npages[i] = (int32_t)ca[j].npages;
            }
            if (is_ref) {
                e = dk::launch_append_refs(dm, t, n, set, hs);
            } else {
                e = dk::launch_append_select(dm, t, n, set, workspace, hs);
                if (e == hipSuccess)
                    e = dk::launch_append_compress(dm, t, n, set, ma[0].hidden, ma[0].act, hs);
            }
        }
    } else {
        for (int i = 0; i < n_items && e == hipSuccess; ++i) {
            e = dk::launch_build_refs(dm, items[i].x, t, t + 1, ca[i], hs);
            if (e == hipSuccess && !is_ref)
                e = dk::launch_compress(dm, items[i].x, t, t + 1, ma[i], ca[i], workspace,
                                        workspace_bytes, nullptr, hs);
        }
    }
    st = from_hip(e, "deltakv_append");
    if (st == DELTAKV_OK)
        for (int i = 0; i < n_items; ++i) items[i].cache->n_built = items[i].cache->n_compressed =
            t + 1;
    return st;
}

}  // extern "C"

namespace {

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

deltakv_status check_mlp_f32(const deltakv_mlp_f32 *m, const char *name, dk::MlpF32 *a) {
    if (!m) return fail(DELTAKV_ERR_INVALID_ARG, "%s is NULL", name);
    if (!m->w1 || !m->b1 || !m->w2 || !m->b2)
        return fail(DELTAKV_ERR_INVALID_ARG, "%s: w1, b1, w2 and b2 must all be given", name);
    if (!aligned4(m->w1) || !aligned4(m->b1) || !aligned4(m->w2) || !aligned4(m->b2))
        return fail(DELTAKV_ERR_INVALID_ARG, "%s: arrays must be 4-byte aligned", name);
    if (m->in_dim < 1 || m->in_dim > 4096 || m->hidden < 1 || m->hidden > 4096 ||
        m->out_dim < 1 || m->out_dim > 4096)
        return fail(DELTAKV_ERR_INVALID_ARG, "%s: dimensions %d -> %d -> %d not in [1, 4096]",
                    name, m->in_dim, m->hidden, m->out_dim);
    if (m->act != DELTAKV_ACT_GELU && m->act != DELTAKV_ACT_IDENTITY)
        return fail(DELTAKV_ERR_INVALID_ARG, "%s activation %d unknown", name, m->act);
    *a = dk::MlpF32{m->w1, m->b1, m->w2, m->b2, m->in_dim, m->hidden, m->out_dim, m->act};
    return DELTAKV_OK;
}

deltakv_status check_pair(const deltakv_mlp_f32 *c, const deltakv_mlp_f32 *d, int64_t n_rows,
                          dk::MlpF32 *ca, dk::MlpF32 *da) {
    deltakv_status st;
    if ((st = check_mlp_f32(c, "compressor", ca)) != DELTAKV_OK) return st;
    if ((st = check_mlp_f32(d, "decompressor", da)) != DELTAKV_OK) return st;
    if (d->in_dim != c->out_dim || d->out_dim != c->in_dim)
        return fail(DELTAKV_ERR_INVALID_ARG,
                    "decompressor maps %d -> %d; the compressor maps %d -> %d", d->in_dim,
                    d->out_dim, c->in_dim, c->out_dim);
    if (n_rows < 1 || n_rows > ((int64_t)1 << 31))
        return fail(DELTAKV_ERR_INVALID_ARG, "n_rows %lld not in [1, 2^31]",
                    (long long)n_rows);
    return DELTAKV_OK;
}

int64_t n_params(const dk::MlpF32 &c, const dk::MlpF32 &d) {
    return (int64_t)c.hidden * (c.in + 1) + (int64_t)c.out * (c.hidden + 1) +
           (int64_t)d.hidden * (d.in + 1) + (int64_t)d.out * (d.hidden + 1);
}

}  // namespace

extern "C" {

deltakv_status deltakv_train_workspace_bytes(const deltakv_mlp_f32 *compressor,
                                             const deltakv_mlp_f32 *decompressor,
                                             int64_t n_rows, size_t *bytes,
                                             int64_t *n_params_out) {
    dk::MlpF32 ca, da;
    deltakv_status st = check_pair(compressor, decompressor, n_rows, &ca, &da);
    if (st != DELTAKV_OK) return st;
    if (!bytes) return fail(DELTAKV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dk::train_ws_bytes(ca.in, ca.hidden, ca.out, da.hidden, n_rows);
    if (n_params_out) *n_params_out = n_params(ca, da);
    return ok();
}

deltakv_status deltakv_train_step(int64_t n_rows, const float *delta,
                                  const deltakv_mlp_f32 *compressor,
                                  const deltakv_mlp_f32 *decompressor, float lr, float momentum,
                                  float *velocity, float *loss, float *grad,
                                  void *const *bf16_weights, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    dk::TrainArgs a{};
    deltakv_status st = check_pair(compressor, decompressor, n_rows, &a.comp, &a.dec);
    if (st != DELTAKV_OK) return st;
    if (!delta || !aligned4(delta))
        return fail(DELTAKV_ERR_INVALID_ARG, "delta must be a 4-byte aligned device array");
    if (!std::isfinite(lr)) return fail(DELTAKV_ERR_INVALID_ARG, "lr must be finite");
    if (!(momentum >= 0.f && momentum < 1.f))
        return fail(DELTAKV_ERR_INVALID_ARG, "momentum %g not in [0, 1)", (double)momentum);
    if (momentum != 0.f && !velocity)
        return fail(DELTAKV_ERR_INVALID_ARG, "momentum %g needs a velocity array",
                    (double)momentum);
    if ((velocity && !aligned4(velocity)) || (loss && !aligned4(loss)) ||
        (grad && !aligned4(grad)))
        return fail(DELTAKV_ERR_INVALID_ARG, "velocity, loss and grad must be 4-byte aligned");
    if (bf16_weights)
        for (int i = 0; i < 4; ++i)
            if (bf16_weights[i] && (reinterpret_cast<uintptr_t>(bf16_weights[i]) & 1u))
                return fail(DELTAKV_ERR_INVALID_ARG, "bf16_weights[%d] must be 2-byte aligned",
                            i);
    const size_t need =
        dk::train_ws_bytes(a.comp.in, a.comp.hidden, a.comp.out, a.dec.hidden, n_rows);
    if (workspace_bytes < need || !workspace)
        return fail(DELTAKV_ERR_WORKSPACE, "train step needs %zu workspace bytes, got %zu",
                    need, workspace_bytes);
    if (!aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    a.n = n_rows;
    a.delta = delta;
    a.lr = lr;
    a.momentum = momentum;
    a.velocity = velocity;
    a.grad = grad;
    a.loss = loss;
    for (int i = 0; i < 4; ++i) a.wexp[i] = bf16_weights ? bf16_weights[i] : nullptr;
    a.ws = workspace;
    return from_hip(dk::launch_train_step(a, (hipStream_t)stream), "deltakv_train_step");
}

}  // extern "C"

namespace {

// Paged caches: the wave-specialised decode's shapes and one block table for
// K and V.
deltakv_status check_paged_decode(const dk::Dims &dm, const deltakv_cache *k_cache,
                                  const dk::MlpArgs &km, const deltakv_cache *v_cache,
                                  const dk::MlpArgs &vm) {
    if (!dm.pr) return DELTAKV_OK;
    if (!dk::decode_counts_supported(dm, km, vm))
        return fail(DELTAKV_ERR_UNSUPPORTED, "paged caches: decode needs k 4 or 8, d_c <= 32 and "
                    "GELU decompressors of one hidden width, 128 or 256");
    if (k_cache->block_table != v_cache->block_table)
        return fail(DELTAKV_ERR_UNSUPPORTED, "paged caches: K and V must share one block table");
    return DELTAKV_OK;
}

// Argument checks of the dense decode (everything but the workspace).
deltakv_status check_decode(const deltakv_shape *shape, int32_t num_q_heads, int64_t n_tokens,
                            const void *q, const deltakv_cache *k_cache,
                            const deltakv_mlp *k_dec, const deltakv_cache *v_cache,
                            const deltakv_mlp *v_dec, float softmax_scale, const float *out,
                            dk::Dims &dm, dk::CacheArgs &kc, dk::MlpArgs &km, dk::CacheArgs &vc,
                            dk::MlpArgs &vm) {
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if (num_q_heads < 1 || num_q_heads % dm.H != 0 || num_q_heads / dm.H > 8)
        return fail(DELTAKV_ERR_UNSUPPORTED,
                    "num_q_heads %d must be a multiple of num_kv_heads %d, at most 8x",
                    num_q_heads, dm.H);
    if (n_tokens < 1 || n_tokens > dm.cap)
        return fail(n_tokens > dm.cap ? DELTAKV_ERR_CAPACITY : DELTAKV_ERR_INVALID_ARG,
                    "n_tokens %lld not in [1, capacity %lld]", (long long)n_tokens,
                    (long long)dm.cap);
    if (!q || !out) return fail(DELTAKV_ERR_INVALID_ARG, "q / out is NULL");
    if (!aligned16(q) || !aligned16(out))
        return fail(DELTAKV_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!std::isfinite(softmax_scale))
        return fail(DELTAKV_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((st = check_mlp(k_dec, "k_dec", dm.dc, dm.d, &km)) != DELTAKV_OK) return st;
    if ((st = check_mlp(v_dec, "v_dec", dm.dc, dm.d, &vm)) != DELTAKV_OK) return st;
    if (dm.lat_fmt && !dk::decode_q4_supported(dm, km, vm))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: decode needs k 4 or 8 and GELU "
                    "decompressors of one hidden width, 128 or 256");
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc, n_tokens)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc, n_tokens)) != DELTAKV_OK) return st;
    return check_paged_decode(dm, k_cache, km, v_cache, vm);
}

}  // namespace

extern "C" {

deltakv_status deltakv_decode_attn(const deltakv_shape *shape, int32_t num_q_heads,
                                   int64_t n_tokens, const void *q,
                                   const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                   const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                   float softmax_scale, float *out, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
    deltakv_status st = check_decode(shape, num_q_heads, n_tokens, q, k_cache, k_dec, v_cache,
                                     v_dec, softmax_scale, out, dm, kc, km, vc, vm);
    if (st != DELTAKV_OK) return st;
    const size_t need = dk::decode_ws_bytes(dm, num_q_heads, n_tokens);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(DELTAKV_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need,
                    workspace_bytes);
    if (workspace && !aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return from_hip(dk::launch_decode(dm, num_q_heads, n_tokens, q, kc, km, vc, vm,
                                      softmax_scale, out, workspace, workspace_bytes,
                                      (hipStream_t)stream),
                    "deltakv_decode_attn");
}

}  // extern "C"

// ---- the decode entry point that allocates nothing --------------------------
// Its workspace is this file-scope device array: each device the library runs
// on holds one copy, at its own address, from the first call on that device
// until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: the per-device address comes from
// hipGetSymbolAddress and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[DELTAKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device, looked up once per device.
deltakv_status scratch_of_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DELTAKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DELTAKV_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(DELTAKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DELTAKV_OK;
}

}  // namespace

extern "C" {

deltakv_status deltakv_decode_attn_noalloc(const deltakv_shape *shape, int32_t num_q_heads,
                                           int64_t n_tokens, const void *q,
                                           const deltakv_cache *k_cache,
                                           const deltakv_mlp *k_dec,
                                           const deltakv_cache *v_cache,
                                           const deltakv_mlp *v_dec, float softmax_scale,
                                           float *out, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
    deltakv_status st = check_decode(shape, num_q_heads, n_tokens, q, k_cache, k_dec, v_cache,
                                     v_dec, softmax_scale, out, dm, kc, km, vc, vm);
    if (st != DELTAKV_OK) return st;
    const size_t need = dk::decode_ws_bytes(dm, num_q_heads, n_tokens);
    if (need > (size_t)DELTAKV_NOALLOC_SCRATCH_BYTES)
        return fail(DELTAKV_ERR_WORKSPACE,
                    "decode needs %zu bytes of scratch, more than the %zu the allocation-free "
                    "entry point holds; call deltakv_decode_attn with a workspace", need,
                    (size_t)DELTAKV_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != DELTAKV_OK) return st;
    // every region of the workspace is written by the call before it is read
    // (query tables, then partial records, then the merge), so nothing has to
    // be cleared first
    return from_hip(dk::launch_decode(dm, num_q_heads, n_tokens, q, kc, km, vc, vm,
                                      softmax_scale, out, ws,
                                      (size_t)DELTAKV_NOALLOC_SCRATCH_BYTES,
                                      (hipStream_t)stream),
                    "deltakv_decode_attn_noalloc");
}

deltakv_status deltakv_decode_attn_sparse(const deltakv_shape *shape, int32_t num_q_heads,
                                          int64_t n_tokens, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          const int32_t *positions, int32_t n_sel,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, n_tokens)) != DELTAKV_OK) return st;
    if (n_sel < 1 || n_sel > DELTAKV_MAX_SPARSE_SELECT)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_sel %d not in [1, %d]", n_sel,
                    DELTAKV_MAX_SPARSE_SELECT);
    if (!positions) return fail(DELTAKV_ERR_INVALID_ARG, "positions is NULL");
    if (!aligned16(positions))
        return fail(DELTAKV_ERR_INVALID_ARG, "positions must be 16-byte aligned");
    if (!q || !out) return fail(DELTAKV_ERR_INVALID_ARG, "q / out is NULL");
    if (!aligned16(q) || !aligned16(out))
        return fail(DELTAKV_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!std::isfinite(softmax_scale))
        return fail(DELTAKV_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((st = check_mlp(k_dec, "k_dec", dm.dc, dm.d, &km)) != DELTAKV_OK) return st;
    if ((st = check_mlp(v_dec, "v_dec", dm.dc, dm.d, &vm)) != DELTAKV_OK) return st;
    if (dm.lat_fmt && !dk::decode_q4_supported(dm, km, vm))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: decode needs k 4 or 8 and GELU "
                    "decompressors of one hidden width, 128 or 256");
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc, n_tokens)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc, n_tokens)) != DELTAKV_OK) return st;
    if (dm.pr) return fail(DELTAKV_ERR_UNSUPPORTED, "sparse decode over a paged cache");
    const size_t need = dk::decode_sparse_ws_bytes(dm, num_q_heads, n_tokens, n_sel);
    if (workspace_bytes < need || !workspace)
        return fail(DELTAKV_ERR_WORKSPACE, "sparse decode needs %zu workspace bytes, got %zu",
                    need, workspace_bytes);
    if (!aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return from_hip(dk::launch_decode_sparse(dm, num_q_heads, n_tokens, q, kc, km, vc, vm,
                                             positions, n_sel, softmax_scale, out, workspace,
                                             workspace_bytes, (hipStream_t)stream),
                    "deltakv_decode_attn_sparse");
}

deltakv_status deltakv_decode_attn_select(const deltakv_shape *shape, int32_t num_q_heads,
                                          int64_t n_tokens, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          float softmax_scale, float *out, int32_t n_keep,
                                          int32_t *positions, float *scores, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, n_tokens)) != DELTAKV_OK) return st;
    if (n_keep < 1 || n_keep > DELTAKV_MAX_SPARSE_SELECT)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_keep %d not in [1, %d]", n_keep,
                    DELTAKV_MAX_SPARSE_SELECT);
    if (!positions) return fail(DELTAKV_ERR_INVALID_ARG, "positions is NULL");
    if (!aligned16(positions) || (scores && !aligned16(scores)))
        return fail(DELTAKV_ERR_INVALID_ARG, "positions / scores must be 16-byte aligned");
    if (!q || !out) return fail(DELTAKV_ERR_INVALID_ARG, "q / out is NULL");
    if (!aligned16(q) || !aligned16(out))
        return fail(DELTAKV_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!std::isfinite(softmax_scale))
        return fail(DELTAKV_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((st = check_mlp(k_dec, "k_dec", dm.dc, dm.d, &km)) != DELTAKV_OK) return st;
    if ((st = check_mlp(v_dec, "v_dec", dm.dc, dm.d, &vm)) != DELTAKV_OK) return st;
    if (dm.lat_fmt && !dk::decode_q4_supported(dm, km, vm))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: decode needs k 4 or 8 and GELU "
                    "decompressors of one hidden width, 128 or 256");
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc, n_tokens)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc, n_tokens)) != DELTAKV_OK) return st;
    if ((st = check_paged_decode(dm, k_cache, km, v_cache, vm)) != DELTAKV_OK) return st;
    const size_t need = dk::decode_select_ws_bytes(dm, num_q_heads, n_tokens);
    if (workspace_bytes < need || !workspace)
        return fail(DELTAKV_ERR_WORKSPACE, "decode with selection needs %zu workspace bytes, "
                    "got %zu", need, workspace_bytes);
    if (!aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return from_hip(dk::launch_decode_select(dm, num_q_heads, n_tokens, q, kc, km, vc, vm,
                                             softmax_scale, out, n_keep, positions, scores,
                                             workspace, workspace_bytes, (hipStream_t)stream),
                    "deltakv_decode_attn_select");
}

deltakv_status deltakv_decode_attn_window(const deltakv_shape *shape, int32_t num_q_heads,
                                          int64_t n_tokens, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          const void *k_win, const void *v_win, int64_t n_win,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_heads_tokens(dm, num_q_heads, n_tokens)) != DELTAKV_OK) return st;
    if (n_win < 1 || n_win > 65535)
        return fail(DELTAKV_ERR_INVALID_ARG, "n_win %lld not in [1, 65535]", (long long)n_win);
    if (!k_win || !v_win) return fail(DELTAKV_ERR_INVALID_ARG, "k_win / v_win is NULL");
    if (!aligned16(k_win) || !aligned16(v_win))
        return fail(DELTAKV_ERR_INVALID_ARG, "k_win / v_win must be 16-byte aligned");
    if (!q || !out) return fail(DELTAKV_ERR_INVALID_ARG, "q / out is NULL");
    if (!aligned16(q) || !aligned16(out))
        return fail(DELTAKV_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!std::isfinite(softmax_scale))
        return fail(DELTAKV_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((st = check_mlp(k_dec, "k_dec", dm.dc, dm.d, &km)) != DELTAKV_OK) return st;
    if ((st = check_mlp(v_dec, "v_dec", dm.dc, dm.d, &vm)) != DELTAKV_OK) return st;
    if (dm.lat_fmt && !dk::decode_q4_supported(dm, km, vm))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: decode needs k 4 or 8 and GELU "
                    "decompressors of one hidden width, 128 or 256");
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc, n_tokens)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc, n_tokens)) != DELTAKV_OK) return st;
    if ((st = check_paged_decode(dm, k_cache, km, v_cache, vm)) != DELTAKV_OK) return st;
    const size_t need = dk::decode_window_ws_bytes(dm, num_q_heads, n_tokens, n_win);
    if (workspace_bytes < need || !workspace)
        return fail(DELTAKV_ERR_WORKSPACE, "decode with a window needs %zu workspace bytes, "
                    "got %zu", need, workspace_bytes);
    if (!aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return from_hip(dk::launch_decode_window(dm, num_q_heads, n_tokens, q, kc, km, vc, vm, k_win,
                                             v_win, n_win, softmax_scale, out, workspace,
                                             workspace_bytes, (hipStream_t)stream),
                    "deltakv_decode_attn_window");
}

deltakv_status deltakv_decode_attn_varlen(const deltakv_shape *shape, int32_t num_q_heads,
                                          const int64_t *lengths, int64_t max_tokens,
                                          const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if (!lengths) return fail(DELTAKV_ERR_INVALID_ARG, "lengths is NULL");
    if (reinterpret_cast<uintptr_t>(lengths) & 7u)
        return fail(DELTAKV_ERR_INVALID_ARG, "lengths must be 8-byte aligned");
    if ((st = check_heads_tokens(dm, num_q_heads, max_tokens)) != DELTAKV_OK) return st;
    if (max_tokens > DELTAKV_MAX_SPARSE_SELECT)
        return fail(DELTAKV_ERR_UNSUPPORTED, "max_tokens %lld above %d", (long long)max_tokens,
                    DELTAKV_MAX_SPARSE_SELECT);
    const int64_t nmax = max_tokens;
    if (!q || !out) return fail(DELTAKV_ERR_INVALID_ARG, "q / out is NULL");
    if (!aligned16(q) || !aligned16(out))
        return fail(DELTAKV_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!std::isfinite(softmax_scale))
        return fail(DELTAKV_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((st = check_mlp(k_dec, "k_dec", dm.dc, dm.d, &km)) != DELTAKV_OK) return st;
    if ((st = check_mlp(v_dec, "v_dec", dm.dc, dm.d, &vm)) != DELTAKV_OK) return st;
    if (dm.lat_fmt && !dk::decode_q4_supported(dm, km, vm))
        return fail(DELTAKV_ERR_UNSUPPORTED, "4-bit latents: decode needs k 4 or 8 and GELU "
                    "decompressors of one hidden width, 128 or 256");
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc, max_tokens)) != DELTAKV_OK)
        return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc, max_tokens)) != DELTAKV_OK)
        return st;
    if ((st = check_paged_decode(dm, k_cache, km, v_cache, vm)) != DELTAKV_OK) return st;
    const size_t need = dk::decode_varlen_ws_bytes(dm, num_q_heads, nmax);
    if (workspace_bytes < need || !workspace)
        return fail(DELTAKV_ERR_WORKSPACE, "mixed-length decode needs %zu workspace bytes, "
                    "got %zu", need, workspace_bytes);
    if (!aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return from_hip(dk::launch_decode_varlen(dm, num_q_heads, lengths, nmax, q, kc, km, vc, vm,
                                             softmax_scale, out, workspace, workspace_bytes,
                                             (hipStream_t)stream),
                    "deltakv_decode_attn_varlen");
}

deltakv_status deltakv_peak_probe(int32_t kind, int32_t blocks, int32_t iters, float *sink,
                                  void *stream) {
    if (kind != DELTAKV_PEAK_MFMA_BF16 && kind != DELTAKV_PEAK_GELU_F16)
        return fail(DELTAKV_ERR_INVALID_ARG, "probe kind %d unknown", kind);
    if (blocks < 1 || iters < 1 || !sink)
        return fail(DELTAKV_ERR_INVALID_ARG, "probe needs blocks >= 1, iters >= 1 and a sink");
    const hipError_t e = kind == DELTAKV_PEAK_MFMA_BF16
                             ? dk::launch_peak_mfma(blocks, iters, sink, (hipStream_t)stream)
                             : dk::launch_peak_gelu(blocks, iters, sink, (hipStream_t)stream);
    return from_hip(e, "deltakv_peak_probe");
}

const char *deltakv_status_string(deltakv_status status) {
    switch (status) {
        case DELTAKV_OK: return "DELTAKV_OK";
        case DELTAKV_ERR_INVALID_ARG: return "DELTAKV_ERR_INVALID_ARG";
        case DELTAKV_ERR_UNSUPPORTED: return "DELTAKV_ERR_UNSUPPORTED";
        case DELTAKV_ERR_CAPACITY: return "DELTAKV_ERR_CAPACITY";
        case DELTAKV_ERR_WORKSPACE: return "DELTAKV_ERR_WORKSPACE";
        case DELTAKV_ERR_HIP: return "DELTAKV_ERR_HIP";
    }
    return "DELTAKV_ERR_UNKNOWN";
}

const char *deltakv_last_error(void) { return g_last_error.c_str(); }

const char *deltakv_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
