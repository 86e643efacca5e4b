// api.cpp -- the C ABI of libdeltakv.so (declared in include/deltakv.h):
// argument validation, cache / workspace sizing and dispatch to the kernel
// launchers.  Validation happens before any HIP call, so every error that an
// argument can cause is returned synchronously and without a device.
#include "deltakv.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "dk_common.h"
#include "dk_launch.h"

namespace {

thread_local std::string g_last_error;

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

deltakv_status check_cache(const deltakv_cache *c, const dk::Dims &dm, const char *name,
                           bool need_tokens, dk::CacheArgs *a) {
    if (!c) return fail(DELTAKV_ERR_INVALID_ARG, "%s is NULL", name);
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
    if (refs_bytes) *refs_bytes = units * dm.R * dm.d * elt_bytes(dm);
    if (ref_sqnorm_bytes) *ref_sqnorm_bytes = units * dm.R * sizeof(float);
    if (latents_bytes) *latents_bytes = units * (size_t)dk::lat_unit_bytes(dm);
    if (idx_bytes) *idx_bytes = units * dm.N * dm.k * sizeof(uint16_t);
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
                                  int64_t t1, const deltakv_cache *cache, void *stream) {
    dk::Dims dm;
    dk::CacheArgs ca;
    deltakv_status st = check_shape(shape, &dm);
    if (st != DELTAKV_OK) return st;
    if ((st = check_range(dm, t0, t1)) != DELTAKV_OK) return st;
    if (!x) return fail(DELTAKV_ERR_INVALID_ARG, "x is NULL");
    if (!aligned16(x)) return fail(DELTAKV_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if ((st = check_cache(cache, dm, "cache", false, &ca)) != DELTAKV_OK) return st;
    return from_hip(dk::launch_build_refs(dm, x, t0, t1, ca, (hipStream_t)stream),
                    "deltakv_build_refs");
}

deltakv_status deltakv_compress(const deltakv_shape *shape, const void *x, int64_t t0,
                                int64_t t1, const deltakv_mlp *compressor,
                                const deltakv_cache *cache, void *workspace,
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
    const size_t need = dk::compress_ws_bytes(dm, t0, t1);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(DELTAKV_ERR_WORKSPACE, "compress needs %zu workspace bytes, got %zu", need,
                    workspace_bytes);
    if (workspace && !aligned16(workspace))
        return fail(DELTAKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (dk::toks_upto(t1, dm.s) == dk::toks_upto(t0, dm.s)) return ok();  // only references
    return from_hip(dk::launch_compress(dm, x, t0, t1, ma, ca, workspace, workspace_bytes, stats,
                                        (hipStream_t)stream),
                    "deltakv_compress");
}

deltakv_status deltakv_decode_attn(const deltakv_shape *shape, int32_t num_q_heads,
                                   int64_t n_tokens, const void *q,
                                   const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                   const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                   float softmax_scale, float *out, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    dk::Dims dm;
    dk::CacheArgs kc, vc;
    dk::MlpArgs km, vm;
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
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc)) != DELTAKV_OK) return st;
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
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc)) != DELTAKV_OK) return st;
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
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc)) != DELTAKV_OK) return st;
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
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc)) != DELTAKV_OK) return st;
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
                                          const int64_t *lengths, const void *q,
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
    int64_t nmax = 0;
    for (int b = 0; b < dm.B; ++b) {
        if (lengths[b] < 1 || lengths[b] > dm.cap)
            return fail(lengths[b] > dm.cap ? DELTAKV_ERR_CAPACITY : DELTAKV_ERR_INVALID_ARG,
                        "lengths[%d] = %lld not in [1, capacity %lld]", b,
                        (long long)lengths[b], (long long)dm.cap);
        nmax = std::max(nmax, lengths[b]);
    }
    if ((st = check_heads_tokens(dm, num_q_heads, nmax)) != DELTAKV_OK) return st;
    if (nmax > DELTAKV_MAX_SPARSE_SELECT)
        return fail(DELTAKV_ERR_UNSUPPORTED, "longest sequence %lld above %d", (long long)nmax,
                    DELTAKV_MAX_SPARSE_SELECT);
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
    if ((st = check_cache(k_cache, dm, "k_cache", true, &kc)) != DELTAKV_OK) return st;
    if ((st = check_cache(v_cache, dm, "v_cache", true, &vc)) != DELTAKV_OK) return st;
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
