/*
 * deltakv.h -- C ABI of libdeltakv.so: DeltaKV residual KV-cache compression
 * and decode attention over the compressed cache, on AMD Instinct MI355X
 * (gfx950).
 *
 * Method: "DeltaKV: Residual-Based KV Cache Compression via Long-Range
 * Similarity" (gist.science summary of arXiv 2602.08005).  Section 3
 * ("Metodologia") defines the operation; the page's section 4
 * ("Implementazione") motivates a cache manager for irregular compressed
 * layouts and kernels that reconstruct tokens on demand.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - A "unit" is one (sequence b, KV head h) of one layer and one stream (K or
 *   V).  Units are independent; a call covers the B x H units of one
 *   (layer, stream) cache.
 * - Pointers are DEVICE pointers unless a comment says "host".  The caller owns
 *   every buffer; the library keeps no allocation between calls and allocates
 *   nothing itself (scratch space is the caller's workspace argument).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *   the call returns at once.  Argument errors are returned synchronously,
 *   before anything is enqueued.  Faults inside a kernel surface at the
 *   caller's next synchronisation of the stream.
 * - Storage type (deltakv_dtype): x, reference rows, latents, MLP weights and
 *   queries all use shape->dtype; biases, squared norms and the attention
 *   output are fp32.  bf16 values are raw 16-bit bfloat16 patterns.
 * - Positions: a sequence's tokens are positions 0 .. capacity-1.  Position p
 *   is a REFERENCE token iff p % stride == 0 (reference ordinal j = p / stride;
 *   token 0 is a reference).  All other positions are compressed tokens,
 *   numbered by their "token ordinal" q in increasing position order:
 *       q = (p / s) * (s - 1) + (p % s) - 1,
 *       p = (q / (s - 1)) * s + (q % (s - 1)) + 1       (s = stride >= 2).
 *   With stride 1 every token is a reference and nothing is compressed.
 *   (section 3, "Struttura della Compressione": a small reference set at a
 *   fixed stride, residuals for the rest.)
 * - No C++ exception crosses this boundary.
 */
#ifndef DELTAKV_H
#define DELTAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DELTAKV_OK = 0,
    DELTAKV_ERR_INVALID_ARG = 1,  /* null pointer, bad range, inconsistent sizes */
    DELTAKV_ERR_UNSUPPORTED = 2,  /* a size outside the compiled set (see deltakv_shape) */
    DELTAKV_ERR_CAPACITY = 3,     /* t1 > capacity, or more references than 16-bit indices hold */
    DELTAKV_ERR_WORKSPACE = 4,    /* workspace smaller than the matching *_workspace_bytes */
    DELTAKV_ERR_HIP = 5           /* a HIP runtime call (e.g. a launch) failed */
} deltakv_status;

typedef enum { DELTAKV_F32 = 0, DELTAKV_BF16 = 1 } deltakv_dtype;

/* Storage of the latents (deltakv_shape.latent_format). */
typedef enum {
    DELTAKV_LATENT_DTYPE = 0,  /* d_c values per token in shape->dtype */
    DELTAKV_LATENT_Q4 = 1      /* 4-bit codes and a per-token shift / scale; see deltakv_cache */
} deltakv_latent_format;

typedef enum {
    DELTAKV_ACT_GELU = 0,      /* GELU, erf form: u * Phi(u) */
    DELTAKV_ACT_IDENTITY = 1   /* linear MLP (used by the exact-reconstruction check) */
} deltakv_act;

/* Sizes of one (layer, stream) cache: the quantities the method is stated in.
 * Supported: head_dim in {64, 128}; stride >= 1; 1 <= k <= 8;
 * d_c in {16, 32, 64, 128}; capacity >= 1 with ceil(capacity / stride) <= 65535
 * (reference ordinals are stored as uint16).  latent_format
 * DELTAKV_LATENT_Q4 needs bf16, d_c in {16, 32}, and calls whose MLPs are
 * GELU with hidden width 128 or 256 (the same for K and V) and k in {4, 8};
 * other calls on such a cache return UNSUPPORTED. */
typedef struct {
    int32_t batch;         /* B: sequences */
    int32_t num_kv_heads;  /* H: KV heads of the layer */
    int32_t head_dim;      /* d */
    int32_t stride;        /* s: every s-th position is a reference token */
    int32_t k;             /* references averaged per compressed token */
    int32_t d_c;           /* latent width */
    int64_t capacity;      /* maximum context length in tokens (per sequence) */
    int32_t dtype;         /* deltakv_dtype */
    int32_t latent_format; /* deltakv_latent_format (0: latents in dtype) */
} deltakv_shape;

/* A light MLP: out = W2 act(W1 in + b1) + b2 (section 3, step 4: the
 * Compressor maps d -> d_c; "Ricostruzione": the Decompressor maps d_c -> d).
 * Weights row-major [out][in] in shape->dtype; biases fp32 or NULL (= zero).
 * Supported hidden widths: 64, 128, 256.  Read-only. */
typedef struct {
    const void *w1;      /* [hidden][in_dim] */
    const float *b1;     /* [hidden] or NULL */
    const void *w2;      /* [out_dim][hidden] */
    const float *b2;     /* [out_dim] or NULL */
    int32_t in_dim;
    int32_t hidden;
    int32_t out_dim;
    int32_t act;         /* deltakv_act */
} deltakv_mlp;

/* Compressed cache of one (layer, stream), structure of arrays.  With
 * R = ceil(capacity / stride) and N = capacity - R:
 *   refs        [B][H][R][d]     reference rows, verbatim copies of the input
 *   ref_sqnorm  [B][H][R]        fp32 squared L2 norm of each reference row
 *   latents     [B][H][N][d_c]   Compressor outputs, by token ordinal
 *               (DELTAKV_LATENT_Q4: per unit, N rows of d_c / 2 bytes of 4-bit
 *               codes, two per byte, the lower latent index in the low
 *               nibble, then N 32-bit words holding the row's bf16 shift (low
 *               half) and bf16 scale (high half).  The Compressor output z,
 *               rounded to bf16, is stored as shift = min(z), scale =
 *               bf16((max(z) - min(z)) * fp32(1/15)), code = clamp(rint((z -
 *               shift) * (1 / scale)), 0, 15) in fp32 arithmetic, the
 *               reciprocal correctly rounded (scale 0: codes 0); the decode
 *               reads shift + code * scale.  This is the 4-bit latent
 *               storage that the DeltaKV page's section 5 quotes its memory
 *               figure with; the page gives no format.)
 *   idx         [B][H][N][k]     reference ordinals averaged into KV_R, nearest
 *                                first; 0xFFFF marks an unused slot (a token at
 *                                position p has min(k, ceil(p / s)) candidates)
 * deltakv_cache_bytes gives the byte size of each array.  The caller allocates
 * them; the library reads and writes them in place. */
typedef struct {
    void *refs;
    float *ref_sqnorm;
    void *latents;
    uint16_t *idx;
} deltakv_cache;

/* Host-only.  Byte sizes of the four cache arrays for `shape` (any output
 * pointer may be NULL).  Returns INVALID_ARG / UNSUPPORTED / CAPACITY for a
 * shape the other entry points would reject. */
deltakv_status deltakv_cache_bytes(const deltakv_shape *shape, size_t *refs_bytes,
                                   size_t *ref_sqnorm_bytes, size_t *latents_bytes,
                                   size_t *idx_bytes);

/* Host-only.  Workspace that deltakv_compress needs for positions [t0, t1). */
deltakv_status deltakv_compress_workspace_bytes(const deltakv_shape *shape, int64_t t0,
                                                int64_t t1, size_t *bytes);

/* Host-only.  Workspace that deltakv_decode_attn needs for num_q_heads query
 * heads over n_tokens cached tokens. */
deltakv_status deltakv_decode_workspace_bytes(const deltakv_shape *shape, int32_t num_q_heads,
                                              int64_t n_tokens, size_t *bytes);

/* Reference-set build (section 3, "Struttura della Compressione"): for every
 * reference position p in [t0, t1), copy the input row into refs[p / s] and
 * store its fp32 squared norm.
 *   x: [B][H][t1 - t0][d], row i holding position t0 + i (read-only).
 * Requires 0 <= t0 < t1 <= capacity.  Streaming callers call it chunk by chunk
 * (t0 = previous t1); one call with t0 = 0, t1 = T builds an offline prefix. */
deltakv_status deltakv_build_refs(const deltakv_shape *shape, const void *x, int64_t t0,
                                  int64_t t1, const deltakv_cache *cache, void *stream);

/* Compression of the non-reference positions in [t0, t1) (section 3,
 * "Processo di Compressione", steps 1-4):
 *   1. among the reference ordinals j with j * s < p, pick the k nearest to
 *      x_p by L2 distance; distances are ranked exactly (fp64, coordinates
 *      summed in order, no fused multiply-add) with equal distances ordered by
 *      the lower ordinal; write them to idx, nearest first;
 *   2. KV_R = mean of those k_eff = min(k, ceil(p / s)) reference rows;
 *   3. residual = x_p - KV_R;
 *   4. latents[q(p)] = compressor(residual).
 * x: as for deltakv_build_refs.  Precondition: deltakv_build_refs has covered
 * positions [0, t1) (earlier chunks included) and its work is ordered before
 * this call on `stream`.  compressor: in_dim = d, out_dim = d_c.
 * workspace: device scratch of deltakv_compress_workspace_bytes(shape, t0, t1).
 * stats: NULL or a device uint32 to which the number of tokens whose
 * selection needed the exhaustive fallback scan is added atomically. */
deltakv_status deltakv_compress(const deltakv_shape *shape, const void *x, int64_t t0,
                                int64_t t1, const deltakv_mlp *compressor,
                                const deltakv_cache *cache, void *workspace,
                                size_t workspace_bytes, uint32_t *stats, void *stream);

/* Decode attention over the compressed cache ("Ricostruzione" in section 3,
 * with textbook softmax attention): for every query head g of sequence b,
 * with KV head h = g / (num_q_heads / H),
 *   out[b][g] = sum_t softmax_t(scale * q[b][g] . K^_t) V^_t,   t = 0..n_tokens-1,
 * where a reference position's K^/V^ is its stored row and a compressed
 * token's is KV_R (mean of its idx rows) + decompressor(latent).
 *   q:   [B][num_q_heads][d] in shape->dtype;  out: [B][num_q_heads][d] fp32.
 *   k_dec / v_dec: in_dim = d_c, out_dim = d.
 * num_q_heads must be a multiple of H with num_q_heads / H <= 8; 1 <= n_tokens
 * <= capacity and every position < n_tokens must have been built and
 * compressed.  workspace: deltakv_decode_workspace_bytes(shape, num_q_heads,
 * n_tokens) bytes. */
deltakv_status deltakv_decode_attn(const deltakv_shape *shape, int32_t num_q_heads,
                                   int64_t n_tokens, const void *q,
                                   const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                   const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                   float softmax_scale, float *out, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* Largest position list per (sequence, KV head) that the sparse decode takes. */
#define DELTAKV_MAX_SPARSE_SELECT 1048576

/* Host-only.  Workspace that deltakv_decode_attn_sparse needs for num_q_heads
 * query heads over n_tokens cached tokens and lists of n_sel positions. */
deltakv_status deltakv_decode_sparse_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t n_tokens,
                                                     int32_t n_sel, size_t *bytes);

/* Decode attention with on-demand reconstruction of selected tokens only
 * (section 4, "Implementazione: Sparse-vLLM": the kernels rebuild a
 * compressed token only when a sparse attention selects it, e.g. a
 * query-aware selector of the OmniKV kind).  The selector is the caller's:
 *   positions: device int32 [B][H][n_sel], read-only, the caller's buffer.
 *              Row (b, h) lists the positions that the query heads of KV head
 *              h of sequence b attend to, in any order.  Entries outside
 *              [0, n_tokens) are skipped (padding for shorter lists); an entry
 *              listed twice takes part twice.
 * For each query head g of KV head h,
 *   out[b][g] = sum_{t in list} softmax_t(scale * q[b][g] . K^_t) V^_t
 * with K^/V^ rebuilt exactly as deltakv_decode_attn rebuilds them; a list
 * with no valid entry gives a zero output row.  Listing every position
 * 0..n_tokens-1 gives deltakv_decode_attn's result.  Other arguments, their
 * layouts and requirements are as for deltakv_decode_attn; 1 <= n_sel <=
 * DELTAKV_MAX_SPARSE_SELECT; workspace: deltakv_decode_sparse_workspace_bytes
 * (the split position lists are kept there, so it must not be shared with a
 * call still in flight). */
deltakv_status deltakv_decode_attn_sparse(const deltakv_shape *shape, int32_t num_q_heads,
                                          int64_t n_tokens, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          const int32_t *positions, int32_t n_sel,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream);

/* Host-only.  Workspace that deltakv_decode_attn_window needs. */
deltakv_status deltakv_decode_window_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t n_tokens,
                                                     int64_t n_win, size_t *bytes);

/* Decode attention over the compressed cache plus n_win exact rows kept
 * beside it: a recent window of tokens not yet compressed, or attention sinks
 * kept verbatim (rows the method's reference set does not hold).  For each
 * query head g of KV head h,
 *   out[b][g] = sum over the n_tokens rebuilt tokens and the n_win rows of
 *               softmax(scale * q . K) V,
 * the cache part exactly as deltakv_decode_attn rebuilds it, the window part
 * with the given rows.
 *   k_win, v_win: [B][H][n_win][d] in shape->dtype, read-only.
 * 1 <= n_win <= 65535; other arguments as for deltakv_decode_attn; workspace:
 * deltakv_decode_window_workspace_bytes.  (The two parts run as two decode
 * passes whose outputs are merged by their log-sum-exp.) */
deltakv_status deltakv_decode_attn_window(const deltakv_shape *shape, int32_t num_q_heads,
                                          int64_t n_tokens, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          const void *k_win, const void *v_win, int64_t n_win,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream);

/* Host-only.  Workspace that deltakv_decode_attn_varlen needs when the
 * longest sequence holds max_tokens tokens. */
deltakv_status deltakv_decode_varlen_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t max_tokens,
                                                     size_t *bytes);

/* Decode attention over a batch whose sequences hold different numbers of
 * tokens (a serving batch of mixed lengths): sequence b attends its positions
 * 0 .. lengths[b] - 1, each rebuilt as deltakv_decode_attn rebuilds it.
 *   lengths: HOST int64 [B], 1 <= lengths[b] <= capacity, read during the
 *            call (copied to the workspace on `stream`).
 * Positions at or past a sequence's length may hold anything.  Other
 * arguments as for deltakv_decode_attn; max(lengths) <=
 * DELTAKV_MAX_SPARSE_SELECT; workspace: deltakv_decode_varlen_workspace_bytes
 * with max_tokens = max(lengths).  (Runs as the sparse decode over every
 * position below each sequence's length.) */
deltakv_status deltakv_decode_attn_varlen(const deltakv_shape *shape, int32_t num_q_heads,
                                          const int64_t *lengths, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream);

/* Host-only.  Workspace that deltakv_decode_attn_select needs for num_q_heads
 * query heads over n_tokens cached tokens. */
deltakv_status deltakv_decode_select_workspace_bytes(const deltakv_shape *shape,
                                                     int32_t num_q_heads, int64_t n_tokens,
                                                     size_t *bytes);

/* Dense decode attention that also picks the tokens for sparse attention at
 * later steps or layers: the query-aware selector that section 4 pairs with
 * on-demand reconstruction (OmniKV in its example: a filter layer's full
 * attention chooses the tokens the other layers attend to).  out is written
 * exactly as deltakv_decode_attn writes it.  For each (b, h), with G =
 * num_q_heads / H query heads g of KV head h:
 *   score_p = sum_g softmax_p(scale * q[b][g] . K^_p),   p = 0..n_tokens-1
 * (the attention probability of position p, summed over the group), and
 *   positions [B][H][n_keep] (device int32, written): the n_keep positions of
 *       largest score, equal scores ordered by the lower position, listed in
 *       increasing position order; if n_keep >= n_tokens every position
 *       0..n_tokens-1, then -1.  A valid list for deltakv_decode_attn_sparse
 *       with n_sel = n_keep.
 *   scores [B][H][n_tokens] (device fp32, written; may be NULL): score_p.
 * The scores come from the logits the attention itself uses (the bf16 path's
 * approximations included); the ranking of those fp32 scores is exact.
 * 1 <= n_keep <= DELTAKV_MAX_SPARSE_SELECT; other arguments as for
 * deltakv_decode_attn; workspace: deltakv_decode_select_workspace_bytes. */
deltakv_status deltakv_decode_attn_select(const deltakv_shape *shape, int32_t num_q_heads,
                                          int64_t n_tokens, const void *q,
                                          const deltakv_cache *k_cache, const deltakv_mlp *k_dec,
                                          const deltakv_cache *v_cache, const deltakv_mlp *v_dec,
                                          float softmax_scale, float *out, int32_t n_keep,
                                          int32_t *positions, float *scores, void *workspace,
                                          size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string). */
const char *deltakv_status_string(deltakv_status status);

/* Detail of the last failing call on the calling thread ("" if none). */
const char *deltakv_last_error(void);

/* Library version string, e.g. "0.1.0 gfx950". */
const char *deltakv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTAKV_H */
