/*
 * deltakv_oracle.c -- plain, slow CPU oracle for DeltaKV residual KV-cache
 * compression and decode attention over the compressed cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU path is
 * compared against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  The product library never links it and
 * shares no source with it.
 *
 * Source of the method: the page "DeltaKV: Residual-Based KV Cache Compression
 * via Long-Range Similarity" (gist.science summary of arXiv 2602.08005),
 * section 3 ("Metodologia"), which states:
 *   - a small set of reference tokens is kept at a fixed stride, and only the
 *     remaining tokens are compressed (paragraph "Struttura della Compressione");
 *   - compression of a token: pick the k most similar earlier tokens from the
 *     strided reference set by L2 distance (step 1), average them into KV_R
 *     (step 2), subtract KV_R from the token to get the residual (step 3), and
 *     map the residual through a light MLP "Compressor" to d_c dimensions
 *     (step 4);
 *   - reconstruction adds the Decompressor output to the mean of the
 *     references (paragraph "Ricostruzione").
 * Attention over the rebuilt cache is the textbook softmax attention.
 *
 * Readings taken where the page is silent (each is listed with its reason in
 * the design notes of the repository):
 *   R1  reference positions are p = j*s (j = 0, 1, ...); token 0 is a reference;
 *   R2  "earlier" means: candidate references of the token at position t are
 *       the j with j*s < t;
 *   R3  with fewer than k candidates the mean runs over the k_eff = min(k, n)
 *       that exist; unused index slots hold -1 here (0xFFFF in the GPU layout);
 *   R4  ranking is by squared L2 distance, summed in double precision strictly
 *       in coordinate order with no fused multiply-add; equal distances are
 *       ordered by the lower reference ordinal (lower position);
 *   R5  the MLP is Linear -> activation -> Linear with biases; the activation
 *       is GELU in its exact erf form, or the identity;
 *   R6  attention scale is a caller-given scalar (1/sqrt(head_dim) by default);
 *       reference tokens take part in attention with their exact values.
 *
 * Everything is fp64.  Inputs that the GPU stores in bf16 or fp32 are passed
 * here already widened to double (the widening is exact).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (see build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ACT_GELU 0
#define ORACLE_ACT_IDENTITY 1

/* Number of reference tokens among positions 0..T-1 under reading R1. */
int64_t oracle_num_refs(int64_t T, int32_t s) {
    if (T <= 0) return 0;
    return (T + s - 1) / s;
}

/* Reference set (section 3, "Struttura della Compressione"): the rows at
 * positions 0, s, 2s, ... copied verbatim.  x is T x d, refs receives
 * ceil(T/s) x d. */
void oracle_build_refs(const double *x, int64_t T, int32_t d, int32_t s,
                       double *refs) {
    int64_t n = oracle_num_refs(T, s);
    for (int64_t j = 0; j < n; ++j)
        for (int32_t i = 0; i < d; ++i)
            refs[j * d + i] = x[(j * s) * d + i];
}

/* Squared L2 distance under reading R4: plain left-to-right double sum of
 * squared coordinate differences.  The build uses -ffp-contract=off, so the
 * product and the sum are separately rounded. */
double oracle_sq_dist(const double *a, const double *b, int32_t d) {
    double acc = 0.0;
    for (int32_t i = 0; i < d; ++i) {
        double diff = a[i] - b[i];
        double sq = diff * diff;
        acc = acc + sq;
    }
    return acc;
}

/* Step 1 of section 3: for each requested token (its row in xt, its position
 * in pos[]), the k nearest references among the candidates j with j*s < pos.
 * Results go to idx (n_tok x k), nearest first; slots beyond k_eff hold -1.
 * Ordering: by distance, then by the lower ordinal (R4).  The search is a
 * k-fold minimum scan over all candidates, which is slow and easy to check.
 * Returns 0, or -1 if some position needs more references than n_refs holds
 * or is itself a reference position. */
int oracle_select(const double *xt, const int64_t *pos, int64_t n_tok,
                  const double *refs, int64_t n_refs, int32_t d, int32_t s,
                  int32_t k, int32_t *idx) {
    double *dist = (double *)malloc(sizeof(double) * (size_t)(n_refs > 0 ? n_refs : 1));
    unsigned char *taken = (unsigned char *)malloc((size_t)(n_refs > 0 ? n_refs : 1));
    if (!dist || !taken) { free(dist); free(taken); return -2; }
    int status = 0;
    for (int64_t q = 0; q < n_tok; ++q) {
        int64_t t = pos[q];
        if (t <= 0 || t % s == 0) { status = -1; break; }
        int64_t n_cand = (t + s - 1) / s; /* j*s < t  <=>  j < ceil(t/s) */
        if (n_cand > n_refs) { status = -1; break; }
        const double *x = xt + q * d;
        for (int64_t j = 0; j < n_cand; ++j) {
            dist[j] = oracle_sq_dist(x, refs + j * d, d);
            taken[j] = 0;
        }
        int32_t k_eff = (int32_t)(n_cand < k ? n_cand : k);
        for (int32_t r = 0; r < k; ++r) {
            if (r >= k_eff) { idx[q * k + r] = -1; continue; }
            int64_t best = -1;
            for (int64_t j = 0; j < n_cand; ++j) {
                if (taken[j]) continue;
                /* strict '<' keeps the lower j among equal distances */
                if (best < 0 || dist[j] < dist[best]) best = j;
            }
            taken[best] = 1;
            idx[q * k + r] = (int32_t)best;
        }
    }
    free(dist);
    free(taken);
    return status;
}

/* The erf-form GELU (reading R5): u * Phi(u) with Phi the standard normal CDF. */
double oracle_gelu(double u) {
    return 0.5 * u * (1.0 + erf(u / sqrt(2.0)));
}

/* Light MLP (section 3, step 4 and "Ricostruzione"): out = W2 act(W1 in + b1) + b2.
 * in: n x din, w1: dh x din (row-major, out x in), b1: dh (NULL means zero),
 * w2: dout x dh, b2: dout (NULL means zero), out: n x dout. */
void oracle_mlp(const double *in, int64_t n, int32_t din, int32_t dh,
                int32_t dout, const double *w1, const double *b1,
                const double *w2, const double *b2, int32_t act, double *out) {
    double *hid = (double *)malloc(sizeof(double) * (size_t)dh);
    for (int64_t r = 0; r < n; ++r) {
        const double *v = in + r * din;
        for (int32_t o = 0; o < dh; ++o) {
            double acc = 0.0;
            for (int32_t i = 0; i < din; ++i) acc += w1[(int64_t)o * din + i] * v[i];
            if (b1) acc += b1[o];
            hid[o] = (act == ORACLE_ACT_GELU) ? oracle_gelu(acc) : acc;
        }
        for (int32_t o = 0; o < dout; ++o) {
            double acc = 0.0;
            for (int32_t i = 0; i < dh; ++i) acc += w2[(int64_t)o * dh + i] * hid[i];
            if (b2) acc += b2[o];
            out[r * dout + o] = acc;
        }
    }
    free(hid);
}

/* Step 2 of section 3: KV_R of one token = mean of the references its index
 * row names (k_eff of them, reading R3).  Returns k_eff. */
int32_t oracle_ref_mean(const double *refs, const int32_t *idx_row, int32_t k,
                        int32_t d, double *kvr) {
    int32_t k_eff = 0;
    for (int32_t i = 0; i < d; ++i) kvr[i] = 0.0;
    for (int32_t r = 0; r < k; ++r) {
        int32_t j = idx_row[r];
        if (j < 0) continue;
        ++k_eff;
        for (int32_t i = 0; i < d; ++i) kvr[i] += refs[(int64_t)j * d + i];
    }
    if (k_eff > 0)
        for (int32_t i = 0; i < d; ++i) kvr[i] /= (double)k_eff;
    return k_eff;
}

/* Steps 2-4 of section 3 for n_tok tokens whose references are already
 * chosen: KV_R (mean), residual = x - KV_R, latent = Compressor(residual).
 * kvr_out and resid_out may be NULL. */
void oracle_compress(const double *xt, int64_t n_tok, int32_t d,
                     const double *refs, const int32_t *idx, int32_t k,
                     int32_t hidden, int32_t d_c, const double *w1,
                     const double *b1, const double *w2, const double *b2,
                     int32_t act, double *latent, double *kvr_out,
                     double *resid_out) {
    double *kvr = (double *)malloc(sizeof(double) * (size_t)d);
    double *res = (double *)malloc(sizeof(double) * (size_t)d);
    for (int64_t q = 0; q < n_tok; ++q) {
        oracle_ref_mean(refs, idx + q * k, k, d, kvr);
        for (int32_t i = 0; i < d; ++i) res[i] = xt[q * d + i] - kvr[i];
        oracle_mlp(res, 1, d, hidden, d_c, w1, b1, w2, b2, act, latent + q * d_c);
        if (kvr_out) memcpy(kvr_out + q * d, kvr, sizeof(double) * (size_t)d);
        if (resid_out) memcpy(resid_out + q * d, res, sizeof(double) * (size_t)d);
    }
    free(kvr);
    free(res);
}

/* Reconstruction (section 3, "Ricostruzione") of positions 0..T-1 of one
 * head: reference positions take their stored row verbatim; every other
 * position takes mean(refs named by its index row) + Decompressor(latent).
 * latents / idx hold the non-reference tokens in increasing position order
 * (n_tok = T - ceil(T/s) rows). xhat receives T x d. */
void oracle_reconstruct(const double *refs, const double *latents,
                        const int32_t *idx, int64_t T, int32_t s, int32_t d,
                        int32_t k, int32_t d_c, int32_t hidden,
                        const double *w1, const double *b1, const double *w2,
                        const double *b2, int32_t act, double *xhat) {
    double *kvr = (double *)malloc(sizeof(double) * (size_t)d);
    double *dec = (double *)malloc(sizeof(double) * (size_t)d);
    int64_t q = 0; /* running count of non-reference positions */
    for (int64_t p = 0; p < T; ++p) {
        double *row = xhat + p * d;
        if (p % s == 0) {
            memcpy(row, refs + (p / s) * d, sizeof(double) * (size_t)d);
            continue;
        }
        oracle_ref_mean(refs, idx + q * k, k, d, kvr);
        oracle_mlp(latents + q * d_c, 1, d_c, hidden, d, w1, b1, w2, b2, act, dec);
        for (int32_t i = 0; i < d; ++i) row[i] = kvr[i] + dec[i];
        ++q;
    }
    free(kvr);
    free(dec);
}

/* On-demand reconstruction (section 4, "Implementazione: Sparse-vLLM": the
 * kernels rebuild a token only when the sparse attention asks for it): the
 * rows of the n_pos given positions, in the given order, each rebuilt exactly
 * as oracle_reconstruct rebuilds it.  Every position must lie in [0, T) of a
 * cache laid out as for oracle_reconstruct; a non-reference position p reads
 * latent / index row q = p - (number of reference positions below p) =
 * p - ((p - 1) / s + 1) (reading R1: the references below p are 0, s, 2s, ...
 * up to p - 1).  xhat receives n_pos x d. */
void oracle_reconstruct_at(const double *refs, const double *latents,
                           const int32_t *idx, const int64_t *pos, int64_t n_pos,
                           int32_t s, int32_t d, int32_t k, int32_t d_c, int32_t hidden,
                           const double *w1, const double *b1, const double *w2,
                           const double *b2, int32_t act, double *xhat) {
    double *kvr = (double *)malloc(sizeof(double) * (size_t)d);
    double *dec = (double *)malloc(sizeof(double) * (size_t)d);
    for (int64_t i = 0; i < n_pos; ++i) {
        const int64_t p = pos[i];
        double *row = xhat + i * d;
        if (p % s == 0) {
            memcpy(row, refs + (p / s) * d, sizeof(double) * (size_t)d);
            continue;
        }
        const int64_t q = p - ((p - 1) / s + 1);
        oracle_ref_mean(refs, idx + q * k, k, d, kvr);
        oracle_mlp(latents + q * d_c, 1, d_c, hidden, d, w1, b1, w2, b2, act, dec);
        for (int32_t c = 0; c < d; ++c) row[c] = kvr[c] + dec[c];
    }
    free(kvr);
    free(dec);
}

/* Textbook softmax attention of n_q query rows against T key/value rows:
 * out_g = sum_t softmax_t(scale * q_g . k_t) v_t, with the row maximum
 * subtracted before exponentiation. */
void oracle_attention(const double *q, int32_t n_q, const double *keys,
                      const double *vals, int64_t T, int32_t d, double scale,
                      double *out) {
    double *a = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int32_t g = 0; g < n_q; ++g) {
        const double *qg = q + (int64_t)g * d;
        double m = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            double dot = 0.0;
            for (int32_t i = 0; i < d; ++i) dot += qg[i] * keys[t * d + i];
            a[t] = scale * dot;
            if (a[t] > m) m = a[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            a[t] = exp(a[t] - m);
            l += a[t];
        }
        double *og = out + (int64_t)g * d;
        for (int32_t i = 0; i < d; ++i) og[i] = 0.0;
        for (int64_t t = 0; t < T; ++t)
            for (int32_t i = 0; i < d; ++i) og[i] += a[t] * vals[t * d + i];
        for (int32_t i = 0; i < d; ++i) og[i] /= l;
    }
    free(a);
}

/* Attention mass per key row, summed over a group of query rows (the score a
 * query-aware token selector ranks by; section 4 of the DeltaKV page pairs
 * on-demand reconstruction with such a selector):
 *   mass_t = sum_g softmax_t(scale * q_g . k_t),   t = 0..T-1,
 * each softmax with its row maximum subtracted.  mass receives T values. */
void oracle_group_attention_mass(const double *q, int32_t n_q, const double *keys,
                                 int64_t T, int32_t d, double scale, double *mass) {
    double *a = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int64_t t = 0; t < T; ++t) mass[t] = 0.0;
    for (int32_t g = 0; g < n_q; ++g) {
        const double *qg = q + (int64_t)g * d;
        double m = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            double dot = 0.0;
            for (int32_t i = 0; i < d; ++i) dot += qg[i] * keys[t * d + i];
            a[t] = scale * dot;
            if (a[t] > m) m = a[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            a[t] = exp(a[t] - m);
            l += a[t];
        }
        for (int64_t t = 0; t < T; ++t) mass[t] += a[t] / l;
    }
    free(a);
}
