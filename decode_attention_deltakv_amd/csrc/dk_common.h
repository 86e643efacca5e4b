// dk_common.h -- shared device/host helpers of libdeltakv (gfx950 only).
//
// Layout facts of the compressed cache (one (layer, stream), structure of
// arrays) follow from the method's fixed-stride reference set ("DeltaKV:
// Residual-Based KV Cache Compression via Long-Range Similarity", section 3,
// "Struttura della Compressione"): position p is a reference iff p % s == 0,
// and the remaining positions are numbered densely by a token ordinal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dk {

typedef uint16_t bf16_t;  // raw bfloat16 bits

constexpr uint16_t kIdxUnused = 0xFFFFu;
// Compressed-token ranges up to this length (per unit) are selected by the
// exact block-per-token scan instead of the matrix-core search.
constexpr int64_t kSmallRange = 32;
// Most blocks the reference range of one such token is split over.
constexpr int64_t kSplitMax = 64;

// ---- layout: positions, reference ordinals, token ordinals ---------------------

// Number of reference positions in [0, T).
__host__ __device__ inline int64_t refs_upto(int64_t T, int s) {
    return T <= 0 ? 0 : (T + s - 1) / s;
}
// Number of compressed (non-reference) positions in [0, T).
__host__ __device__ inline int64_t toks_upto(int64_t T, int s) {
    return T - refs_upto(T, s);
}
// Position of token ordinal q (s >= 2).
__host__ __device__ inline int64_t tok_pos(int64_t q, int s) {
    return (q / (s - 1)) * s + (q % (s - 1)) + 1;
}

// ---- paged layout ------------------------------------------------------------------
// A paged cache keeps the rows of every unit in fixed-size pages of one pool
// per array, as a paged KV cache for batched serving does: a page holds the
// rows of pr * s consecutive positions of one unit (pr reference rows and
// pr (s - 1) compressed-token rows), and a block table lists, for each unit,
// the pool page behind each of its logical pages.  Logical page lp of a unit
// covers reference ordinals [lp pr, (lp + 1) pr) and token ordinals
// [lp npp, (lp + 1) npp), npp = pr (s - 1).
constexpr int kMaxPages = 512;   // logical pages per unit (65535 references / 128 per page)

struct PageMap {
    const int32_t *tbl = nullptr;  // [units][maxp]; null: unit-contiguous arrays
    int64_t maxp = 0;              // table row length (logical pages per unit)
    int32_t lg = 0;                // log2 of the reference rows per page
    int32_t npp = 0;               // compressed-token rows per page
    int32_t npages = 0;            // pool pages: entries are clamped into [0, npages)
    uint64_t mag = 0;              // t / npp == (t mag) >> 40 for 0 <= t < 2^24
};

// Pool page behind logical page lp of `unit` (both clamped into range, so a
// bad table entry cannot move an access out of the pool).
__device__ __forceinline__ int64_t pg_page(const PageMap &pm, int64_t unit, int64_t lp) {
    lp = lp < 0 ? 0 : (lp >= pm.maxp ? pm.maxp - 1 : lp);
    const uint32_t v = (uint32_t)pm.tbl[unit * pm.maxp + lp];
    return (int64_t)(v < (uint32_t)pm.npages ? v : (uint32_t)pm.npages - 1u);
}
// Pool row of reference ordinal j of `unit`.
__device__ __forceinline__ int64_t pg_ref_row(const PageMap &pm, int64_t unit, int64_t j) {
    return (pg_page(pm, unit, j >> pm.lg) << pm.lg) + (j & (((int64_t)1 << pm.lg) - 1));
}
// Pool row of token ordinal q of `unit`.
__device__ __forceinline__ int64_t pg_tok_row(const PageMap &pm, int64_t unit, int64_t q) {
    const int64_t lp = (int64_t)(((uint64_t)q * pm.mag) >> 40);
    return pg_page(pm, unit, lp) * pm.npp + (q - lp * pm.npp);
}

// ---- scalar conversions ----------------------------------------------------------

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// The bf16 value nearest to an fp64 value, ties to the even significand,
// rounded once from fp64 (no intermediate fp32 rounding), returned as fp64:
// a bf16 value has 8 significant bits and a step of 2^-133 below 2^-126, so
// x is scaled by a power of two to put its last kept bit at 1, rounded to an
// integer (round half to even) and scaled back, all exactly.  A result past
// the largest finite bf16 converts to infinity in fp32 and bf16.
__device__ __forceinline__ double bf16_grid_f64(double x) {
    const int ex = (int)((__double_as_longlong(x) >> 52) & 0x7ff);  // biased exponent
    if (ex == 0x7ff) return x;                                       // inf / NaN
    const int step = max(ex - 1023 - 7, -133);
    return ldexp(rint(ldexp(x, -step)), step);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf2f(v); }
__device__ __forceinline__ double to_f64(float v) { return (double)v; }
__device__ __forceinline__ double to_f64(bf16_t v) { return (double)bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

// ---- activation ----------------------------------------------------------------------

// GELU in its erf form, u * Phi(u), with the device math library's erff
// (accurate to a few ulp).
__device__ __forceinline__ float gelu_erf(float u) {
    return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}

__device__ __forceinline__ float apply_act(float u, int act) {
    return act == 0 ? gelu_erf(u) : u;
}

// ---- wave helpers ----------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace dk
