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

// ---- scalar conversions ----------------------------------------------------------

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
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
