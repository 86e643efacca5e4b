// dk_mfma.h -- CDNA4 (gfx950) matrix-core helpers and packed-f16 activation.
//
// Operand layouts of the two 16x16x32 MFMA forms used here (checked on the
// hardware): for lane l of a wave64,
//   A (16 x 32, row-major M x K): lane holds A[l % 16][8 * (l / 16) + i], i = 0..7
//   B (32 x 16, K x N):           lane holds B[8 * (l / 16) + i][l % 16]
//   C (16 x 16):                  lane holds C[4 * (l / 16) + r][l % 16], r = 0..3
// The 16x16x16 f16 form has the same pattern with four K values per lane:
//   A: lane holds A[l % 16][4 * (l / 16) + i], B: B[4 * (l / 16) + i][l % 16], i = 0..3.
// and for the 32x32x16 form:
//   A (32 x 16): lane holds A[l % 32][8 * (l / 32) + i]
//   B (16 x 32): lane holds B[8 * (l / 32) + i][l % 32]
//   C (32 x 32): lane holds C[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32], r = 0..15
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16_f16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, let M[i] be the four 16-bit values at lane i's 8-byte address; lane j
// receives {M[4e + j/4][j%4] : e = 0..3} (checked on the hardware).  Two such
// reads build an MFMA operand column slice: with lane i pointing at row
// (base + i/4), columns (4 (i%4) .. +3) of a row-major tile, lane j gets rows
// base .. base+3 of column j.
__device__ __forceinline__ u32x2 lds_read_tr16(const void *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Wait until every vector memory operation of the wave has completed (loads
// into registers and global -> LDS copies).  Written as the builtin, not as
// inline assembly, so the compiler's own wait-count tracking knows that
// nothing is outstanding afterwards and adds no waits of its own.
// gfx9 encoding: vmcnt = 0, expcnt and lgkmcnt left at their maximum.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// base + a 32-bit byte offset.  Written with the offset already in bytes and
// unsigned 32-bit, so the compiler can use the scalar-base + 32-bit vector
// offset addressing form (and fold constant offsets into the instruction)
// instead of 64-bit per-lane address arithmetic.
template <typename T>
__device__ __forceinline__ const T *at_byte(const T *base, uint32_t off) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off);
}

// 16-byte global load of 8 consecutive 16-bit values (pointer 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Two fp32 values -> packed bf16, round to nearest even (gfx950's
// v_cvt_pk_bf16_f32: one instruction).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Two fp32 values -> packed f16 (round toward zero; one instruction).
__device__ __forceinline__ f16x2 pack_f16(float a, float b) {
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// GELU of two fp32 pre-activations, evaluated in packed f16:
//   GELU(u) = u * Phi(u),   Phi(u) ~= clamp01(0.5 + u * Q(u * u)),
// where Q is a degree-4 polynomial fitted (least squares with reweighting
// toward the maximum error) to the standard normal CDF on |u| <= 3.5.  Its
// leading coefficient is positive, so beyond the fitted range the clamp
// saturates Phi to 0 or 1.  The largest error of Phi over the real line is
// below 9e-4 before f16 rounding, and of GELU after it below
// 2.8e-3 * max(1, |u|).  8 packed instructions per pair.  Used only on the
// bf16 decode path, where the hidden activations feed f16 matrix products.
__device__ __forceinline__ f16x2 gelu2_f16(float a, float b) {
    const f16x2 u = pack_f16(a, b);
    const f16x2 half = {(_Float16)0.5f, (_Float16)0.5f};
    const f16x2 t = u * u;
    const f16x2 c4 = {(_Float16)1.20540652e-05f, (_Float16)1.20540652e-05f};
    const f16x2 c3 = {(_Float16)-4.59953350e-04f, (_Float16)-4.59953350e-04f};
    const f16x2 c2 = {(_Float16)7.16798242e-03f, (_Float16)7.16798242e-03f};
    const f16x2 c1 = {(_Float16)-6.16098042e-02f, (_Float16)-6.16098042e-02f};
    const f16x2 c0 = {(_Float16)3.96455769e-01f, (_Float16)3.96455769e-01f};
    f16x2 p = __builtin_elementwise_fma(c4, t, c3);
    p = __builtin_elementwise_fma(p, t, c2);
    p = __builtin_elementwise_fma(p, t, c1);
    p = __builtin_elementwise_fma(p, t, c0);
    f16x2 phi;
    asm("v_pk_fma_f16 %0, %1, %2, %3 clamp" : "=v"(phi) : "v"(u), "v"(p), "v"(half));
    return u * phi;
}

// Two GELU pairs at once (the same polynomial as gelu2_f16), written so that
// the two packed chains interleave: each step issues both pairs' instruction
// before either result is needed.
__device__ __forceinline__ void gelu4_f16(float a, float b, float c, float d, f16x2 &r0,
                                          f16x2 &r1) {
    const f16x2 u0 = pack_f16(a, b), u1 = pack_f16(c, d);
    const f16x2 half = {(_Float16)0.5f, (_Float16)0.5f};
    const f16x2 c4 = {(_Float16)1.20540652e-05f, (_Float16)1.20540652e-05f};
    const f16x2 c3 = {(_Float16)-4.59953350e-04f, (_Float16)-4.59953350e-04f};
    const f16x2 c2 = {(_Float16)7.16798242e-03f, (_Float16)7.16798242e-03f};
    const f16x2 c1 = {(_Float16)-6.16098042e-02f, (_Float16)-6.16098042e-02f};
    const f16x2 c0 = {(_Float16)3.96455769e-01f, (_Float16)3.96455769e-01f};
    const f16x2 t0 = u0 * u0, t1 = u1 * u1;
    f16x2 p0 = __builtin_elementwise_fma(c4, t0, c3);
    f16x2 p1 = __builtin_elementwise_fma(c4, t1, c3);
    p0 = __builtin_elementwise_fma(p0, t0, c2);
    p1 = __builtin_elementwise_fma(p1, t1, c2);
    p0 = __builtin_elementwise_fma(p0, t0, c1);
    p1 = __builtin_elementwise_fma(p1, t1, c1);
    p0 = __builtin_elementwise_fma(p0, t0, c0);
    p1 = __builtin_elementwise_fma(p1, t1, c0);
    f16x2 phi0, phi1;
    asm("v_pk_fma_f16 %0, %2, %3, %6 clamp\n\tv_pk_fma_f16 %1, %4, %5, %6 clamp"
        : "=&v"(phi0), "=v"(phi1)
        : "v"(u0), "v"(p0), "v"(u1), "v"(p1), "v"(half));
    r0 = u0 * phi0;
    r1 = u1 * phi1;
}

// Two GELU pairs with a shorter polynomial: Phi(u) ~= clamp01(0.5 + u *
// Q2(u * u)) with Q2 of degree 2 (minimax fit of the clamped form over the
// real line, |u| <= 2.63 fitted, beyond it the positive leading coefficient
// saturates Phi).  Largest error of Phi below 4.3e-3 before f16 rounding and
// 5.2e-3 after it; of GELU below 5.5e-3 * max(1, |u|).  6 packed instructions
// per pair.  Used for the value-side hidden units, whose errors enter the
// output linearly (the scores, which are exponentiated, keep gelu4_f16).
__device__ __forceinline__ void gelu4_f16_short(float a, float b, float c, float d, f16x2 &r0,
                                                f16x2 &r1) {
    const f16x2 u0 = pack_f16(a, b), u1 = pack_f16(c, d);
    const f16x2 half = {(_Float16)0.5f, (_Float16)0.5f};
    const f16x2 c2 = {(_Float16)2.95325e-03f, (_Float16)2.95325e-03f};
    const f16x2 c1 = {(_Float16)-4.881304e-02f, (_Float16)-4.881304e-02f};
    const f16x2 c0 = {(_Float16)3.8647556e-01f, (_Float16)3.8647556e-01f};
    const f16x2 t0 = u0 * u0, t1 = u1 * u1;
    f16x2 p0 = __builtin_elementwise_fma(c2, t0, c1);
    f16x2 p1 = __builtin_elementwise_fma(c2, t1, c1);
    p0 = __builtin_elementwise_fma(p0, t0, c0);
    p1 = __builtin_elementwise_fma(p1, t1, c0);
    f16x2 phi0, phi1;
    asm("v_pk_fma_f16 %0, %2, %3, %6 clamp\n\tv_pk_fma_f16 %1, %4, %5, %6 clamp"
        : "=&v"(phi0), "=v"(phi1)
        : "v"(u0), "v"(p0), "v"(u1), "v"(p1), "v"(half));
    r0 = u0 * phi0;
    r1 = u1 * phi1;
}

}  // namespace dk
