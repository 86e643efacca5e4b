// k_peaks.hip -- measured denominators for the roofline figures: a
// register-resident bf16 matrix-core loop and a packed-f16 GELU loop (the
// vector-ALU work that the decode's hidden layers spend most of their time
// in).  Not part of the method; bench.py times them beside the hot path.
#include "dk_launch.h"
#include "dk_mfma.h"

namespace dk {
namespace {

// Each wave runs `iters` rounds of 8 independent 16x16x32 bf16 products on
// register operands (8 accumulators, so every product of a round issues
// without waiting for the previous one); 16 * 16 * 32 * 2 flops each.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    u32x4 a = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    u32x4 b = {0x3f803f80u, 0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u};
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = mfma16_bf16(as_bf16x8(a), as_bf16x8(b), acc[i]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    if (s == 12345.f) sink[blockIdx.x] = s;  // keeps the loop alive, never true in practice
}

// Each lane runs `iters` rounds of four independent GELU pairs (packed f16,
// the decode's 8-instruction form).  Empty asm statements mark the inputs as
// changed and the results as used every round, so the loop holds nothing but
// the GELU instructions (no extra arithmetic to keep the compiler honest).
__global__ __launch_bounds__(256) void peak_gelu_kernel(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.25f * (float)(i - 4) + 0.001f * (float)lane;
    f16x2 r0, r1, r2, r3;
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]),
                     "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
        gelu4_f16(x[0], x[1], x[2], x[3], r0, r1);
        gelu4_f16(x[4], x[5], x[6], x[7], r2, r3);
        asm volatile("" ::"v"(r0), "v"(r1), "v"(r2), "v"(r3));
    }
    const float s = (float)r0[0] + (float)r1[1] + (float)r2[0] + (float)r3[1];
    if (s == 12345.f) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_peak_mfma(int blocks, int iters, float *sink, hipStream_t st) {
    hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    return hipGetLastError();
}

hipError_t launch_peak_gelu(int blocks, int iters, float *sink, hipStream_t st) {
    hipLaunchKernelGGL(peak_gelu_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    return hipGetLastError();
}

}  // namespace dk
