// k_compress.hip -- steps 2-4 of DeltaKV compression ("DeltaKV: Residual-Based
// KV Cache Compression via Long-Range Similarity", section 3, "Processo di
// Compressione"): KV_R = mean of the chosen reference rows, residual =
// x - KV_R, latent = Compressor(residual) with the Compressor a
// Linear -> GELU -> Linear block.
//
// A block takes 16 tokens: the residual tile is formed in LDS in fp32, the
// hidden tile W1 r + b1 goes through the activation into LDS, and the latent
// W2 h + b2 is rounded to the storage type.  Weights are read through L1/L2.
#include "dk_common.h"
#include "dk_launch.h"

namespace dk {
namespace {

constexpr int kTB = 16;        // tokens per block
constexpr int kMaxD = 128;     // head_dim
constexpr int kMaxH = 256;     // hidden width

template <typename T>
__global__ __launch_bounds__(256) void compress_mlp_kernel(
    const T *__restrict__ x, int64_t t0, int64_t nrows, int s, int d, int k,
    const T *__restrict__ refs, int64_t Rcap, const uint16_t *__restrict__ idx, int64_t Ncap,
    int64_t q0, int64_t nq, const T *__restrict__ w1, const float *__restrict__ b1,
    const T *__restrict__ w2, const float *__restrict__ b2, int hid, int dc, int act,
    T *__restrict__ lat) {
    __shared__ float res[kTB][kMaxD];
    __shared__ float hsh[kTB][kMaxH];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.y;
    const int64_t qb = (int64_t)blockIdx.x * kTB;
    const int nt = (int)min((int64_t)kTB, nq - qb);

    // residual tile
    for (int i = tid; i < nt * d; i += 256) {
        const int t = i / d, c = i % d;
        const int64_t q = q0 + qb + t;
        const int64_t p = tok_pos(q, s);
        const uint16_t *ir = idx + (unit * Ncap + q) * k;
        float acc = 0.f;
        int keff = 0;
        for (int r = 0; r < k; ++r) {
            const uint16_t j = ir[r];
            if (j == kIdxUnused) continue;
            acc += to_f32(refs[(unit * Rcap + j) * d + c]);
            ++keff;
        }
        const float kvr = acc / (float)keff;
        res[t][c] = to_f32(x[(unit * nrows + (p - t0)) * d + c]) - kvr;
    }
    __syncthreads();
    // hidden tile
    for (int i = tid; i < nt * hid; i += 256) {
        const int t = i / hid, o = i % hid;
        const T *wr = w1 + (int64_t)o * d;
        float acc = b1 ? b1[o] : 0.f;
        for (int c = 0; c < d; ++c) acc += to_f32(wr[c]) * res[t][c];
        hsh[t][o] = apply_act(acc, act);
    }
    __syncthreads();
    // latent
    for (int i = tid; i < nt * dc; i += 256) {
        const int t = i / dc, o = i % dc;
        const T *wr = w2 + (int64_t)o * hid;
        float acc = b2 ? b2[o] : 0.f;
        for (int c = 0; c < hid; ++c) acc += to_f32(wr[c]) * hsh[t][c];
        lat[(unit * Ncap + q0 + qb + t) * dc + o] = from_f32<T>(acc);
    }
}

}  // namespace

// Workspace of one compress call (bf16 path): a 256-byte header holding the
// fallback counter, then one 8-byte fallback-list entry per compressed token
// of the range and unit.
size_t compress_ws_bytes(const Dims &dm, int64_t t0, int64_t t1) {
    if (dm.dtype != 1) return 0;
    const int64_t nq = toks_upto(t1, dm.s) - toks_upto(t0, dm.s);
    return 256 + (size_t)nq * dm.B * dm.H * sizeof(uint64_t);
}

hipError_t launch_compress(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                           const MlpArgs &comp, const CacheArgs &c, void *ws, size_t ws_bytes,
                           uint32_t *stats, hipStream_t st) {
    (void)ws_bytes;
    const int64_t q0 = toks_upto(t0, dm.s);
    const int64_t nq = toks_upto(t1, dm.s) - q0;
    if (nq <= 0) return hipSuccess;
    hipError_t e;
    if (dm.dtype == 1) {
        uint32_t *fcount = (uint32_t *)ws;
        uint64_t *flist = (uint64_t *)((char *)ws + 256);
        e = launch_select_mfma(dm, x, t0, t1, q0, nq, c, flist, fcount, stats, st);
    } else {
        e = launch_select_exact(dm, x, t0, t1, q0, nq, c, nullptr, nullptr, 0, st);
    }
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)((nq + kTB - 1) / kTB), (unsigned)(dm.B * dm.H));
    if (dm.dtype == 0)
        hipLaunchKernelGGL(compress_mlp_kernel<float>, grid, dim3(256), 0, st, (const float *)x,
                           t0, t1 - t0, dm.s, dm.d, dm.k, (const float *)c.refs, dm.R, c.idx,
                           dm.N, q0, nq, (const float *)comp.w1, comp.b1,
                           (const float *)comp.w2, comp.b2, comp.hidden, dm.dc, comp.act,
                           (float *)c.lat);
    else
        hipLaunchKernelGGL(compress_mlp_kernel<bf16_t>, grid, dim3(256), 0, st,
                           (const bf16_t *)x, t0, t1 - t0, dm.s, dm.d, dm.k,
                           (const bf16_t *)c.refs, dm.R, c.idx, dm.N, q0, nq,
                           (const bf16_t *)comp.w1, comp.b1, (const bf16_t *)comp.w2, comp.b2,
                           comp.hidden, dm.dc, comp.act, (bf16_t *)c.lat);
    return hipGetLastError();
}

}  // namespace dk
