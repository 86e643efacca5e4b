// k_train.hip -- the residual rows of compressed tokens and one training step
// of a Compressor / Decompressor pair on them ("DeltaKV: Residual-Based KV
// Cache Compression via Long-Range Similarity", section 3: the residual of
// steps 2-3 of "Processo di Compressione", and the reconstruction-fidelity
// (MSE) half of "Obiettivo di Training Ibrido").
//
// Training step on n residual rows D [n][d] (all fp32):
//   A1 = D W1c^T + b1c, H1 = phi_c(A1)      Z = H1 W2c^T + b2c
//   A2 = Z W1d^T + b1d, H2 = phi_d(A2)      Y = H2 W2d^T + b2d
//   L  = mean over the n x d entries of (Y - D)^2
// then the gradient of L by backpropagation and one step of gradient descent
// with momentum (v <- mu v + g, w <- w - lr v; mu = 0 is plain descent).
// Every product is the one fp32 matrix-core kernel below (16x16x4 f32 MFMA,
// 64 x 64 output tile per block staged through LDS), with an epilogue per
// use.  The weight gradients are products over the n rows (K = n), split over
// blocks into partial sums that one update kernel adds in a fixed order, so
// the step is deterministic; a column of ones appended to the right operand
// gives the bias gradient in the same product.
#include "dk_common.h"
#include "dk_launch.h"
#include "dk_mfma.h"

#include <algorithm>

namespace dk {
namespace {

enum Epi { kEpiAct = 0, kEpiLin = 1, kEpiLoss = 2, kEpiDAct = 3, kEpiPart = 4 };

// C[m][n] = sum_k A(m, k) B(k, n), A(m, k) = A[m sam + k sak], B(k, n) =
// B[k sbk + n sbn] for n < NB and 1 for NB <= n < N; block z sums k in
// [z kchunk, (z + 1) kchunk).
struct GemmP {
    const float *A;
    int64_t sam, sak;
    const float *B;
    int64_t sbk, sbn;
    int64_t M, N, K, NB, kchunk;
    const float *bias;   // [N] or null (kEpiAct, kEpiLin, kEpiLoss)
    float *out;          // [M][ldo] (kEpiPart: [split][M][ldo])
    int64_t ldo;
    float *out2;         // kEpiAct: phi(pre) [M][ldo]
    const float *aux;    // kEpiLoss: target rows; kEpiDAct: pre-activation; [M][ldx]
    int64_t ldx;
    float scale;         // kEpiLoss: factor of the gradient rows
    float *lossp;        // kEpiLoss: one partial sum of squares per block
    int act;             // 0 GELU (erf form), 1 identity
};

__device__ __forceinline__ float act_f(float u, int act) {
    return act == 0 ? 0.5f * u * (1.f + erff(u * 0.70710678118654752f)) : u;
}
// d phi / du: Phi(u) + u phi(u) for the GELU, 1 for the identity
__device__ __forceinline__ float act_df(float u, int act) {
    return act == 0 ? 0.5f * (1.f + erff(u * 0.70710678118654752f)) +
                          u * 0.39894228040143268f * expf(-0.5f * u * u)
                    : 1.f;
}

// Four consecutive operand values from p (stride 1) when all are inside
// [0, lim) and the vector form is allowed, else one by one (out-of-range
// values 0, and `ones_from` onwards (< lim) 1: the appended column of ones).
__device__ __forceinline__ f32x4 ld4(const float *p, int64_t idx0, int64_t lim,
                                     int64_t ones_from, bool vec) {
    if (vec && idx0 + 3 < ones_from) return *reinterpret_cast<const f32x4 *>(p + idx0);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = idx0 + e;
        v[e] = i < ones_from ? p[i] : (i < lim ? 1.f : 0.f);
    }
    return v;
}

// BM x 64 output tile per 256-thread block (4 waves, each (BM / 2) x 32),
// k steps of 32 staged through LDS; the next step's operands are loaded into
// registers while the current one is multiplied.
template <int EP, int BM>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmP p) {
    constexpr int BN = 64, BK = 32, PAD = 4;
    constexpr int MI = BM / 32;                 // 16-row tiles per wave
    constexpr int NA = BM * BK / 4 / 256;       // A float4 groups per thread
    constexpr int NBG = BN * BK / 4 / 256;      // B float4 groups per thread
    __shared__ __attribute__((aligned(16))) float As[BK][BM + PAD];
    __shared__ __attribute__((aligned(16))) float Bs[BK][BN + PAD];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t m0 = (int64_t)blockIdx.x * BM, n0 = (int64_t)blockIdx.y * BN;
    const int64_t kb = (int64_t)blockIdx.z * p.kchunk;
    const int64_t ke = min(p.K, kb + p.kchunk);
    f32x4 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operand orientation (contiguous dimension) and whether 16-byte loads
    // are aligned
    const bool a_kc = p.sak == 1, b_nc = p.sbn == 1;
    const auto al16 = [](const float *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    const bool avec = al16(p.A) && ((a_kc ? p.sam : p.sak) % 4 == 0);
    const bool bvec = al16(p.B) && ((b_nc ? p.sbk : p.sbn) % 4 == 0);
    f32x4 ra[NA], rb[NBG];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int g = tid + 256 * i;
            if (a_kc) {   // rows of A, four k at a time
                const int am = g / (BK / 4), ak = 4 * (g % (BK / 4));
                const int64_t gm = m0 + am;
                ra[i] = gm < p.M ? ld4(p.A + gm * p.sam, k0 + ak, ke, ke, avec)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
            } else {      // columns of A, four m at a time
                const int ak = g / (BM / 4), am = 4 * (g % (BM / 4));
                const int64_t gk = k0 + ak;
                ra[i] = gk < ke ? ld4(p.A + gk * p.sak, m0 + am, p.M, p.M, avec)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int i = 0; i < NBG; ++i) {
            const int g = tid + 256 * i;
            if (b_nc) {   // rows of B, four n at a time (the ones column past NB)
                const int bk = g / (BN / 4), bn = 4 * (g % (BN / 4));
                const int64_t gk = k0 + bk;
                rb[i] = gk < ke ? ld4(p.B + gk * p.sbk, n0 + bn, p.N, p.NB, bvec)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
            } else {      // columns of B, four k at a time
                const int bn = g / (BK / 4), bk = 4 * (g % (BK / 4));
                const int64_t gn = n0 + bn;
                if (gn < p.NB)
                    rb[i] = ld4(p.B + gn * p.sbn, k0 + bk, ke, ke, bvec);
                else {
                    const float one = gn < p.N ? 1.f : 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) rb[i][e] = k0 + bk + e < ke ? one : 0.f;
                }
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int g = tid + 256 * i;
            if (a_kc) {
                const int am = g / (BK / 4), ak = 4 * (g % (BK / 4));
#pragma unroll
                for (int e = 0; e < 4; ++e) As[ak + e][am] = ra[i][e];
            } else {
                const int ak = g / (BM / 4), am = 4 * (g % (BM / 4));
                *reinterpret_cast<f32x4 *>(&As[ak][am]) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NBG; ++i) {
            const int g = tid + 256 * i;
            if (b_nc) {
                const int bk = g / (BN / 4), bn = 4 * (g % (BN / 4));
                *reinterpret_cast<f32x4 *>(&Bs[bk][bn]) = rb[i];
            } else {
                const int bn = g / (BK / 4), bk = 4 * (g % (BK / 4));
#pragma unroll
                for (int e = 0; e < 4; ++e) Bs[bk + e][bn] = rb[i][e];
            }
        }
    };
    if (kb < ke) load(kb);
    for (int64_t k0 = kb; k0 < ke; k0 += BK) {
        store();
        __syncthreads();
        if (k0 + BK < ke) load(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 4) {
            // 16x16x4: lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]
            const int kr = kk + (lane >> 4);
            float a[MI], b[2];
#pragma unroll
            for (int i = 0; i < MI; ++i) a[i] = As[kr][(BM / 2) * wm + 16 * i + (lane & 15)];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = Bs[kr][32 * wn + 16 * j + (lane & 15)];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // epilogue: lane l holds C[4 (l / 16) + r][l % 16] of each 16 x 16 tile
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + (BM / 2) * wm + 16 * i + 4 * (lane >> 4) + r;
                const int64_t col = n0 + 32 * wn + 16 * j + (lane & 15);
                if (row >= p.M || col >= p.N) continue;
                const float v = acc[i][j][r];
                if constexpr (EP == kEpiPart) {
                    p.out[((int64_t)blockIdx.z * p.M + row) * p.ldo + col] = v;
                } else if constexpr (EP == kEpiAct) {
                    const float pre = v + (p.bias ? p.bias[col] : 0.f);
                    p.out[row * p.ldo + col] = pre;
                    p.out2[row * p.ldo + col] = act_f(pre, p.act);
                } else if constexpr (EP == kEpiLin) {
                    p.out[row * p.ldo + col] = v + (p.bias ? p.bias[col] : 0.f);
                } else if constexpr (EP == kEpiLoss) {
                    const float e = (v + (p.bias ? p.bias[col] : 0.f)) - p.aux[row * p.ldx + col];
                    sq += e * e;
                    p.out[row * p.ldo + col] = p.scale * e;
                } else {  // kEpiDAct (in place over the pre-activation is allowed)
                    const float u = p.aux[row * p.ldx + col];
                    p.out[row * p.ldo + col] = v * act_df(u, p.act);
                }
            }
    if constexpr (EP == kEpiLoss) {
        sq = wave_sum(sq);
        if (lane == 0) red[w] = sq;
        __syncthreads();
        if (tid == 0)
            p.lossp[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

// The four layers of a step (compressor 1, 2, decompressor 1, 2): weights
// W [out][in], bias b [out], the split partial sums of [out][in + 1] (column
// in: the bias gradient), their split count, and where the layer's entries
// sit in the packed parameter vector (W row-major, then b).
struct LayerU {
    float *W;
    float *b;
    const float *part;
    bf16_t *wexp;   // bf16 copy of W after the update, or null
    int out, in, nsplit;
    int64_t off;
};
struct UpdateP {
    LayerU L[4];
    int64_t total;
    float lr, mom;
    float *vel;     // [total] or null (mom == 0)
    float *grad;    // [total] or null
    const float *lossp;
    int nloss;
    float inv_count;
    float *loss;    // [1] or null
};

// Gradient (partial sums added in split order), momentum, descent, bf16
// export; block 0 also adds the loss partials in order.
__global__ __launch_bounds__(256) void update_kernel(UpdateP p) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x == 0 && p.loss) {
        // every thread sums a strided share of the loss partials, then a
        // fixed reduction tree (deterministic)
        __shared__ float part[4];
        float s = 0.f;
        for (int i = threadIdx.x; i < p.nloss; i += 256) s += p.lossp[i];
        s = wave_sum(s);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
        __syncthreads();
        if (threadIdx.x == 0) *p.loss = ((part[0] + part[1]) + (part[2] + part[3])) * p.inv_count;
    }
    if (g >= p.total) return;
    int li = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i) li = g >= p.L[i].off ? i : li;
    const LayerU &L = p.L[li];
    const int64_t e = g - L.off;
    const int64_t nw = (int64_t)L.out * L.in;
    const bool isw = e < nw;
    const int64_t row = isw ? e / L.in : e - nw;
    const int64_t col = isw ? e % L.in : L.in;
    const int64_t ld = (int64_t)L.in + 1, ps = (int64_t)L.out * ld;
    // four running sums over interleaved splits (loads of four splits in
    // flight), added in a fixed order
    const float *pp = L.part + row * ld + col;
    float g0 = 0.f, g1 = 0.f, g2 = 0.f, g3 = 0.f;
    int z = 0;
    for (; z + 4 <= L.nsplit; z += 4) {
        g0 += pp[(int64_t)z * ps];
        g1 += pp[(int64_t)(z + 1) * ps];
        g2 += pp[(int64_t)(z + 2) * ps];
        g3 += pp[(int64_t)(z + 3) * ps];
    }
    for (; z < L.nsplit; ++z) g0 += pp[(int64_t)z * ps];
    const float gr = (g0 + g1) + (g2 + g3);
    if (p.grad) p.grad[g] = gr;
    float step = gr;
    if (p.vel) {
        const float v = p.mom * p.vel[g] + gr;
        p.vel[g] = v;
        step = v;
    }
    float *dst = isw ? &L.W[e] : &L.b[row];
    const float nv = *dst - p.lr * step;
    *dst = nv;
    if (isw && L.wexp) L.wexp[e] = f2bf(nv);
}

// Residual rows: 8 consecutive columns per thread (16-byte row loads), d / 8
// threads per compressed token of [q0, q0 + nq): x_p minus the mean of its
// reference rows (fp32 sum over the used slots in slot order, times 1 /
// k_eff).  grid (ceil(nq / (256 / (d / 8))), units).
template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&v)[8]) {
    if constexpr (sizeof(T) == 2) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void residual_kernel(const T *__restrict__ x, int64_t t0,
                                                       int64_t nrows, int s, int k, int d,
                                                       const T *__restrict__ refs, int64_t Rcap,
                                                       const uint16_t *__restrict__ idx,
                                                       int64_t Ncap, int64_t q0, int64_t nq,
                                                       float *__restrict__ out) {
    const int cpr = d / 8;                     // threads per token
    const int tpb = 256 / cpr;                 // tokens per block
    const int64_t qq = (int64_t)blockIdx.x * tpb + threadIdx.x / cpr;
    if (qq >= nq) return;
    const int c0 = 8 * (threadIdx.x % cpr);
    const int64_t unit = blockIdx.y;
    const int64_t q = q0 + qq;
    const int64_t pos = tok_pos(q, s);
    const uint16_t *ir = idx + (unit * Ncap + q) * k;
    const T *ur = refs + unit * Rcap * d + c0;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    int keff = 0;
    for (int sl = 0; sl < k; ++sl) {
        const uint16_t j = ir[sl];
        if (j == kIdxUnused) continue;
        ++keff;
        float r[8];
        load8<T>(ur + (int64_t)j * d, r);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += r[i];
    }
    const float inv = 1.f / (float)max(keff, 1);
    float xv[8];
    load8<T>(x + (unit * nrows + (pos - t0)) * d + c0, xv);
    float *o = out + (unit * nq + qq) * d + c0;
    f32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = xv[i] - acc[i] * inv;
        hi[i] = xv[4 + i] - acc[4 + i] * inv;
    }
    *reinterpret_cast<f32x4 *>(o) = lo;
    *reinterpret_cast<f32x4 *>(o + 4) = hi;
}

// 128-row tiles for the products over the n rows, 64-row tiles for the
// weight gradients (at most a few hundred output rows).  The loss epilogue's
// partial sums are laid out per 128-row tile (train_layout).
template <int EP>
void gemm(const GemmP &p, int nsplit, hipStream_t st) {
    if (p.M >= 1024 || EP == kEpiLoss) {
        const dim3 grid((unsigned)((p.M + 127) / 128), (unsigned)((p.N + 63) / 64), (unsigned)nsplit);
        hipLaunchKernelGGL((gemm_f32_kernel<EP, 128>), grid, dim3(256), 0, st, p);
    } else {
        const dim3 grid((unsigned)((p.M + 63) / 64), (unsigned)((p.N + 63) / 64), (unsigned)nsplit);
        hipLaunchKernelGGL((gemm_f32_kernel<EP, 64>), grid, dim3(256), 0, st, p);
    }
}

// Split of a weight-gradient product over its n rows: about 768 blocks,
// chunks of whole 32-row steps.
void wsplit(int64_t n, int out, int in, int *nsplit, int64_t *kchunk) {
    const int64_t tiles = ((out + 63) / 64) * ((in + 1 + 63) / 64);
    int64_t s = std::max<int64_t>(1, std::min<int64_t>((768 + tiles - 1) / tiles, (n + 63) / 64));
    int64_t c = (n + s - 1) / s;
    c = (c + 31) / 32 * 32;
    *kchunk = c;
    *nsplit = (int)((n + c - 1) / c);
}

struct TrainLayout {
    size_t a1, h1, z, a2, h2, g4, dz, lossp, part[4], total;
    int nloss, nsplit[4];
    int64_t kchunk[4];
};

TrainLayout train_layout(int d, int h1, int dc, int h2, int64_t n) {
    TrainLayout t;
    size_t o = 0;
    auto take = [&](size_t floats) {
        const size_t at = o;
        o += (floats * sizeof(float) + 255) & ~(size_t)255;
        return at;
    };
    t.a1 = take((size_t)n * h1);   // later the gradient at A1
    t.h1 = take((size_t)n * h1);
    t.z = take((size_t)n * dc);
    t.a2 = take((size_t)n * h2);   // later the gradient at A2
    t.h2 = take((size_t)n * h2);
    t.g4 = take((size_t)n * d);
    t.dz = take((size_t)n * dc);
    t.nloss = (int)(((n + 127) / 128) * ((d + 63) / 64));
    t.lossp = take((size_t)t.nloss);
    const int outs[4] = {h1, dc, h2, d}, ins[4] = {d, h1, dc, h2};
    for (int l = 0; l < 4; ++l) {
        wsplit(n, outs[l], ins[l], &t.nsplit[l], &t.kchunk[l]);
        t.part[l] = take((size_t)t.nsplit[l] * outs[l] * (ins[l] + 1));
    }
    t.total = o;
    return t;
}

}  // namespace

size_t train_ws_bytes(int d, int h1, int dc, int h2, int64_t n) {
    return train_layout(d, h1, dc, h2, n).total;
}

hipError_t launch_residuals(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                            const CacheArgs &c, float *out, hipStream_t st) {
    const int64_t q0 = toks_upto(t0, dm.s);
    const int64_t nq = toks_upto(t1, dm.s) - q0;
    if (nq <= 0) return hipSuccess;
    const int tpb = 256 / (dm.d / 8);
    const dim3 grid((unsigned)((nq + tpb - 1) / tpb), (unsigned)(dm.B * dm.H));
    if (dm.dtype == 0)
        hipLaunchKernelGGL(residual_kernel<float>, grid, dim3(256), 0, st, (const float *)x, t0,
                           t1 - t0, dm.s, dm.k, dm.d, (const float *)c.refs, dm.R, c.idx, dm.N,
                           q0, nq, out);
    else
        hipLaunchKernelGGL(residual_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t *)x,
                           t0, t1 - t0, dm.s, dm.k, dm.d, (const bf16_t *)c.refs, dm.R, c.idx,
                           dm.N, q0, nq, out);
    return hipGetLastError();
}

hipError_t launch_train_step(const TrainArgs &a, hipStream_t st) {
    const int d = a.comp.in, h1 = a.comp.hidden, dc = a.comp.out, h2 = a.dec.hidden;
    const int64_t n = a.n;
    const TrainLayout t = train_layout(d, h1, dc, h2, n);
    char *ws = (char *)a.ws;
    float *A1 = (float *)(ws + t.a1), *H1 = (float *)(ws + t.h1), *Z = (float *)(ws + t.z);
    float *A2 = (float *)(ws + t.a2), *H2 = (float *)(ws + t.h2), *G4 = (float *)(ws + t.g4);
    float *dZ = (float *)(ws + t.dz), *lossp = (float *)(ws + t.lossp);
    float *part[4];
    for (int l = 0; l < 4; ++l) part[l] = (float *)(ws + t.part[l]);
    const float *D = a.delta;

    auto rows = [&](const float *A, int64_t lda, const float *W, int64_t ldw_k, int64_t ldw_n,
                    int64_t N, int64_t K) {
        GemmP p{};
        p.A = A;
        p.sam = lda;
        p.sak = 1;
        p.B = W;
        p.sbk = ldw_k;
        p.sbn = ldw_n;
        p.M = n;
        p.N = N;
        p.NB = N;
        p.K = K;
        p.kchunk = K;
        return p;
    };
    // ---- forward
    GemmP p = rows(D, d, a.comp.w1, 1, d, h1, d);      // A1 = D W1c^T + b1c
    p.bias = a.comp.b1;
    p.out = A1;
    p.out2 = H1;
    p.ldo = h1;
    p.act = a.comp.act;
    gemm<kEpiAct>(p, 1, st);
    p = rows(H1, h1, a.comp.w2, 1, h1, dc, h1);         // Z = H1 W2c^T + b2c
    p.bias = a.comp.b2;
    p.out = Z;
    p.ldo = dc;
    gemm<kEpiLin>(p, 1, st);
    p = rows(Z, dc, a.dec.w1, 1, dc, h2, dc);           // A2 = Z W1d^T + b1d
    p.bias = a.dec.b1;
    p.out = A2;
    p.out2 = H2;
    p.ldo = h2;
    p.act = a.dec.act;
    gemm<kEpiAct>(p, 1, st);
    p = rows(H2, h2, a.dec.w2, 1, h2, d, h2);           // G4 = 2 (Y - D) / (n d)
    p.bias = a.dec.b2;
    p.out = G4;
    p.ldo = d;
    p.aux = D;
    p.ldx = d;
    p.scale = (float)(2.0 / ((double)n * (double)d));
    p.lossp = lossp;
    gemm<kEpiLoss>(p, 1, st);
    // ---- backward: weight gradients (A = gradient rows^T, B = layer input
    // rows and a column of ones) and the gradient rows of the layer below
    auto wgrad = [&](int l, const float *G, int64_t ldg, int outd, const float *X, int64_t ldx_,
                     int ind) {
        GemmP q{};
        q.A = G;
        q.sam = 1;
        q.sak = ldg;
        q.B = X;
        q.sbk = ldx_;
        q.sbn = 1;
        q.M = outd;
        q.N = ind + 1;
        q.NB = ind;
        q.K = n;
        q.kchunk = t.kchunk[l];
        q.out = part[l];
        q.ldo = ind + 1;
        gemm<kEpiPart>(q, t.nsplit[l], st);
    };
    wgrad(3, G4, d, d, H2, h2, h2);                     // dW2d, db2d
    p = rows(G4, d, a.dec.w2, h2, 1, h2, d);            // dA2 = (G4 W2d) phi_d'(A2)
    p.out = A2;
    p.ldo = h2;
    p.aux = A2;
    p.ldx = h2;
    p.act = a.dec.act;
    gemm<kEpiDAct>(p, 1, st);
    wgrad(2, A2, h2, h2, Z, dc, dc);                    // dW1d, db1d
    p = rows(A2, h2, a.dec.w1, dc, 1, dc, h2);          // dZ = dA2 W1d
    p.out = dZ;
    p.ldo = dc;
    gemm<kEpiLin>(p, 1, st);
    wgrad(1, dZ, dc, dc, H1, h1, h1);                   // dW2c, db2c
    p = rows(dZ, dc, a.comp.w2, h1, 1, h1, dc);         // dA1 = (dZ W2c) phi_c'(A1)
    p.out = A1;
    p.ldo = h1;
    p.aux = A1;
    p.ldx = h1;
    p.act = a.comp.act;
    gemm<kEpiDAct>(p, 1, st);
    wgrad(0, A1, h1, h1, D, d, d);                      // dW1c, db1c
    // ---- update
    UpdateP u{};
    const MlpF32 *m[4] = {&a.comp, &a.comp, &a.dec, &a.dec};
    const int outs[4] = {h1, dc, h2, d}, ins[4] = {d, h1, dc, h2};
    int64_t off = 0;
    for (int l = 0; l < 4; ++l) {
        const bool first = (l % 2) == 0;
        u.L[l].W = first ? m[l]->w1 : m[l]->w2;
        u.L[l].b = first ? m[l]->b1 : m[l]->b2;
        u.L[l].part = part[l];
        u.L[l].wexp = (bf16_t *)a.wexp[l];
        u.L[l].out = outs[l];
        u.L[l].in = ins[l];
        u.L[l].nsplit = t.nsplit[l];
        u.L[l].off = off;
        off += (int64_t)outs[l] * (ins[l] + 1);
    }
    u.total = off;
    u.lr = a.lr;
    u.mom = a.momentum;
    u.vel = a.velocity;
    u.grad = a.grad;
    u.lossp = lossp;
    u.nloss = t.nloss;
    u.inv_count = (float)(1.0 / ((double)n * (double)d));
    u.loss = a.loss;
    hipLaunchKernelGGL(update_kernel, dim3((unsigned)((off + 255) / 256)), dim3(256), 0, st, u);
    return hipGetLastError();
}

}  // namespace dk
