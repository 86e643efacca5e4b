// k_decode.hip -- decode attention over the compressed cache ("DeltaKV:
// Residual-Based KV Cache Compression via Long-Range Similarity", section 3,
// "Ricostruzione": a compressed token is rebuilt as the mean of its reference
// rows plus the Decompressor output; reference tokens are used as stored).
//
// The rebuilt rows are never materialised.  With the Decompressor
// x^ = KV_R + W2 h + b2, h = act(W1 z + b1), the score and value sums split
// exactly into
//   q . K^_t   = mean_{j in idx_t} (q . R^K_j) + (W2K^T q) . hK_t + q . b2K
//   sum_t p_t V^_t = sum_t p_t mean_{j in idx_t} R^V_j + W2V (sum_t p_t hV_t)
//                    + (sum_{t compressed} p_t) b2V + sum_{refs} p_j R^V_j,
// so each step needs: the q . R^K table over reference rows (one pass over the
// K references), the per-token hidden activations hK, hV (the only per-token
// MLP work), and the V reference rows.  Softmax is online (running maximum and
// sum per query head) over token partitions, merged by log-sum-exp.
//
// Kernels, in stream order:
//   qprep     u_g = W2K^T q_g and c_g = q_g . b2K for every query head
//   refscore  qR[j][g] = q_g . R^K_j for every reference row
//   main      one block per (partition, KV head, sequence): token partitions
//             rebuild hidden tiles and fold them into (m, l, acc_r, acc_h);
//             reference partitions fold the reference tokens themselves
//   combine   log-sum-exp merge of the partitions, W2V applied once to acc_h
#include <math.h>

#include "dk_common.h"
#include "dk_launch.h"

namespace dk {
namespace {

constexpr int kMaxG = 8;       // query heads per KV head
constexpr int kMaxD = 128;
constexpr int kMaxH = 256;
constexpr int kMaxDC = 128;
constexpr int kMaxK = 8;
constexpr int kTB = 16;        // tokens per tile
constexpr int kTokPart = 1024; // compressed tokens per partition
constexpr int kRefPart = 1024; // reference rows per partition
constexpr int kPStride = 4 + kMaxD + kMaxH;  // floats per (partition, query head)

struct DecWs {
    float *u;      // [B][Hq][kMaxH]
    float *cq;     // [B][Hq]
    float *qr;     // [B][H][Rt][G]
    float *part;   // [B][H][P][G][kPStride]
};

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecPlan {
    int64_t Rt, Nt, Ptok, Pref, P;
    size_t off_u, off_cq, off_qr, off_part, total;
};

DecPlan plan_decode(const Dims &dm, int Hq, int64_t T) {
    DecPlan p;
    const int G = Hq / dm.H;
    p.Rt = refs_upto(T, dm.s);
    p.Nt = T - p.Rt;
    p.Ptok = (p.Nt + kTokPart - 1) / kTokPart;
    p.Pref = (p.Rt + kRefPart - 1) / kRefPart;
    p.P = p.Ptok + p.Pref;
    size_t off = 0;
    p.off_u = off;
    off += align_up((size_t)dm.B * Hq * kMaxH * 4);
    p.off_cq = off;
    off += align_up((size_t)dm.B * Hq * 4);
    p.off_qr = off;
    off += align_up((size_t)dm.B * dm.H * p.Rt * G * 4);
    p.off_part = off;
    off += align_up((size_t)dm.B * dm.H * p.P * G * kPStride * 4);
    p.total = off;
    return p;
}

// u_g = W2K^T q_g (hidden entries), c_g = q_g . b2K.  grid (Hq, B).
template <typename T>
__global__ __launch_bounds__(256) void qprep_kernel(const T *__restrict__ q, int Hq, int d,
                                                    const T *__restrict__ w2, int hid,
                                                    const float *__restrict__ b2,
                                                    float *__restrict__ u,
                                                    float *__restrict__ cq) {
    __shared__ float qs[kMaxD];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const T *qrow = q + ((int64_t)b * Hq + g) * d;
    if (tid < d) qs[tid] = to_f32(qrow[tid]);
    __syncthreads();
    if (tid < hid) {
        float acc = 0.f;
        for (int c = 0; c < d; ++c) acc += to_f32(w2[(int64_t)c * hid + tid]) * qs[c];
        u[((int64_t)b * Hq + g) * kMaxH + tid] = acc;
    }
    if (tid == 0) {
        float acc = 0.f;
        if (b2)
            for (int c = 0; c < d; ++c) acc += qs[c] * b2[c];
        cq[(int64_t)b * Hq + g] = acc;
    }
}

// qR[j][g] = q_g . R^K_j over the Rt reference rows.  grid (ceil(Rt/64), H, B).
template <typename T>
__global__ __launch_bounds__(256) void refscore_kernel(const T *__restrict__ q, int Hq, int G,
                                                       int d, const T *__restrict__ krefs,
                                                       int64_t Rcap, int64_t Rt,
                                                       float *__restrict__ qr) {
    __shared__ float qs[kMaxG][kMaxD];
    const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, H = gridDim.y;
    for (int i = tid; i < G * d; i += 256)
        qs[i / d][i % d] = to_f32(q[((int64_t)b * Hq + h * G + i / d) * d + i % d]);
    __syncthreads();
    const int64_t unit = (int64_t)b * H + h;
    for (int i = tid; i < 64 * G; i += 256) {
        const int64_t j = (int64_t)blockIdx.x * 64 + i / G;
        const int g = i % G;
        if (j >= Rt) continue;
        const T *r = krefs + (unit * Rcap + j) * d;
        float acc = 0.f;
        for (int c = 0; c < d; ++c) acc += qs[g][c] * to_f32(r[c]);
        qr[(unit * Rt + j) * G + g] = acc;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void main_kernel(
    int Hq, int G, int d, int dc, int k, int s, int64_t Rcap, int64_t Ncap, int64_t Rt,
    int64_t Nt, int64_t Ptok, const T *__restrict__ kref, const T *__restrict__ klat,
    const uint16_t *__restrict__ kidx, const T *__restrict__ vref, const T *__restrict__ vlat,
    const uint16_t *__restrict__ vidx, const T *__restrict__ kw1, const float *__restrict__ kb1,
    int khid, int kact, const T *__restrict__ vw1, const float *__restrict__ vb1, int vhid,
    int vact, float scale, const float *__restrict__ u, const float *__restrict__ cq,
    const float *__restrict__ qr, float *__restrict__ part) {
    (void)kref;
    (void)s;
    __shared__ float us[kMaxG][kMaxH];
    __shared__ float cqs[kMaxG];
    __shared__ float z[kTB][kMaxDC];
    __shared__ float hs[kTB][kMaxH];
    __shared__ uint16_t ids[kTB][kMaxK];
    __shared__ float kinv[kTB];
    __shared__ float sc[kMaxG][64];
    __shared__ float acc_h[kMaxG][kMaxH];
    __shared__ float acc_r[kMaxG][kMaxD];
    __shared__ float ms[kMaxG], ls[kMaxG], alphas[kMaxG];

    const int pidx = blockIdx.x, h = blockIdx.y, b = blockIdx.z, H = gridDim.y;
    const int tid = threadIdx.x;
    const int64_t unit = (int64_t)b * H + h;
    const int P = gridDim.x;

    for (int i = tid; i < G * kMaxH; i += 256) acc_h[i / kMaxH][i % kMaxH] = 0.f;
    for (int i = tid; i < G * kMaxD; i += 256) acc_r[i / kMaxD][i % kMaxD] = 0.f;
    if (tid < G) {
        ms[tid] = -INFINITY;
        ls[tid] = 0.f;
    }

    if (pidx < Ptok) {
        for (int i = tid; i < G * khid; i += 256)
            us[i / khid][i % khid] = u[((int64_t)b * Hq + h * G + i / khid) * kMaxH + i % khid];
        if (tid < G) cqs[tid] = cq[(int64_t)b * Hq + h * G + tid];
        __syncthreads();
        const int64_t qa = (int64_t)pidx * kTokPart;
        const int64_t qb = min(Nt, qa + kTokPart);
        for (int64_t q0 = qa; q0 < qb; q0 += kTB) {
            const int nt = (int)min((int64_t)kTB, qb - q0);
            // ---- K side: hidden tile and scores
            for (int i = tid; i < nt * dc; i += 256)
                z[i / dc][i % dc] = to_f32(klat[(unit * Ncap + q0 + i / dc) * dc + i % dc]);
            for (int i = tid; i < nt * k; i += 256)
                ids[i / k][i % k] = kidx[(unit * Ncap + q0 + i / k) * k + i % k];
            __syncthreads();
            for (int i = tid; i < nt * khid; i += 256) {
                const int t = i / khid, o = i % khid;
                float acc = kb1 ? kb1[o] : 0.f;
                for (int c = 0; c < dc; ++c) acc += to_f32(kw1[(int64_t)o * dc + c]) * z[t][c];
                hs[t][o] = apply_act(acc, kact);
            }
            __syncthreads();
            for (int i = tid; i < G * nt; i += 256) {
                const int g = i / nt, t = i % nt;
                float rs = 0.f;
                int keff = 0;
                for (int r = 0; r < k; ++r) {
                    const uint16_t j = ids[t][r];
                    if (j == kIdxUnused) continue;
                    rs += qr[(unit * Rt + j) * G + g];
                    ++keff;
                }
                float hsum = 0.f;
                for (int o = 0; o < khid; ++o) hsum += us[g][o] * hs[t][o];
                sc[g][t] = scale * (rs / (float)keff + hsum + cqs[g]);
            }
            __syncthreads();
            // ---- online softmax update
            if (tid < G) {
                const int g = tid;
                float tmax = -INFINITY;
                for (int t = 0; t < nt; ++t) tmax = fmaxf(tmax, sc[g][t]);
                const float mnew = fmaxf(ms[g], tmax);
                const float alpha = expf(ms[g] - mnew);
                float lsum = 0.f;
                for (int t = 0; t < nt; ++t) {
                    const float pv = expf(sc[g][t] - mnew);
                    sc[g][t] = pv;
                    lsum += pv;
                }
                ls[g] = ls[g] * alpha + lsum;
                ms[g] = mnew;
                alphas[g] = alpha;
            }
            // ---- V side: latents, hidden tile
            for (int i = tid; i < nt * dc; i += 256)
                z[i / dc][i % dc] = to_f32(vlat[(unit * Ncap + q0 + i / dc) * dc + i % dc]);
            for (int i = tid; i < nt * k; i += 256)
                ids[i / k][i % k] = vidx[(unit * Ncap + q0 + i / k) * k + i % k];
            __syncthreads();
            for (int i = tid; i < G * kMaxH; i += 256) acc_h[i / kMaxH][i % kMaxH] *= alphas[i / kMaxH];
            for (int i = tid; i < G * kMaxD; i += 256) acc_r[i / kMaxD][i % kMaxD] *= alphas[i / kMaxD];
            if (tid < nt) {
                int keff = 0;
                for (int r = 0; r < k; ++r) keff += ids[tid][r] != kIdxUnused;
                kinv[tid] = 1.f / (float)keff;
            }
            for (int i = tid; i < nt * vhid; i += 256) {
                const int t = i / vhid, o = i % vhid;
                float acc = vb1 ? vb1[o] : 0.f;
                for (int c = 0; c < dc; ++c) acc += to_f32(vw1[(int64_t)o * dc + c]) * z[t][c];
                hs[t][o] = apply_act(acc, vact);
            }
            __syncthreads();
            for (int i = tid; i < G * vhid; i += 256) {
                const int g = i / vhid, o = i % vhid;
                float acc = 0.f;
                for (int t = 0; t < nt; ++t) acc += sc[g][t] * hs[t][o];
                acc_h[g][o] += acc;
            }
            for (int i = tid; i < G * d; i += 256) {
                const int g = i / d, c = i % d;
                float acc = 0.f;
                for (int t = 0; t < nt; ++t) {
                    float rsum = 0.f;
                    for (int r = 0; r < k; ++r) {
                        const uint16_t j = ids[t][r];
                        if (j == kIdxUnused) continue;
                        rsum += to_f32(vref[(unit * Rcap + j) * d + c]);
                    }
                    acc += sc[g][t] * kinv[t] * rsum;
                }
                acc_r[g][c] += acc;
            }
            __syncthreads();
        }
    } else {
        // reference tokens: score = scale * qR, value = stored V row
        __syncthreads();
        const int64_t ja = (pidx - Ptok) * (int64_t)kRefPart;
        const int64_t jb = min(Rt, ja + kRefPart);
        for (int64_t j0 = ja; j0 < jb; j0 += 64) {
            const int nj = (int)min((int64_t)64, jb - j0);
            for (int i = tid; i < G * nj; i += 256) {
                const int g = i / nj, t = i % nj;
                sc[g][t] = scale * qr[(unit * Rt + j0 + t) * G + g];
            }
            __syncthreads();
            if (tid < G) {
                const int g = tid;
                float tmax = -INFINITY;
                for (int t = 0; t < nj; ++t) tmax = fmaxf(tmax, sc[g][t]);
                const float mnew = fmaxf(ms[g], tmax);
                const float alpha = expf(ms[g] - mnew);
                float lsum = 0.f;
                for (int t = 0; t < nj; ++t) {
                    const float pv = expf(sc[g][t] - mnew);
                    sc[g][t] = pv;
                    lsum += pv;
                }
                ls[g] = ls[g] * alpha + lsum;
                ms[g] = mnew;
                alphas[g] = alpha;
            }
            __syncthreads();
            for (int i = tid; i < G * d; i += 256) {
                const int g = i / d, c = i % d;
                float acc = acc_r[g][c] * alphas[g];
                for (int t = 0; t < nj; ++t)
                    acc += sc[g][t] * to_f32(vref[(unit * Rcap + j0 + t) * d + c]);
                acc_r[g][c] = acc;
            }
            __syncthreads();
        }
    }
    __syncthreads();
    // partial record: m, l, l over compressed tokens, acc_r[d], acc_h[hidden]
    float *pr = part + ((unit * P + pidx) * G) * kPStride;
    for (int i = tid; i < G * kPStride; i += 256) {
        const int g = i / kPStride, e = i % kPStride;
        float v = 0.f;
        if (e == 0) v = ms[g];
        else if (e == 1) v = ls[g];
        else if (e == 2) v = (pidx < Ptok) ? ls[g] : 0.f;
        else if (e >= 4 && e < 4 + kMaxD) v = (e - 4 < d) ? acc_r[g][e - 4] : 0.f;
        else if (e >= 4 + kMaxD) v = acc_h[g][e - 4 - kMaxD];
        pr[(int64_t)g * kPStride + e] = v;
    }
}

// Log-sum-exp merge of the partitions of one query head; W2V applied to the
// merged hidden sum.  grid (Hq, B).
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(int Hq, int G, int d, int H, int64_t P,
                                                      const float *__restrict__ part,
                                                      const T *__restrict__ vw2, int vhid,
                                                      const float *__restrict__ vb2,
                                                      float *__restrict__ out) {
    __shared__ float acch[kMaxH];
    __shared__ float red[3];
    const int gq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int h = gq / G, g = gq % G;
    const int64_t unit = (int64_t)b * H + h;
    const float *base = part + (unit * P * G + g) * kPStride;
    const int64_t pstep = (int64_t)G * kPStride;
    if (tid == 0) {
        float M = -INFINITY;
        for (int64_t p = 0; p < P; ++p) M = fmaxf(M, base[p * pstep]);
        float L = 0.f, Lt = 0.f;
        for (int64_t p = 0; p < P; ++p) {
            const float w = expf(base[p * pstep] - M);
            L += w * base[p * pstep + 1];
            Lt += w * base[p * pstep + 2];
        }
        red[0] = M;
        red[1] = L;
        red[2] = Lt;
    }
    __syncthreads();
    const float M = red[0], L = red[1], Lt = red[2];
    if (tid < vhid) {
        float a = 0.f;
        for (int64_t p = 0; p < P; ++p)
            a += expf(base[p * pstep] - M) * base[p * pstep + 4 + kMaxD + tid];
        acch[tid] = a;
    }
    __syncthreads();
    if (tid < d) {
        float a = 0.f;
        for (int64_t p = 0; p < P; ++p) a += expf(base[p * pstep] - M) * base[p * pstep + 4 + tid];
        float w = 0.f;
        for (int o = 0; o < vhid; ++o) w += to_f32(vw2[(int64_t)tid * vhid + o]) * acch[o];
        const float bias = vb2 ? vb2[tid] : 0.f;
        out[((int64_t)b * Hq + gq) * d + tid] = (a + w + Lt * bias) / L;
    }
}

template <typename T>
hipError_t launch_decode_t(const Dims &dm, int Hq, int64_t T_, const void *q,
                           const CacheArgs &kc, const MlpArgs &kd, const CacheArgs &vc,
                           const MlpArgs &vd, float scale, float *out, void *ws,
                           hipStream_t st) {
    const DecPlan pl = plan_decode(dm, Hq, T_);
    const int G = Hq / dm.H;
    char *w = (char *)ws;
    float *u = (float *)(w + pl.off_u);
    float *cq = (float *)(w + pl.off_cq);
    float *qr = (float *)(w + pl.off_qr);
    float *part = (float *)(w + pl.off_part);
    hipLaunchKernelGGL(qprep_kernel<T>, dim3(Hq, dm.B), dim3(256), 0, st, (const T *)q, Hq, dm.d,
                       (const T *)kd.w2, kd.hidden, kd.b2, u, cq);
    hipLaunchKernelGGL(refscore_kernel<T>, dim3((unsigned)((pl.Rt + 63) / 64), dm.H, dm.B),
                       dim3(256), 0, st, (const T *)q, Hq, G, dm.d, (const T *)kc.refs, dm.R,
                       pl.Rt, qr);
    hipLaunchKernelGGL(main_kernel<T>, dim3((unsigned)pl.P, dm.H, dm.B), dim3(256), 0, st, Hq, G,
                       dm.d, dm.dc, dm.k, dm.s, dm.R, dm.N, pl.Rt, pl.Nt, pl.Ptok,
                       (const T *)kc.refs, (const T *)kc.lat, kc.idx, (const T *)vc.refs,
                       (const T *)vc.lat, vc.idx, (const T *)kd.w1, kd.b1, kd.hidden, kd.act,
                       (const T *)vd.w1, vd.b1, vd.hidden, vd.act, scale, u, cq, qr, part);
    hipLaunchKernelGGL(combine_kernel<T>, dim3(Hq, dm.B), dim3(256), 0, st, Hq, G, dm.d, dm.H,
                       pl.P, part, (const T *)vd.w2, vd.hidden, vd.b2, out);
    return hipGetLastError();
}

}  // namespace

size_t decode_ws_bytes(const Dims &dm, int Hq, int64_t T) { return plan_decode(dm, Hq, T).total; }

hipError_t launch_decode(const Dims &dm, int Hq, int64_t T, const void *q, const CacheArgs &kc,
                         const MlpArgs &kdec, const CacheArgs &vc, const MlpArgs &vdec,
                         float scale, float *out, void *ws, size_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;
    if (dm.dtype == 0)
        return launch_decode_t<float>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, st);
    return launch_decode_t<bf16_t>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, st);
}

}  // namespace dk
