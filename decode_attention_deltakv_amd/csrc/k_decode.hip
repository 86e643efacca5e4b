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
//   prep      qR[j][g] = q_g . R^K_j for every reference row, and
//             u_g = W2K^T q_g, c_g = q_g . b2K for every query head
//   main      one block per (partition, KV head, sequence): token partitions
//             rebuild hidden tiles and fold them into (m, l, acc_r, acc_h);
//             reference partitions fold the reference tokens themselves
//   combine   log-sum-exp merge of the partitions, W2V applied once to acc_h
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "dk_common.h"
#include "dk_launch.h"
#include "dk_mfma.h"

namespace dk {
namespace {

constexpr int kMaxG = 8;       // query heads per KV head
constexpr int kMaxD = 128;
constexpr int kMaxH = 256;
constexpr int kMaxDC = 128;
constexpr int kMaxK = 8;
constexpr int kTB = 16;        // tokens per tile (general path)
constexpr int kTileTok = 32;   // tokens per tile (matrix-core path); partitions hold whole tiles
constexpr int kTargetBlocks = 512;
constexpr int kRefPart = 512;  // reference rows per partition
constexpr int kMaxParts = 4096; // partitions per unit (combine keeps their weights in LDS)
constexpr int kPStride = 4 + kMaxD + kMaxH;  // floats per (partition, query head)
constexpr int kCombThreads = 256;               // threads of the combine kernel
constexpr int kSpTiles = 16;   // most 32-token tiles per partition of a sparse call

// The q.R^K table keeps its query heads padded to a multiple of 4 (zeros), so
// a lane can read the 4 heads of its row group with one 16-byte load, and one
// extra all-zero row after the Rt reference rows, which unused index slots
// read instead of a masked load.
__host__ __device__ inline int qr_heads(int G) { return (G + 3) & ~3; }
__host__ __device__ inline int64_t qr_rows(int64_t Rt) { return Rt + 1; }
// selection keys of a unit: T entries, rows padded to a multiple of 4
__host__ __device__ inline int64_t keys_stride(int64_t T) { return (T + 3) & ~(int64_t)3; }

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecPlan {
    int64_t Rt, Nt, Ptok, Pref, P;
    int tiles_per_part;
    size_t off_u, off_cq, off_qr, off_part, off_ord, off_cnt, total;
};

// Partitions and workspace of one decode call over T cached tokens; with
// nsel >= 0, of a sparse call whose units list nsel positions each (the
// partitions then cover the most compressed tokens and references such a
// list can hold, and the workspace adds the split lists and their counts).
DecPlan plan_decode(const Dims &dm, int Hq, int64_t T, int64_t nsel = -1) {
    DecPlan p;
    const int G = Hq / dm.H;
    p.Rt = refs_upto(T, dm.s);
    p.Nt = T - p.Rt;
    const int64_t nc = nsel >= 0 ? std::min(nsel, p.Nt) : p.Nt;
    const int64_t nr = nsel >= 0 ? std::min(nsel, p.Rt) : p.Rt;
    // about kTargetBlocks blocks per launch over all units, whole 32-token tiles
    const int64_t U = (int64_t)dm.B * dm.H;
    const int64_t tiles = (nc + kTileTok - 1) / kTileTok;
    const int64_t want = std::max<int64_t>(1, (kTargetBlocks + U - 1) / U);
    p.tiles_per_part = (int)std::max<int64_t>(2, (tiles + want - 1) / want);
    p.Pref = (nr + kRefPart - 1) / kRefPart;
    if (nsel >= 0) {
        // a sparse call is short: its token and reference blocks together
        // should fit the kTargetBlocks that run at once (two per CU), or the
        // blocks past them run as a second round
        const int64_t ptok_max = std::max<int64_t>(1, kTargetBlocks / U - p.Pref);
        p.tiles_per_part = (int)std::max<int64_t>(1, (tiles + ptok_max - 1) / ptok_max);
    }
    // keep the partition count within what the merge holds in LDS
    const int64_t max_tok_parts = kMaxParts - p.Pref;
    if ((tiles + p.tiles_per_part - 1) / p.tiles_per_part > max_tok_parts)
        p.tiles_per_part = (int)((tiles + max_tok_parts - 1) / max_tok_parts);
    // a sparse partition stages its list entries in LDS: at most kSpTiles tiles
    if (nsel >= 0) p.tiles_per_part = std::min(p.tiles_per_part, kSpTiles);
    p.Ptok = (tiles + p.tiles_per_part - 1) / p.tiles_per_part;
    p.P = p.Ptok + p.Pref;
    size_t off = 0;
    p.off_u = off;
    off += align_up((size_t)dm.B * Hq * kMaxH * 4);
    p.off_cq = off;
    off += align_up((size_t)dm.B * Hq * 4);
    p.off_qr = off;
    off += align_up((size_t)dm.B * dm.H * qr_rows(p.Rt) * qr_heads(G) * 4);
    p.off_part = off;
    off += align_up((size_t)dm.B * dm.H * p.P * G * kPStride * 4);
    p.off_ord = off;
    if (nsel >= 0) off += align_up((size_t)2 * U * nsel * 4);
    p.off_cnt = off;
    if (nsel >= 0) off += align_up((size_t)2 * U * 4);
    p.total = off;
    return p;
}

template <typename T>
__global__ __launch_bounds__(256) void main_kernel(
    int Hq, int G, int d, int dc, int k, int s, int64_t Rcap, int64_t Ncap, int64_t Rt,
    int64_t Nt, int64_t Ptok, int64_t tok_per_part, const T *__restrict__ kref,
    const T *__restrict__ klat,
    const uint16_t *__restrict__ kidx, const T *__restrict__ vref, const T *__restrict__ vlat,
    const uint16_t *__restrict__ vidx, const T *__restrict__ kw1, const float *__restrict__ kb1,
    int khid, int kact, const T *__restrict__ vw1, const float *__restrict__ vb1, int vhid,
    int vact, float scale, const float *__restrict__ u, const float *__restrict__ cq,
    const float *__restrict__ qr, float *__restrict__ part, const int32_t *__restrict__ sord,
    const int32_t *__restrict__ scnt, int nsel, float *__restrict__ logc,
    float *__restrict__ logr) {
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
    // sparse mode (sord non-null): list positions of the unit's selected
    // compressed-token ordinals (sord[0][unit]) and reference ordinals
    // (sord[1][unit]) replace consecutive ordinals
    const bool sp = sord != nullptr;
    const int32_t *cord_u = sp ? sord + unit * nsel : nullptr;
    const int32_t *rord_u = sp ? sord + ((int64_t)gridDim.y * gridDim.z + unit) * nsel : nullptr;
    const int64_t Nt_u = sp ? (int64_t)scnt[2 * unit] : Nt;
    const int64_t Rt_u = sp ? (int64_t)scnt[2 * unit + 1] : Rt;

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
        const int64_t qa = (int64_t)pidx * tok_per_part;
        const int64_t qb = min(Nt_u, qa + tok_per_part);
        for (int64_t q0 = qa; q0 < qb; q0 += kTB) {
            const int nt = (int)min((int64_t)kTB, qb - q0);
            // ---- K side: hidden tile and scores
            for (int i = tid; i < nt * dc; i += 256) {
                const int64_t o = sp ? cord_u[q0 + i / dc] : q0 + i / dc;
                z[i / dc][i % dc] = to_f32(klat[(unit * Ncap + o) * dc + i % dc]);
            }
            for (int i = tid; i < nt * k; i += 256) {
                const int64_t o = sp ? cord_u[q0 + i / k] : q0 + i / k;
                ids[i / k][i % k] = kidx[(unit * Ncap + o) * k + i % k];
            }
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
                    rs += qr[(unit * qr_rows(Rt) + j) * qr_heads(G) + g];
                    ++keff;
                }
                float hsum = 0.f;
                for (int o = 0; o < khid; ++o) hsum += us[g][o] * hs[t][o];
                sc[g][t] = scale * (rs / (float)keff + hsum + cqs[g]);
                if (!sp && logc) logc[(unit * G + g) * Nt + q0 + t] = sc[g][t];
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
            for (int i = tid; i < nt * dc; i += 256) {
                const int64_t o = sp ? cord_u[q0 + i / dc] : q0 + i / dc;
                z[i / dc][i % dc] = to_f32(vlat[(unit * Ncap + o) * dc + i % dc]);
            }
            for (int i = tid; i < nt * k; i += 256) {
                const int64_t o = sp ? cord_u[q0 + i / k] : q0 + i / k;
                ids[i / k][i % k] = vidx[(unit * Ncap + o) * k + i % k];
            }
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
        const int64_t jb = min(Rt_u, ja + kRefPart);
        for (int64_t j0 = ja; j0 < jb; j0 += 64) {
            const int nj = (int)min((int64_t)64, jb - j0);
            for (int i = tid; i < G * nj; i += 256) {
                const int g = i / nj, t = i % nj;
                const int64_t j = sp ? rord_u[j0 + t] : j0 + t;
                sc[g][t] = scale * qr[(unit * qr_rows(Rt) + j) * qr_heads(G) + g];
                if (!sp && logr) logr[(unit * G + g) * Rt + j] = sc[g][t];
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
                for (int t = 0; t < nj; ++t) {
                    const int64_t j = sp ? rord_u[j0 + t] : j0 + t;
                    acc += sc[g][t] * to_f32(vref[(unit * Rcap + j) * d + c]);
                }
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

// Block-wide max or sum (256 threads).
template <int NW = 4>
__device__ __forceinline__ float block_reduce(float v, float *red, bool is_max) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < NW; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

// Eight consecutive elements as fp32 (16-byte loads; 16-byte aligned).
__device__ __forceinline__ void load8(const bf16_t *p, float (&v)[8]) {
    const u32x4 w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[4 + i] = b[i];
    }
}

// Split of one unit's sparse position list (on-demand reconstruction of
// selected tokens), run by one 256-thread block.  The valid entries
// (0 <= p < T) of pos[unit][0..nsel) are written, in list order, as
// compressed-token ordinals q = p - ((p - 1) / s + 1) to ord[0][unit][..] and
// as reference ordinals p / s to ord[1][unit][..]; the two counts go to
// cnt[unit][0..1].  Entries outside [0, T) are skipped.  Chunks of 4096
// entries: all of a chunk's loads are issued before any is used.
__device__ __forceinline__ void sparse_split_block(const int32_t *__restrict__ pos, int nsel,
                                                   int64_t T, int s, int U, int unit,
                                                   int32_t *__restrict__ ord,
                                                   int32_t *__restrict__ cnt) {
    constexpr int PER = 16;  // entries per thread and chunk
    __shared__ uint32_t wtot[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int32_t *pu = pos + (int64_t)unit * nsel;
    int32_t *cu = ord + (int64_t)unit * nsel;
    int32_t *ru = ord + ((int64_t)U + unit) * nsel;
    int nc = 0, nr = 0;  // entries written so far (block-uniform)
    for (int base = 0; base < nsel; base += 256 * PER) {
        int32_t v[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int i = base + tid * PER + e;
            v[e] = i < nsel ? pu[i] : -1;
        }
        uint32_t mine = 0;  // compressed count | reference count << 16
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const bool ok = v[e] >= 0 && (int64_t)v[e] < T;
            mine += ok ? (v[e] % s == 0 ? 0x10000u : 1u) : 0u;
        }
        // exclusive scan of the packed counts over the block
        uint32_t inc = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane == 63) wtot[w] = inc;
        __syncthreads();
        uint32_t before = inc - mine, total = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            before += i < w ? wtot[i] : 0u;
            total += wtot[i];
        }
        int oc = nc + (int)(before & 0xffffu), orr = nr + (int)(before >> 16);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int32_t p = v[e];
            if (p < 0 || (int64_t)p >= T) continue;
            if (p % s == 0) ru[orr++] = p / s;
            else cu[oc++] = p - ((p - 1) / s + 1);
        }
        nc += (int)(total & 0xffffu);
        nr += (int)(total >> 16);
        __syncthreads();  // wtot is rewritten by the next chunk
    }
    if (tid == 0) {
        cnt[2 * unit] = nc;
        cnt[2 * unit + 1] = nr;
    }
}

// Query-side tables of one decode step, one launch.  grid (nrb + G, H, B):
//   blockIdx.x <  nrb  rows [256 x, 256 x + 256) of qR[j][g] = q_g . R^K_j
//                      (bf16: matrix cores; row Rt is the zero row)
//   nrb <= x < nrb + G u_g = W2K^T q_g and c_g = q_g . b2K for query head
//                      g = x - nrb of the KV head
//   x == nrb + G       (sparse calls only, pos non-null, one more block) the
//                      split of the unit's position list (sparse_split_block)
// PG: paged reference rows, looked up through the block table in pm.
template <typename T, bool PG>
__global__ __launch_bounds__(256) void prep_kernel(const T *__restrict__ q, int Hq, int G, int d,
                                                   const T *__restrict__ krefs, int64_t Rcap,
                                                   int64_t Rt, int nrb, const T *__restrict__ w2,
                                                   int hid, const float *__restrict__ b2,
                                                   float *__restrict__ u, float *__restrict__ cq,
                                                   float *__restrict__ qr,
                                                   const int32_t *__restrict__ pos, int nsel,
                                                   int64_t ntok, int s, int32_t *__restrict__ ord,
                                                   int32_t *__restrict__ cnt, PageMap pm) {
    __shared__ float qs[kMaxG][kMaxD];
    __shared__ float red[1][32][kMaxH];
    const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, H = gridDim.y;
    // the query rows in LDS (fp32), for every block but the matrix-core
    // qR blocks, which load their operands straight into registers together
    // with the reference rows (one memory round trip)
    auto stage_q = [&]() {
        for (int i = tid; i < G * d; i += 256)
            qs[i / d][i % d] = to_f32(q[((int64_t)b * Hq + h * G + i / d) * d + i % d]);
        __syncthreads();
    };
    const int64_t unit = (int64_t)b * H + h;
    const int GQ = qr_heads(G);
    if (pos && (int)blockIdx.x == nrb + G) {
        sparse_split_block(pos, nsel, ntok, s, H * (int)gridDim.z, (int)unit, ord, cnt);
        return;
    }
    if (sizeof(T) != 2 || (int)blockIdx.x >= nrb) stage_q();
    if ((int)blockIdx.x < nrb) {
        if constexpr (sizeof(T) == 2) {
            // bf16: matrix cores, qR^T tile = R (16 rows x d) . Q^T (d x 16
            // heads); reference rows come straight from global memory
            const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4;
            const u32x4 zero4 = {0u, 0u, 0u, 0u};
            const T *qg = q + ((int64_t)b * Hq + h * G + (l16 < G ? l16 : 0)) * d;
            bf16x8 qb[kMaxD / 32];
#pragma unroll
            for (int ks = 0; ks < kMaxD / 32; ++ks)
                qb[ks] = as_bf16x8(l16 < G && 32 * ks < d ? ld16(qg + 32 * ks + 8 * lq) : zero4);
            // all of the block's row loads first (every load issued: rows
            // past the range read the last row, columns past d the last
            // chunk, both under zero weight or never stored)
            constexpr int NKS = kMaxD / 32;
            u32x4 rv[4][NKS];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t j0 = (int64_t)blockIdx.x * 256 + 64 * it + 16 * w;
                const int64_t jr = min(j0 + l16, Rt - 1 < 0 ? 0 : Rt - 1);
                const T *r = krefs + (PG ? pg_ref_row(pm, unit, jr) : unit * Rcap + jr) * d;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) rv[it][ks] = ld16(r + min(32 * ks, d - 32) + 8 * lq);
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t j0 = (int64_t)blockIdx.x * 256 + 64 * it + 16 * w;
                if (j0 > Rt) break;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) acc = mfma16_bf16(as_bf16x8(rv[it][ks]), qb[ks], acc);
                // acc[r] = qR[j0 + 4 lq + r][head l16]
                if (l16 < GQ) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t j = j0 + 4 * lq + e;
                        if (j <= Rt)
                            qr[(unit * qr_rows(Rt) + j) * GQ + l16] = (j < Rt && l16 < G) ? acc[e] : 0.f;
                    }
                }
            }
            return;
        } else {
            const int64_t j = (int64_t)blockIdx.x * 256 + tid;
            if (j > Rt) return;
            float acc[kMaxG];
#pragma unroll
            for (int g = 0; g < kMaxG; ++g) acc[g] = 0.f;
            if (j < Rt) {
                const T *r = krefs + (PG ? pg_ref_row(pm, unit, j) : unit * Rcap + j) * d;
                for (int c0 = 0; c0 < d; c0 += 8) {
                    float v[8];
                    load8(r + c0, v);
#pragma unroll
                    for (int g = 0; g < kMaxG; ++g) {
                        if (g >= G) break;
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[g] += qs[g][c0 + e] * v[e];
                    }
                }
            }
            float *dst = qr + (unit * qr_rows(Rt) + j) * GQ;
#pragma unroll
            for (int g4 = 0; g4 < kMaxG; g4 += 4) {
                if (g4 >= GQ) break;
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = g4 + e < G ? acc[g4 + e] : 0.f;
                *reinterpret_cast<f32x4 *>(dst + g4) = o;
            }
            return;
        }
    }
    // u_g = W2K^T q_g for query head g = blockIdx.x - nrb: thread (hb, cg)
    // sums 8 consecutive hidden units (one 16-byte load per row) over a slice
    // of head_dim; the slices are then added in LDS
    const int g = (int)blockIdx.x - nrb;
    const int NHB = hid / 8, NCG = 256 / NHB, cper = d / NCG;
    const int hb = tid % NHB, cg = tid / NHB;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int c = cg * cper; c < (cg + 1) * cper; ++c) {
        float v[8];
        load8(w2 + (int64_t)c * hid + 8 * hb, v);
        const float qv = qs[g][c];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[e] * qv;
    }
    float *redf = &red[0][0][0];  // [NCG][hid]
#pragma unroll
    for (int e = 0; e < 8; ++e) redf[cg * hid + 8 * hb + e] = acc[e];
    __syncthreads();
    for (int i = tid; i < hid; i += 256) {
        float sum = 0.f;
        for (int k2 = 0; k2 < NCG; ++k2) sum += redf[k2 * hid + i];
        u[((int64_t)b * Hq + h * G + g) * kMaxH + i] = sum;
    }
    if (tid < 64) {
        float v = 0.f;
        if (b2)
            for (int c = tid; c < d; c += 64) v += qs[g][c] * b2[c];
        v = wave_sum(v);
        if (tid == 0) cq[(int64_t)b * Hq + h * G + g] = v;
    }
}

// Query-aware token selection from the logits a dense decode wrote (the
// selector a sparse attention uses at a filter layer: tokens are ranked by
// the attention they received).  Six launches: the keys, three histogram
// passes, the per-slice counts and the ordered write.
//
// select_keys_kernel, grid (ceil(T / 2048), U), 256 threads: for every
// position p < T of unit u,
//   key_p = sum over the unit's G query heads g of exp(logit_{g,p} - lse_g)
// (the attention probability of p summed over the group) into keys[u][p]
// and, if non-null, scores[u][p]; the counts of the keys' first (most
// significant) byte are added to hist0[u][256], which the merge kernel
// cleared.
constexpr int kKeyPer = 8;  // positions per thread of the key kernel
constexpr int kSelHist = 4 * 256;  // histogram words per unit (four radix passes)
__global__ __launch_bounds__(256) void select_keys_kernel(
    const float *__restrict__ logc, const float *__restrict__ logr,
    const float *__restrict__ lse, int Hq, int G, int H, int64_t T, int64_t Nt, int64_t Rt,
    int s, uint32_t *__restrict__ keys, float *__restrict__ scores,
    uint32_t *__restrict__ hist0) {
    __shared__ uint32_t lh[256];
    const int unit = blockIdx.y, b = unit / H, h = unit % H;
    lh[threadIdx.x] = 0u;
    float lg[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) lg[g] = g < G ? lse[(int64_t)b * Hq + h * G + g] : 0.f;
    const float *lc = logc + (int64_t)unit * G * Nt;
    const float *lr = logr + (int64_t)unit * G * Rt;
    const int64_t p0 = (int64_t)blockIdx.x * (256 * kKeyPer) + threadIdx.x;
    float v[kKeyPer][kMaxG];
#pragma unroll
    for (int e = 0; e < kKeyPer; ++e) {
        const int64_t p = min(p0 + 256 * e, T - 1);
        const bool ref = p % s == 0;
        const float *src = ref ? lr + p / s : lc + (p - ((p - 1) / s + 1));
        const int64_t gs = ref ? Rt : Nt;
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) v[e][g] = g < G ? src[g * gs] : 0.f;
    }
    __syncthreads();  // lh cleared
#pragma unroll
    for (int e = 0; e < kKeyPer; ++e) {
        const int64_t p = p0 + 256 * e;
        if (p >= T) break;
        float sg = 0.f;
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
            if (g < G) sg += __expf(v[e][g] - lg[g]);
        keys[unit * keys_stride(T) + p] = __float_as_uint(sg);
        if (scores) scores[(int64_t)unit * T + p] = sg;
        atomicAdd(&lh[__float_as_uint(sg) >> 24], 1u);
    }
    __syncthreads();
    // the block's counts of the keys' first byte into the unit's histogram
    if (lh[threadIdx.x]) atomicAdd(&hist0[unit * kSelHist + threadIdx.x], lh[threadIdx.x]);
}

// The multi-block radix select that follows the key kernel.  Per unit the
// workspace holds four 256-bin histograms (hist[u][j]: counts of byte 3 - j of
// the keys that share the bytes fixed by passes 0 .. j - 1), cleared by the
// merge kernel; every block re-derives the fixed bytes from them.  Keys of a
// unit are cut into slices of kSelSlice positions, one block each.
constexpr int kSelSlice = 4096;

// prefix / mask of the bytes fixed by the first np passes and rem, the rank
// (from the top, 1-based) of the n_keep-th largest key among the keys that
// share them; sh: 256 + 2 words of LDS; all threads of the block call it.
__device__ __forceinline__ void sel_resolve(const uint32_t *__restrict__ uh, int np,
                                            uint32_t n_keep, uint32_t *sh, uint32_t &prefix,
                                            uint32_t &mask, uint32_t &rem) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    prefix = 0u;
    mask = 0u;
    rem = n_keep;
    for (int j = 0; j < np; ++j) {
        __syncthreads();
        for (int i = tid; i < 256; i += blockDim.x) sh[i] = uh[256 * j + i];
        __syncthreads();
        if (w == 0) {
            // lane l holds bins 255 - 4 l .. 252 - 4 l (from the top)
            uint32_t c[4], tot = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = sh[255 - 4 * lane - i];
                tot += c[i];
            }
            uint32_t inc = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(inc, o, 64);
                if (lane >= o) inc += y;
            }
            const uint32_t excl = inc - tot;
            if (excl < rem && rem <= inc) {
                uint32_t r = rem - excl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (r <= c[i]) {
                        sh[256] = (uint32_t)(255 - 4 * lane - i);
                        sh[257] = r;
                        break;
                    }
                    r -= c[i];
                }
            }
        }
        __syncthreads();
        const int shift = 24 - 8 * j;
        prefix |= sh[256] << shift;
        mask |= 255u << shift;
        rem = sh[257];
    }
    __syncthreads();
}

// Pass `pass` (1..3) of the radix select: the counts of byte 3 - pass of the
// slice's keys that share the bytes fixed so far, added to hist[u][pass].
// grid (slices, U), 256 threads.
__global__ __launch_bounds__(256) void select_hist_kernel(const uint32_t *__restrict__ keys,
                                                          uint32_t *__restrict__ hist, int64_t T,
                                                          int n_keep, int pass) {
    __shared__ uint32_t sh[258];
    __shared__ uint32_t lh[256];
    if (n_keep >= T) return;
    const int unit = blockIdx.y, tid = threadIdx.x;
    uint32_t *uh = hist + (int64_t)unit * kSelHist;
    uint32_t prefix, mask, rem;
    sel_resolve(uh, pass, (uint32_t)n_keep, sh, prefix, mask, rem);
    lh[tid] = 0u;
    __syncthreads();
    const int shift = 24 - 8 * pass;
    const int64_t p0 = (int64_t)blockIdx.x * kSelSlice;
    const uint32_t *ku = keys + (int64_t)unit * keys_stride(T);
    // 16 consecutive keys per thread (16-byte loads; the slice start and the
    // unit's row are multiples of 4 entries)
    constexpr int PER = kSelSlice / 256;
    u32x4 kv[PER / 4];
    const int64_t pt = p0 + (int64_t)tid * PER;
#pragma unroll
    for (int e = 0; e < PER / 4; ++e) {
        const int64_t p = pt + 4 * e;
        kv[e] = p < T ? *reinterpret_cast<const u32x4 *>(ku + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < PER / 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (pt + 4 * e + j < T && (kv[e][j] & mask) == prefix)
                atomicAdd(&lh[(kv[e][j] >> shift) & 255u], 1u);
    __syncthreads();
    if (lh[tid]) atomicAdd(&uh[256 * pass + tid], lh[tid]);
}

// The ordered write.  select_count_kernel: per slice, the numbers of keys
// above the threshold and equal to it (cnt[u][slice][0..1]).
// select_write_kernel: every taken position of the slice at its place in the
// unit's list (position order; of the keys equal to the threshold, the first
// rem of the unit are taken).
__global__ __launch_bounds__(256) void select_count_kernel(const uint32_t *__restrict__ keys,
                                                           const uint32_t *__restrict__ hist,
                                                           int64_t T, int n_keep,
                                                           uint32_t *__restrict__ cnt) {
    __shared__ uint32_t sh[258];
    __shared__ uint32_t red[2][4];
    if (n_keep >= T) return;
    const int unit = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint32_t thr, mask, rem;
    sel_resolve(hist + (int64_t)unit * kSelHist, 4, (uint32_t)n_keep, sh, thr, mask, rem);
    const int64_t p0 = (int64_t)blockIdx.x * kSelSlice;
    const uint32_t *ku = keys + (int64_t)unit * keys_stride(T);
    constexpr int PER = kSelSlice / 256;
    const int64_t pt = p0 + (int64_t)tid * PER;
    uint32_t cg = 0u, ce = 0u;
#pragma unroll
    for (int e = 0; e < PER / 4; ++e) {
        const int64_t p = pt + 4 * e;
        const u32x4 v = p < T ? *reinterpret_cast<const u32x4 *>(ku + p) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool inr = p + j < T;
            cg += (inr && v[j] > thr) ? 1u : 0u;
            ce += (inr && v[j] == thr) ? 1u : 0u;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        cg += __shfl_xor(cg, o, 64);
        ce += __shfl_xor(ce, o, 64);
    }
    if (lane == 0) {
        red[0][w] = cg;
        red[1][w] = ce;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t *c = cnt + ((int64_t)unit * gridDim.x + blockIdx.x) * 2;
        c[0] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        c[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    }
}

__global__ __launch_bounds__(256) void select_write_kernel(const uint32_t *__restrict__ keys,
                                                           const uint32_t *__restrict__ hist,
                                                           const uint32_t *__restrict__ cnt,
                                                           int64_t T, int n_keep,
                                                           int32_t *__restrict__ positions) {
    __shared__ uint32_t sh[258];
    __shared__ uint32_t wtot[4];
    __shared__ uint32_t base[2];
    const int unit = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t *pu = positions + (int64_t)unit * n_keep;
    const int64_t p0 = (int64_t)blockIdx.x * kSelSlice;
    if (n_keep >= T) {
        // every position in order, then -1 (the first slice writes the tail)
        for (int64_t i = p0 + tid; i < min(T, p0 + kSelSlice); i += 256) pu[i] = (int32_t)i;
        if (blockIdx.x == 0)
            for (int64_t i = T + tid; i < n_keep; i += 256) pu[i] = -1;
        return;
    }
    uint32_t thr, mask, rem;
    sel_resolve(hist + (int64_t)unit * kSelHist, 4, (uint32_t)n_keep, sh, thr, mask, rem);
    // taken keys before this slice (slices in order)
    if (w == 0) {
        uint32_t g = 0u, e = 0u;
        for (int i = lane; i < (int)blockIdx.x; i += 64) {
            const uint32_t *c = cnt + ((int64_t)unit * gridDim.x + i) * 2;
            g += c[0];
            e += c[1];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            g += __shfl_xor(g, o, 64);
            e += __shfl_xor(e, o, 64);
        }
        if (lane == 0) {
            base[0] = g;
            base[1] = e;
        }
    }
    __syncthreads();
    const uint32_t *ku = keys + (int64_t)unit * keys_stride(T);
    constexpr int PER = kSelSlice / 256;
    const int64_t pt = p0 + (int64_t)tid * PER;
    u32x4 kv[PER / 4];
#pragma unroll
    for (int e = 0; e < PER / 4; ++e) {
        const int64_t p = pt + 4 * e;
        kv[e] = p < T ? *reinterpret_cast<const u32x4 *>(ku + p) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t cg = 0u, ce = 0u;
#pragma unroll
    for (int e = 0; e < PER / 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool inr = pt + 4 * e + j < T;
            cg += (inr && kv[e][j] > thr) ? 1u : 0u;
            ce += (inr && kv[e][j] == thr) ? 1u : 0u;
        }
    const uint32_t mine = cg | (ce << 16);   // at most 16 per thread
    uint32_t inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    uint32_t before = inc - mine;
#pragma unroll
    for (int i = 0; i < 4; ++i) before += i < w ? wtot[i] : 0u;
    uint32_t g0 = base[0] + (before & 0xffffu), e0 = base[1] + (before >> 16);
#pragma unroll
    for (int e = 0; e < PER / 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t p = pt + 4 * e + j;
            const uint32_t k = kv[e][j];
            if (p < T && k > thr) {
                pu[g0 + min(e0, rem)] = (int32_t)p;
                ++g0;
            } else if (p < T && k == thr) {
                if (e0 < rem) pu[g0 + e0] = (int32_t)p;
                ++e0;
            }
        }
}

// Merge of two normalised attention results over disjoint key sets (the
// compressed cache and exact window rows): with e_i = exp(lse_i - max),
// out = (e_1 out_1 + e_2 out_2) / (e_1 + e_2).  grid B * Hq, d threads.
__global__ __launch_bounds__(kMaxD) void merge2_kernel(const float *__restrict__ o1,
                                                       const float *__restrict__ l1,
                                                       const float *__restrict__ o2,
                                                       const float *__restrict__ l2, int d,
                                                       float *__restrict__ out) {
    const int64_t r = blockIdx.x;
    const int c = threadIdx.x;
    const float a = l1[r], b = l2[r];
    const float m = fmaxf(a, b);
    const float ea = a == -INFINITY ? 0.f : __expf(a - m);
    const float eb = b == -INFINITY ? 0.f : __expf(b - m);
    const float den = ea + eb;
    if (c < d) out[r * d + c] = den > 0.f ? (ea * o1[r * d + c] + eb * o2[r * d + c]) / den : 0.f;
}

// Log-sum-exp merge of the partitions of one query head, then W2V applied to
// the merged hidden sum.  grid (Hq, B).  The merge of the record vectors runs
// with one float4 column per thread and the partitions split across thread
// groups, so all partition loads of a thread are independent.
template <typename T>
__global__ __launch_bounds__(kCombThreads) void combine2_kernel(int Hq, int G, int d, int H, int64_t P,
                                                       const float *__restrict__ part,
                                                       const T *__restrict__ vw2, int vhid,
                                                       const float *__restrict__ vb2,
                                                       float *__restrict__ out,
                                                       float *__restrict__ lse,
                                                       uint32_t *__restrict__ hist0) {
    constexpr int NT = kCombThreads, NW = NT / 64, NGR = 8;
    __shared__ float wgt[kMaxParts];
    __shared__ f32x4 gred[NGR][(kMaxD + kMaxH) / 4];
    __shared__ float accr[kMaxD];
    __shared__ float acch[kMaxH];
    __shared__ float ored[NT / 64][kMaxD];
    __shared__ float red[NW];
    const int gq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int h = gq / G, g = gq % G;
    const int64_t unit = (int64_t)b * H + h;
    const float *base = part + (unit * P * G + g) * kPStride;
    // token selection: the first query head of the group clears the unit's
    // key histogram that the key kernel fills next
    if (hist0 && g == 0)
        for (int i = tid; i < kSelHist; i += NT) hist0[unit * kSelHist + i] = 0u;
    const int64_t pstep = (int64_t)G * kPStride;
    float mx = -INFINITY;
    for (int64_t p = tid; p < P; p += NT) mx = fmaxf(mx, base[p * pstep]);
    // M = -inf only when no partition holds a token (a sparse selection with
    // no valid position): every weight is then 0 and the output row 0
    const float M0 = block_reduce<NW>(mx, red, true);
    const float M = M0 == -INFINITY ? 0.f : M0;
    float lsum = 0.f, ltsum = 0.f;
    for (int64_t p = tid; p < P; p += NT) {
        const float wp = __expf(base[p * pstep] - M);
        wgt[p] = wp;
        lsum += wp * base[p * pstep + 1];
        ltsum += wp * base[p * pstep + 2];
    }
    const float L = block_reduce<NW>(lsum, red, false);
    const float Lt = block_reduce<NW>(ltsum, red, false);  // (its barriers also publish wgt)
    if (lse && tid == 0) lse[(int64_t)b * Hq + gq] = L > 0.f ? M + __logf(L) : -INFINITY;
    // columns: acc_r as d/4 float4s, then acc_h as vhid/4 float4s
    const int ncr = d / 4, nc = ncr + vhid / 4;
    const int ngrp = min(NGR, NT / nc);
    const int col = tid % nc, grp = tid / nc;
    if (grp < ngrp) {
        const int off = col < ncr ? 4 + 4 * col : 4 + kMaxD + 4 * (col - ncr);
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int64_t p = grp; p < P; p += ngrp) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(base + p * pstep + off);
            a += wgt[p] * v;
        }
        gred[grp][col] = a;
    }
    __syncthreads();
    if (tid < nc) {
        f32x4 a = gred[0][tid];
        for (int k2 = 1; k2 < ngrp; ++k2) a += gred[k2][tid];
        float *dst = tid < ncr ? &accr[4 * tid] : &acch[4 * (tid - ncr)];
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = a[e];
    }
    __syncthreads();
    // out[c] = (acc_r[c] + W2V[c] . acc_h + Lt b2V[c]) / L; the hidden sum of
    // a row is split over nsp threads, at least 8 hidden units each
    const int nsp = min(NT / d, vhid / 8);
    const int c = tid % d, sp = tid / d;
    const int oper = vhid / nsp;
    if (sp < nsp) {
        float wsum = 0.f;
        const T *wr = vw2 + (int64_t)c * vhid + sp * oper;
        for (int o = 0; o < oper; o += 8) {
            float v[8];
            load8(wr + o, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) wsum += v[e] * acch[sp * oper + o + e];
        }
        ored[sp][c] = wsum;
    }
    __syncthreads();
    if (tid < d) {
        float ws = 0.f;
        for (int k2 = 0; k2 < nsp; ++k2) ws += ored[k2][tid];
        const float bias = vb2 ? vb2[tid] : 0.f;
        out[((int64_t)b * Hq + gq) * d + tid] = L > 0.f ? (accr[tid] + ws + Lt * bias) / L : 0.f;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core path (bf16 storage, hidden width 128 or 256).
//
// A block owns one KV head (unit) and a range of compressed tokens, walked in
// tiles of 32.  The 4 waves split the hidden units (wave w: [w*HW, (w+1)*HW))
// and the head_dim columns of the value sums (wave w: [w*D/4, (w+1)*D/4)).
// Per tile:
//   K side  hK^T = W1K z^T + b1K           bf16 MFMA, hidden x tokens
//           GELU in packed f16
//           partial scores U hK^T          f16 MFMA, U = W2K^T q (query heads x hidden)
//   merge   scores of the 4 waves + mean_j q.R^K_j (from the qR table) + q.b2K,
//           online softmax per query head (one thread per (head, token))
//   V side  hV = z W1V^T + b1V             bf16 MFMA, tokens x hidden
//           acc_h += P hV                  f16 MFMA
//           acc_r += P~ R^V_gathered       bf16 MFMA over (token, slot) rows; the
//                                          referenced V rows are staged in LDS
// The next tile's latents and index rows are loaded while the current tile
// computes, and the V-row gather is issued at the start of the tile so its
// latency hides behind the K side.  Reference tokens are separate partitions
// (VALU), as in the general path.
//
// LDS layouts: V rows are stored row-major with their 16-byte chunks XOR-
// swizzled by 2 * (row % 4), so that the transposing reads of the B operand
// (4 consecutive rows x 32 bytes per 16-lane group) fall in disjoint banks;
// the per-head weight rows carry 16 bytes of padding for the same reason.
template <int D, int DC, int HID, int KP, bool SP>
__global__ __launch_bounds__(256, 2) void main_mfma_kernel(
    int U, int Hq, int G, int k, int64_t Rcap, int64_t Ncap, int64_t Rt, int64_t Nt,
    int tiles_per_part, int Ptok, int P, const bf16_t *__restrict__ klat,
    const uint16_t *__restrict__ kidx, const bf16_t *__restrict__ vref,
    const bf16_t *__restrict__ vlat, const uint16_t *__restrict__ vidx,
    const bf16_t *__restrict__ kw1, const float *__restrict__ kb1,
    const bf16_t *__restrict__ vw1, const float *__restrict__ vb1, float scale,
    const float *__restrict__ ubuf, const float *__restrict__ cq, const float *__restrict__ qr,
    float *__restrict__ part, const int32_t *__restrict__ sord, const int32_t *__restrict__ scnt,
    int nsel, float *__restrict__ logc, float *__restrict__ logr) {
    constexpr int TT = 32;              // tokens per tile
    constexpr int HW = HID / 4;         // hidden units per wave
    constexpr int MT = HW / 16;         // 16-row hidden tiles per wave
    constexpr int KJ = HW / 32;         // 32-wide hidden k-steps per wave
    constexpr int KS = (DC + 31) / 32;  // 32-wide latent k-steps
    constexpr int DW = D / 4;           // value columns per wave
    constexpr int NR = DW / 16;
    constexpr int ROWS = TT * KP;       // gathered (token, slot) rows per tile
    constexpr int CH = D / 8;           // 16-byte chunks per V row
    constexpr int GIT = ROWS * CH / 256;  // gather chunks per thread
    constexpr int WPAD = ROWS + 8;
    constexpr int NB = (ROWS * D * 2 <= 32768) ? 2 : 1;  // V-row buffers
    static_assert(HW % 32 == 0, "hidden width per wave must be a multiple of 32");
    static_assert((ROWS * CH) % 256 == 0, "gather must split evenly");

    __shared__ float sp[4][kMaxG][TT + 4];
    __shared__ float alpha_s[kMaxG];
    __shared__ __attribute__((aligned(16))) _Float16 pperm[kMaxG][TT + 8];
    __shared__ __attribute__((aligned(16))) bf16_t wrow[kMaxG][WPAD];
    // V rows of the current and the next tile (two objects, so the compiler
    // can tell an LDS fill of one from reads of the other)
    __shared__ __attribute__((aligned(16))) bf16_t vrowA[ROWS][D];
    __shared__ __attribute__((aligned(16))) bf16_t vrowB[NB == 2 ? ROWS : 1][D];
    __shared__ __attribute__((aligned(16))) float bias_k[HID];
    __shared__ float bias_v[HID];
    // first Decompressor layers (K, V) as LDS operand tiles only when the V-row
    // tile is single-buffered; rows padded by 16 bytes against bank conflicts
    constexpr bool WL = NB == 1 && 2 * HID * (KS * 32 + 8) * 2 <= 40960;
    __shared__ __attribute__((aligned(16))) bf16_t w1s[WL ? 2 : 1][WL ? HID : 1][KS * 32 + 8];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int unit = blockIdx.x % U;
    const int pidx = blockIdx.x / U;
    const int H = Hq / G;
    const int h = unit % H;
    const int bseq = unit / H;
    float *prec = part + (((int64_t)unit * P + pidx) * G) * kPStride;

    const int hbase = w * HW;
    const int cbase = w * DW;
    const bf16_t *vref_u = vref + (int64_t)unit * Rcap * D;
    const int GQ = qr_heads(G);
    const float *qr_u = qr + (int64_t)unit * qr_rows(Rt) * GQ;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // Sparse mode (SP): the block walks the unit's lists of selected
    // compressed-token ordinals (sord[0][unit]) and reference ordinals
    // (sord[1][unit]) instead of consecutive ordinals; the list lengths are
    // the unit's counts.  Ranges below are list positions, ord_c / the
    // reference lookups map them to ordinals.
    const int32_t *cord_u = SP ? sord + (int64_t)unit * nsel : nullptr;
    const int32_t *rord_u = SP ? sord + ((int64_t)U + unit) * nsel : nullptr;
    const int64_t Nt_u = SP ? (int64_t)scnt[2 * unit] : Nt;
    const int64_t Rt_u = SP ? (int64_t)scnt[2 * unit + 1] : Rt;
    // a sparse partition's compressed-token ordinals, staged in LDS once
    __shared__ int32_t ordl[SP ? kSpTiles * TT : 1];
    const int64_t qa_ = (int64_t)pidx * tiles_per_part * TT;
    const int64_t qe_ = min(Nt_u, qa_ + (int64_t)tiles_per_part * TT);
    // per-unit bases; all in-loop offsets are 32-bit
    const bf16_t *klat_u = klat + (int64_t)unit * Ncap * DC;
    const bf16_t *vlat_u = vlat + (int64_t)unit * Ncap * DC;
    const uint16_t *kidx_u = kidx + (int64_t)unit * Ncap * k;
    const uint16_t *vidx_u = vidx + (int64_t)unit * Ncap * k;
    const int qa32 = (int)qa_, qe32 = (int)qe_;
    const bool gl = l16 < G;  // lane carries a query-head row of the P operands

    f32x4 acc_h[MT], acc_r[NR];
#pragma unroll
    for (int n = 0; n < MT; ++n) acc_h[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NR; ++n) acc_r[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // softmax role: (query head sg, token st)
    const int sg = tid >> 5, st = tid & 31;
    const bool sg_ok = sg < G;
    float m_run = -INFINITY, l_run = 0.f;

    // V rows of one tile straight into LDS (global -> LDS, 16 bytes per lane,
    // the lanes of a wave fill consecutive 16-byte slots); the XOR swizzle is
    // applied on the source side.  gr holds the raw index entries of this
    // thread's chunks; slots that are past the range or unused load row 0
    // (their weight is 0).
    auto issue_gather = [&](int t0, const uint32_t (&gr)[GIT], bf16_t (*dst)[D]) {
#pragma unroll
        for (int m = 0; m < GIT; ++m) {
            const int it = tid + 256 * m;
            const int row = it / CH, c8 = it % CH;
            const int t = row / KP, i = row % KP;
            const int sc8 = c8 ^ (2 * (row & 3));
            const bool ok = t0 + t < qe32 && i < k && gr[m] != kIdxUnused;
            __builtin_amdgcn_global_load_lds(
                (const void *)(vref_u + (uint32_t)((ok ? gr[m] : 0u) * D + 8 * sc8)),
                (__attribute__((address_space(3))) void *)&dst[(256 * m + 64 * w) / CH][0],
                16, 0, 0);
        }
    };

    if (pidx >= Ptok) {
        // ---------------- reference tokens ----------------
        // A reference token is attended with its stored rows: score
        // scale * qR[j], value R^V_j.  Tiles of 32 consecutive references:
        // the rows go straight to LDS and enter the same value MFMA with one
        // slot per token and weight p.
        const int64_t ja = (int64_t)(pidx - Ptok) * kRefPart;
        const int64_t je = min(Rt_u, ja + kRefPart);
        for (int64_t j0 = ja; j0 < je; j0 += TT) {
            __syncthreads();
#pragma unroll
            for (int m = 0; m < (TT * CH) / 256; ++m) {
                const int it = tid + 256 * m;
                const int row = it / CH, c8 = it % CH;
                const int sc8 = c8 ^ (2 * (row & 3));
                const int64_t j = SP ? (int64_t)rord_u[min(j0 + row, je - 1)]
                                     : min(j0 + row, Rt - 1);
                __builtin_amdgcn_global_load_lds(
                    (const void *)(vref_u + j * D + 8 * sc8),
                    (__attribute__((address_space(3))) void *)&vrowA[(256 * m + 64 * w) / CH][0],
                    16, 0, 0);
            }
            if (sg_ok) {
                const bool ok = j0 + st < je;
                const int64_t jr = SP ? (int64_t)rord_u[min(j0 + st, je - 1)] : j0 + st;
                const float s = ok ? scale * qr_u[jr * GQ + sg] : -INFINITY;
                if (!SP && logr && ok) logr[((int64_t)unit * G + sg) * Rt + j0 + st] = s;
                float tmax = s;
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 32));
                const float mnew = fmaxf(m_run, tmax);
                const float alpha = __expf(m_run - mnew);
                const float pv = ok ? __expf(s - mnew) : 0.f;
                float psum = pv;
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 32);
                l_run = l_run * alpha + psum;
                m_run = mnew;
                if (st == 0) alpha_s[sg] = alpha;
                wrow[sg][st] = f2bf(pv);
            }
            wait_vm_all();
            __syncthreads();
            float al[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) al[r] = (4 * lq + r < G) ? alpha_s[4 * lq + r] : 0.f;
#pragma unroll
            for (int n = 0; n < NR; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc_r[n][r] *= al[r];
            const int rb = 8 * lq;
            const bf16x8 pw = as_bf16x8(gl ? *reinterpret_cast<const u32x4 *>(&wrow[l16][rb]) : zero4);
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                const int c = cbase + 16 * n + 4 * (l16 & 3);
                const int pcol = (((c >> 3) ^ (2 * (l16 >> 2))) << 3) | (c & 7);
                const u32x2 lo = lds_read_tr16(&vrowA[rb + (l16 >> 2)][pcol]);
                const u32x2 hi = lds_read_tr16(&vrowA[rb + 4 + (l16 >> 2)][pcol]);
                const u32x4 bv = {lo[0], lo[1], hi[0], hi[1]};
                acc_r[n] = mfma16_bf16(pw, as_bf16x8(bv), acc_r[n]);
            }
        }
        if (sg_ok && st == 0) {
            prec[(int64_t)sg * kPStride + 0] = m_run;
            prec[(int64_t)sg * kPStride + 1] = l_run;
            prec[(int64_t)sg * kPStride + 2] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int g = 4 * lq + r;
            if (g >= G) continue;
            float *pg = prec + (int64_t)g * kPStride;
#pragma unroll
            for (int n = 0; n < MT; ++n) pg[4 + kMaxD + hbase + 16 * n + l16] = 0.f;
#pragma unroll
            for (int n = 0; n < NR; ++n) pg[4 + cbase + 16 * n + l16] = acc_r[n][r];
        }
        return;
    }

    // ---------------- compressed tokens (matrix cores) ----------------
    if (SP && qa32 >= qe32) {
        // a partition past the end of this unit's list: a neutral record
        for (int i = tid; i < G * kPStride; i += 256)
            prec[i] = (i % kPStride == 0) ? -INFINITY : 0.f;
        return;
    }
    // weights into registers
    bf16x8 wK[WL ? 1 : MT][KS], wV[WL ? 1 : MT][KS];
    if constexpr (WL) {
        // rows of W1K / W1V, zero-padded to whole 32-wide k-steps
        for (int i = tid; i < 2 * HID * KS * 4; i += 256) {
            const int mat = i / (HID * KS * 4), rem = i % (HID * KS * 4);
            const int row = rem / (KS * 4), c8 = rem % (KS * 4);
            const bf16_t *src = mat == 0 ? kw1 : vw1;
            *reinterpret_cast<u32x4 *>(&w1s[mat][row][8 * c8]) =
                8 * c8 < DC ? ld16(src + (int64_t)row * DC + 8 * c8) : zero4;
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = 32 * ks + 8 * lq;
                wK[m][ks] = as_bf16x8(ch < DC ? ld16(kw1 + (int64_t)(hbase + 16 * m + l16) * DC + ch)
                                              : zero4);
                wV[m][ks] = as_bf16x8(ch < DC ? ld16(vw1 + (int64_t)(hbase + 16 * m + l16) * DC + ch)
                                              : zero4);
            }
        }
    }
    auto w1op = [&](int mat, int m, int ks) -> bf16x8 {
        if constexpr (WL)
            return as_bf16x8(*reinterpret_cast<const u32x4 *>(
                &w1s[mat][hbase + 16 * m + l16][32 * ks + 8 * lq]));
        else
            return mat == 0 ? wK[m][ks] : wV[m][ks];
    };
    for (int i = tid; i < HID; i += 256) {
        bias_k[i] = kb1 ? kb1[i] : 0.f;
        bias_v[i] = vb1 ? vb1[i] : 0.f;
    }
    if constexpr (SP)
        for (int i = tid; i < qe32 - qa32; i += 256) ordl[i] = cord_u[qa32 + i];
    __syncthreads();
    auto ord_c = [&](int i) -> uint32_t { return SP ? (uint32_t)ordl[i - qa32] : (uint32_t)i; };
    // U = W2K^T q in f16, hidden permuted to match the hK^T operand layout
    f16x8 uA[KJ];
    {
        const float *ug = ubuf + ((int64_t)bseq * Hq + h * G + (gl ? l16 : 0)) * kMaxH;
        float uv[KJ][8];
#pragma unroll
        for (int j = 0; j < KJ; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                uv[j][e] = ug[hbase + 32 * j + (e < 4 ? 4 * lq + e : 16 + 4 * lq + (e - 4))];
        const float gm = gl ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < KJ; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) uA[j][e] = (_Float16)(uv[j][e] * gm);
    }
    const float cq_g = sg_ok ? cq[(int64_t)bseq * Hq + h * G + sg] : 0.f;
    // inverse of the token permutation of the P operand
    const int st_slot = st < 16 ? 8 * (st >> 2) + (st & 3) : 8 * ((st - 16) >> 2) + 4 + (st & 3);


    // ---- loaders.  Loads go to clamped, always-valid addresses and keep
    // their raw values; validity is applied where the values are used (a
    // tile later), so no load forces an early wait.
    struct TileIn {
        uint32_t ik[KP], iv[KP];   // the softmax thread's token's K / V index rows
        bf16x8 zk[2][KS], zv[2][KS];
    };
    auto load_tile = [&](int t0, TileIn &T) {
        const uint32_t tk = ord_c(min(t0 + st, qe32 - 1));
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const uint32_t ic = (uint32_t)(i < k ? i : k - 1);
            T.ik[i] = kidx_u[tk * k + ic];
            T.iv[i] = vidx_u[tk * k + ic];
        }
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            const uint32_t tz = ord_c(min(t0 + 16 * n2 + l16, qe32 - 1));  // tail: a valid row
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = 32 * ks + 8 * lq;
                T.zk[n2][ks] = as_bf16x8(ch < DC ? ld16(klat_u + (tz * DC + ch)) : zero4);
                T.zv[n2][ks] = as_bf16x8(ch < DC ? ld16(vlat_u + (tz * DC + ch)) : zero4);
            }
        }
    };
    auto load_rows = [&](int t0, uint32_t (&gr)[GIT]) {
#pragma unroll
        for (int m = 0; m < GIT; ++m) {
            const int row = (tid + 256 * m) / CH;
            const int t = row / KP, i = row % KP;
            const uint32_t tk = ord_c(min(t0 + t, qe32 - 1));
            gr[m] = vidx_u[tk * k + (uint32_t)(i < k ? i : k - 1)];
        }
    };

    // ---- one tile: T holds its inputs; the next tile's inputs go to Tn, the
    // V-row ordinals of the tile after that to grn; gr are the next tile's
    auto tile = [&](auto bufc, int q0, TileIn &T, TileIn &Tn, const uint32_t (&gr)[GIT],
                    uint32_t (&grn)[GIT]) {
        constexpr int BUF = decltype(bufc)::value;
        bf16_t (*cur)[D] = (NB == 2 && BUF == 1) ? vrowB : vrowA;
        bf16_t (*nxt)[D] = (NB == 2 && BUF == 0) ? vrowB : vrowA;
        const bool tok_ok = q0 + st < qe32;
        // qR of this tile's references (latency hides behind the K side)
        float qv[KP];
        int kek = 0;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const bool ok = sg_ok && i < k && T.ik[i] != kIdxUnused;
            qv[i] = qr_u[(uint32_t)((ok ? T.ik[i] : 0u) * GQ + (sg_ok ? sg : 0))];
            qv[i] = ok ? qv[i] : 0.f;
            kek += ok;
        }
        // ---- K side: hidden tile (hidden x tokens), GELU, partial scores.
        // All hidden-tile products are issued before any GELU reads them.
        f32x4 cK[2][MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const f32x4 bk = *reinterpret_cast<const f32x4 *>(&bias_k[hbase + 16 * m + 4 * lq]);
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2) {
                cK[n2][m] = bk;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    cK[n2][m] = mfma16_bf16(w1op(0, m, ks), T.zk[n2][ks], cK[n2][m]);
            }
        }
        f32x4 S[2];
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            S[n2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const f16x2 h0 = gelu2_f16(cK[n2][2 * j][0], cK[n2][2 * j][1]);
                const f16x2 h1 = gelu2_f16(cK[n2][2 * j][2], cK[n2][2 * j][3]);
                const f16x2 h2 = gelu2_f16(cK[n2][2 * j + 1][0], cK[n2][2 * j + 1][1]);
                const f16x2 h3 = gelu2_f16(cK[n2][2 * j + 1][2], cK[n2][2 * j + 1][3]);
                u32x4 hv = {as_u32(h0), as_u32(h1), as_u32(h2), as_u32(h3)};
                S[n2] = mfma16_f16(uA[j], as_f16x8(hv), S[n2]);
            }
        }
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int g = 4 * lq + r;
                if (g < G) sp[w][g][16 * n2 + l16] = S[n2][r];
            }
        wait_vm_all();  // this tile's V rows landed
        __syncthreads();
        // every wave is past the previous tile's V side: the other V-row
        // buffer is free for the next tile
        const bool more = q0 + TT < qe32;
        if (NB == 2 && more) issue_gather(q0 + TT, gr, nxt);

        // ---- merge scores, online softmax (thread = (query head sg, token st))
        if (sg_ok) {
            float s = -INFINITY;
            if (tok_ok) {
                float rs = 0.f;
#pragma unroll
                for (int i = 0; i < KP; ++i) rs += qv[i];
                s = scale * (sp[0][sg][st] + sp[1][sg][st] + sp[2][sg][st] + sp[3][sg][st] +
                             rs / (float)kek + cq_g);
                if (!SP && logc) logc[((int64_t)unit * G + sg) * Nt + q0 + st] = s;
            }
            float tmax = s;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 32));
            const float mnew = fmaxf(m_run, tmax);
            const float alpha = __expf(m_run - mnew);
            const float pv = tok_ok ? __expf(s - mnew) : 0.f;
            float psum = pv;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 32);
            l_run = l_run * alpha + psum;
            m_run = mnew;
            if (st == 0) alpha_s[sg] = alpha;
            pperm[sg][st_slot] = (_Float16)pv;
            int kev = 0;
#pragma unroll
            for (int i = 0; i < KP; ++i) kev += (i < k && T.iv[i] != kIdxUnused);
            const float wv = kev > 0 ? pv / (float)kev : 0.f;
#pragma unroll
            for (int i = 0; i < KP; ++i)
                wrow[sg][st * KP + i] = (i < k && T.iv[i] != kIdxUnused) ? f2bf(wv) : (bf16_t)0;
        }
        __syncthreads();

        // ---- the next tile's loads (their latency hides behind the V side)
        if (more) {
            load_tile(q0 + TT, Tn);
            load_rows(q0 + 2 * TT, grn);
        }

        // ---- V side
        {
            float al[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) al[r] = (4 * lq + r < G) ? alpha_s[4 * lq + r] : 0.f;
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc_h[n][r] *= al[r];
#pragma unroll
            for (int n = 0; n < NR; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc_r[n][r] *= al[r];
        }
        const f16x8 pa = as_f16x8(gl ? *reinterpret_cast<const u32x4 *>(&pperm[l16][8 * lq]) : zero4);
        f32x4 cV[MT][2];
#pragma unroll
        for (int n = 0; n < MT; ++n) {
            const float bv_ = bias_v[hbase + 16 * n + l16];
            cV[n][0] = f32x4{bv_, bv_, bv_, bv_};
            cV[n][1] = cV[n][0];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 wv_ = w1op(1, n, ks);
                cV[n][0] = mfma16_bf16(T.zv[0][ks], wv_, cV[n][0]);
                cV[n][1] = mfma16_bf16(T.zv[1][ks], wv_, cV[n][1]);
            }
        }
#pragma unroll
        for (int n = 0; n < MT; ++n) {
            const f16x2 h0 = gelu2_f16(cV[n][0][0], cV[n][0][1]);
            const f16x2 h1 = gelu2_f16(cV[n][0][2], cV[n][0][3]);
            const f16x2 h2 = gelu2_f16(cV[n][1][0], cV[n][1][1]);
            const f16x2 h3 = gelu2_f16(cV[n][1][2], cV[n][1][3]);
            u32x4 hv = {as_u32(h0), as_u32(h1), as_u32(h2), as_u32(h3)};
            acc_h[n] = mfma16_f16(pa, as_f16x8(hv), acc_h[n]);
        }
        // value reference rows: acc_r += P~ R, P~[g][row] = p[g][t] / k_eff(t)
#pragma unroll
        for (int ks = 0; ks < ROWS / 32; ++ks) {
            const int rb = 32 * ks + 8 * lq;
            const bf16x8 pw = as_bf16x8(gl ? *reinterpret_cast<const u32x4 *>(&wrow[l16][rb]) : zero4);
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                // B operand: rows rb .. rb+7 of column cbase + 16 n + l16, two
                // transposing reads (rows rb + l16/4 and rb + 4 + l16/4)
                const int c = cbase + 16 * n + 4 * (l16 & 3);
                const int pcol = (((c >> 3) ^ (2 * (l16 >> 2))) << 3) | (c & 7);
                const u32x2 lo = lds_read_tr16(&cur[rb + (l16 >> 2)][pcol]);
                const u32x2 hi = lds_read_tr16(&cur[rb + 4 + (l16 >> 2)][pcol]);
                const u32x4 bv = {lo[0], lo[1], hi[0], hi[1]};
                acc_r[n] = mfma16_bf16(pw, as_bf16x8(bv), acc_r[n]);
            }
        }
        if (NB == 1 && more) {
            __syncthreads();  // single V-row buffer: every wave is done reading it
            issue_gather(q0 + TT, gr, vrowA);
        }
    };

    // ---- pipeline: prologue, then tiles in pairs with ping-pong register sets
    TileIn TA, TB;
    uint32_t g0[GIT], g1[GIT];
    {
        uint32_t gfirst[GIT];
        load_rows(qa32, gfirst);
        load_tile(qa32, TA);
        load_rows(qa32 + TT, g1);
        issue_gather(qa32, gfirst, vrowA);
    }
    for (int q0 = qa32; q0 < qe32; q0 += 2 * TT) {
        tile(std::integral_constant<int, 0>(), q0, TA, TB, g1, g0);
        if (q0 + TT < qe32) tile(std::integral_constant<int, 1>(), q0 + TT, TB, TA, g0, g1);
    }

    // ---- partial record: m, l, l over compressed tokens, acc_r[d], acc_h[hidden]
    if (sg_ok && st == 0) {
        prec[(int64_t)sg * kPStride + 0] = m_run;
        prec[(int64_t)sg * kPStride + 1] = l_run;
        prec[(int64_t)sg * kPStride + 2] = l_run;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int g = 4 * lq + r;
        if (g >= G) continue;
        float *pg = prec + (int64_t)g * kPStride;
#pragma unroll
        for (int n = 0; n < MT; ++n) pg[4 + kMaxD + hbase + 16 * n + l16] = acc_h[n][r];
#pragma unroll
        for (int n = 0; n < NR; ++n) pg[4 + cbase + 16 * n + l16] = acc_r[n][r];
    }
}

// ---------------------------------------------------------------------------
// Wave-specialised matrix-core path (bf16 storage, k = 4, d_c <= 32, hidden
// width 128 or 256).
//
// Waves 0 and 1 ("score waves") each own 16 of a tile's 32 tokens and the
// whole hidden width of the K Decompressor:
//   hK^T = W1K z^T + b1K   bf16 MFMA (hidden x 16 tokens), bias from LDS as C
//   GELU                   packed f16
//   scores U hK^T          f16 MFMA, U = W2K^T q (query heads x hidden)
//   + mean_j q.R^K_j + q.b2K, then the online softmax of those 16 tokens.
// Softmax weights are taken relative to a reference maximum per query head:
// the larger of the two waves' maxima published with the previous tile.  A
// wave raises its own only when one of its scores exceeds that by more than
// kSlack (a wave-wide vote; then a row reduction), so in the common tile both
// waves use the same reference, no cross-lane reduction runs, and p stays
// below e^kSlack.  Per tile each score wave publishes, in LDS, p (f16, per
// token), p / k_eff (bf16, per (token, slot) row of the value gather) and the
// maxima it used, and keeps its own running sum.
//
// Waves 2 and 3 ("value waves") each own half of the V hidden units and half
// of the value columns for all 32 tokens:
//   hV = z W1V^T + b1V     bf16 MFMA (tokens x hidden), bias as C
//   GELU                   packed f16
//   acc_h += P hV          f16 MFMA (16x16x16), one per score wave's tokens
//   acc_r += P~ R^V        bf16 MFMA over the gathered (token, slot) rows
// Their accumulators are relative to the larger published maximum and are
// rescaled only when it moves; in a tile where the two waves' maxima differ,
// the weights of the lower one are scaled down first.  The referenced
// V rows go global -> LDS by DMA (16-byte chunks, XOR swizzle on the source
// side), double-buffered.
//
// Schedule: the score waves run one tile ahead.  Between two barriers the
// score waves produce tile i+1 while the value waves consume tile i and gather
// the V rows of tile i+1 into the other buffer: one barrier per tile.
// Reference tokens are separate partitions handled by all four waves.
constexpr float kSlack = 8.f;

// EG: groups of 4 query heads per KV head (1 for G <= 4, 2 for G <= 8).
// KX: references per token (k = 4 or k = 8).
// PG: paged caches (K and V share the block table in pm): the unit's table row
// is staged in LDS; a tile's latent and index rows lie in one page (tiles and
// pages are whole multiples of 32 tokens), and each gathered or reference row
// is looked up by its ordinal.
template <int D, int DC, int HID, int EG, int KX, bool SP, bool Q4, bool PG>
__global__ __launch_bounds__(256, 2) void main_ws_kernel(
    int U, int Hq, int G, int64_t Rcap, int64_t Ncap, int64_t Rt, int64_t Nt,
    int tiles_per_part, int Ptok, int P, const bf16_t *__restrict__ klat,
    const uint16_t *__restrict__ kidx, const bf16_t *__restrict__ vref,
    const bf16_t *__restrict__ vlat, const uint16_t *__restrict__ vidx,
    const bf16_t *__restrict__ kw1, const float *__restrict__ kb1,
    const bf16_t *__restrict__ vw1, const float *__restrict__ vb1, float scale,
    const float *__restrict__ ubuf, const float *__restrict__ cq, const float *__restrict__ qr,
    float *__restrict__ part, float *__restrict__ logc, float *__restrict__ logr,
    const int32_t *__restrict__ sord, const int32_t *__restrict__ scnt, int nsel, PageMap pm) {
    constexpr int TT = 32;             // tokens per tile
    constexpr int TH = 16;             // tokens per score wave
    constexpr int MB = HID / 16;       // 16-row hidden blocks (score waves)
    constexpr int KJ = HID / 32;       // 32-wide hidden steps of the score product
    constexpr int HV = HID / 2;        // hidden units per value wave
    constexpr int NBV = HV / 16;
    constexpr int DV = D / 2;          // value columns per value wave
    constexpr int NC = DV / 16;
    constexpr int ROWS = TT * KX;      // gathered V rows per tile
    constexpr int BROWS = 128;         // rows per LDS buffer (a tile at k = 4, half at 8)
    constexpr int WH = KX == 4 ? 16 : 4 * EG;  // query-head rows kept of the row weights
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int RPD = 64 / CH;       // rows per gather instruction
    constexpr int NDMA = (ROWS / 2) / RPD;  // gather instructions per value wave per tile
    constexpr int WR = ROWS + 8;       // padded weight row (bf16)
    constexpr int PR = TH + 4;         // padded p row (f16)
    static_assert(DC <= 32, "one 32-wide latent step");
    static_assert(HID == 128 || HID == 256, "hidden width");
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(KX == 4 || KX == 8, "references per token");
    static_assert(!(PG && (SP || Q4)), "paged caches: dense calls with latents in bf16");
    using IdxV = typename std::conditional<KX == 4, u32x2, u32x4>::type;

    // V rows of two tiles: two objects, so the compiler can tell the DMA fill
    // of one from reads of the other (one array would make it wait for the
    // fill before every read)
    __shared__ __attribute__((aligned(16))) bf16_t vbufA[BROWS][D];
    __shared__ __attribute__((aligned(16))) bf16_t vbufB[BROWS][D];
    __shared__ __attribute__((aligned(16))) bf16_t wr[2][WH][WR];
    __shared__ __attribute__((aligned(16))) _Float16 pw[2][2][16][PR];
    __shared__ __attribute__((aligned(16))) float msl[2][2][16];
    __shared__ __attribute__((aligned(16))) float biask[HID];
    __shared__ float lfin[2][16], mfin[2][16];
    __shared__ float alpha_s[kMaxG];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int unit = blockIdx.x % U;
    const int pidx = blockIdx.x / U;
    const int H = Hq / G;
    const int h = unit % H;
    const int bseq = unit / H;
    const int GQ = qr_heads(G);
    float *prec = part + (((int64_t)unit * P + pidx) * G) * kPStride;
    const bf16_t *vref_u = vref + (int64_t)unit * Rcap * D;
    const float *qr_u = qr + (int64_t)unit * qr_rows(Rt) * GQ;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // sparse mode (SP): list positions of the unit's selected compressed-token
    // ordinals (sord[0][unit]) and reference ordinals (sord[1][unit]) replace
    // consecutive ordinals; the lists' lengths are the unit's counts
    const int32_t *cord_u = SP ? sord + (int64_t)unit * nsel : nullptr;
    const int32_t *rord_u = SP ? sord + ((int64_t)U + unit) * nsel : nullptr;
    // counts mode (not SP, scnt non-null): consecutive ordinals, but each unit
    // holds only scnt[unit] tokens (a batch of sequences of different lengths)
    const bool cmode = !SP && scnt != nullptr;
    const int64_t Nt_u = (SP || cmode) ? (int64_t)scnt[2 * unit] : Nt;
    const int64_t Rt_u = (SP || cmode) ? (int64_t)scnt[2 * unit + 1] : Rt;
    __shared__ int32_t ordl[SP ? kSpTiles * 32 : 1];
    // paged layout: the unit's block-table row, clamped into the pool, held
    // as byte shifts of the reference pool: entry lp is (page - lp) P 2D, so
    // that reference j lies at byte j 2D + ptab[j / P] of the pool (32-bit
    // arithmetic: the pool holds at most 2 GiB, so the shifts fit an int32
    // and the offsets an unsigned one); the page itself is lp + ptab[lp] >>
    // (log2 P + log2 2D)
    constexpr int LRB = D == 128 ? 8 : 7;   // log2 of a row's bytes
    __shared__ int32_t ptab[PG ? kMaxPages : 1];
    // the score waves, which read every token's V index entries a tile ahead
    // anyway, turn them into the byte offsets of the V rows (pool offsets for
    // paged caches; one entry per (token, slot) row) for the value waves'
    // gathers of that tile, which then need no index loads of their own after
    // the first tile (two slots: the value waves gather tile i + 1 while the
    // score waves write tile i + 2).  At k = 4 only: at k = 8 the value waves
    // gather a tile at its start, and reading 32 offsets per lane from LDS
    // there puts the LDS latency ahead of every gather (measured 15% slower
    // than their own index loads, issued a tile ahead)
    constexpr bool PGS = KX == 4;
    __shared__ uint32_t voff[PGS ? 2 : 1][PGS ? 32 * KX : 1];
    if constexpr (PG) {
        for (int i = tid; i < (int)pm.maxp; i += 256)
            ptab[i] = (int32_t)((pg_page(pm, unit, i) - i) << (pm.lg + LRB));
        __syncthreads();
    }
    // byte offset of reference row j (paged: in the pool; else in the unit's rows)
    auto ref_off = [&](uint32_t j) -> uint32_t {
        if constexpr (PG)
            return j * (uint32_t)(D * 2) + (uint32_t)ptab[j >> pm.lg];
        else
            return j * (uint32_t)(D * 2);
    };

    // ---------------- reference tokens ----------------
    // Reference partition r: rows [r kRefPart, (r + 1) kRefPart) of the unit,
    // record rec.  Score scale * qR[j], value = the stored row.  Tiles of 32
    // references, rows straight to LDS; the four waves split the value columns.
    auto ref_part = [&](int r, float *rec) {
        constexpr int NR = D / 64;
        const int sg = tid >> 5, st = tid & 31;
        const bool sg_ok = sg < G;
        const bool gl = l16 < G;
        const int cbase = w * (D / 4);
        float m_run = -INFINITY, l_run = 0.f;
        f32x4 acc[NR];
#pragma unroll
        for (int n = 0; n < NR; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t ja = (int64_t)r * kRefPart;
        const int64_t je = min(Rt_u, ja + kRefPart);
        for (int64_t j0 = ja; j0 < je; j0 += TT) {
            __syncthreads();
#pragma unroll
            for (int m = 0; m < (TT * CH) / 256; ++m) {
                const int it = tid + 256 * m;
                const int row = it / CH, c8 = it % CH;
                const int sc8 = c8 ^ (2 * (row & 3));
                const int64_t j = SP ? (int64_t)rord_u[min(j0 + row, je - 1)]
                                     : min(j0 + row, je - 1);
                __builtin_amdgcn_global_load_lds(
                    (const void *)(PG ? (const char *)vref + (ref_off((uint32_t)j) + 16u * sc8)
                                      : (const char *)(vref_u + j * D + 8 * sc8)),
                    (__attribute__((address_space(3))) void *)&vbufA[(256 * m + 64 * w) / CH][0],
                    16, 0, 0);
            }
            if (sg_ok) {
                const bool ok = j0 + st < je;
                const int64_t jr = SP ? (int64_t)rord_u[min(j0 + st, je - 1)] : j0 + st;
                const float s = ok ? scale * qr_u[jr * GQ + sg] : -INFINITY;
                if (!SP && logr && ok) logr[((int64_t)unit * G + sg) * Rt + j0 + st] = s;
                float tmax = s;
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 32));
                const float mnew = fmaxf(m_run, tmax);
                const float alpha = __expf(m_run - mnew);
                const float pv = ok ? __expf(s - mnew) : 0.f;
                float psum = pv;
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 32);
                l_run = l_run * alpha + psum;
                m_run = mnew;
                if (st == 0) alpha_s[sg] = alpha;
                wr[0][sg][st] = f2bf(pv);
            }
            wait_vm_all();
            __syncthreads();
            float al[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) al[r] = (4 * lq + r < G) ? alpha_s[4 * lq + r] : 0.f;
#pragma unroll
            for (int n = 0; n < NR; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[n][r] *= al[r];
            const int rb = 8 * lq;
            const bf16x8 pwv =
                as_bf16x8(gl ? *reinterpret_cast<const u32x4 *>(&wr[0][min(l16, WH - 1)][rb]) : zero4);
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                const int c = cbase + 16 * n + 4 * (l16 & 3);
                const int pcol = (((c >> 3) ^ (2 * (l16 >> 2))) << 3) | (c & 7);
                const u32x2 lo = lds_read_tr16(&vbufA[rb + (l16 >> 2)][pcol]);
                const u32x2 hi = lds_read_tr16(&vbufA[rb + 4 + (l16 >> 2)][pcol]);
                const u32x4 bv = {lo[0], lo[1], hi[0], hi[1]};
                acc[n] = mfma16_bf16(pwv, as_bf16x8(bv), acc[n]);
            }
        }
        if (sg_ok && st == 0) {
            rec[(int64_t)sg * kPStride + 0] = m_run;
            rec[(int64_t)sg * kPStride + 1] = l_run;
            rec[(int64_t)sg * kPStride + 2] = 0.f;
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int g = 4 * lq + rr;
            if (g >= G) continue;
            float *pg = rec + (int64_t)g * kPStride;
#pragma unroll
            for (int n = 0; n < HID / 64; ++n) pg[4 + kMaxD + w * (HID / 4) + 16 * n + l16] = 0.f;
#pragma unroll
            for (int n = 0; n < NR; ++n) pg[4 + cbase + 16 * n + l16] = acc[n][rr];
        }
    };
    if (pidx >= Ptok) {
        ref_part(pidx - Ptok, prec);
        return;
    }

    // ---------------- compressed tokens ----------------
    const int64_t qa_ = (int64_t)pidx * tiles_per_part * TT;
    const int qa = (int)qa_;
    const int qe = (int)min(Nt_u, qa_ + (int64_t)tiles_per_part * TT);
    if ((SP || cmode) && qa >= qe) {
        // a partition past the end of this unit's list: a neutral record
        for (int i = tid; i < G * kPStride; i += 256)
            prec[i] = (i % kPStride == 0) ? -INFINITY : 0.f;
        return;
    }
    const int ntile = (qe - qa + TT - 1) / TT;
    const int Ntm1 = (int)Nt - 1;
    const bf16_t *klat_u = klat + (int64_t)unit * Ncap * DC;
    const bf16_t *vlat_u = vlat + (int64_t)unit * Ncap * DC;
    // Q4: the unit's code rows (d_c / 2 bytes each), then its (shift, scale)
    // words; a lane's eight latent values are one 32-bit word of codes
    const uint8_t *kq_u = reinterpret_cast<const uint8_t *>(klat) + (int64_t)unit * Ncap * (DC / 2 + 4);
    const uint8_t *vq_u = reinterpret_cast<const uint8_t *>(vlat) + (int64_t)unit * Ncap * (DC / 2 + 4);
    const uint32_t qpar = (uint32_t)Ncap * (DC / 2);  // byte offset of the words
    auto zrow = [&](const bf16_t *lat_u, const uint8_t *q_u, uint32_t tok) -> bf16x8 {
        if (8 * lq >= DC) return as_bf16x8(zero4);
        if constexpr (Q4) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(q_u + tok * (DC / 2) + 4u * lq);
            const uint32_t pr = *reinterpret_cast<const uint32_t *>(q_u + qpar + tok * 4u);
            const float shift = __uint_as_float(pr << 16), sc = __uint_as_float(pr & 0xffff0000u);
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __builtin_fmaf((float)((w >> (8 * e)) & 15u), sc, shift);
                const float b = __builtin_fmaf((float)((w >> (8 * e + 4)) & 15u), sc, shift);
                o[e] = pack_bf16(a, b);
            }
            return as_bf16x8(o);
        } else {
            return as_bf16x8(ld16(at_byte(lat_u, (tok * DC + 8 * lq) * 2u)));
        }
    };
    const uint16_t *kidx_u = kidx + (int64_t)unit * Ncap * KX;
    const uint16_t *vidx_u = vidx + (int64_t)unit * Ncap * KX;

    // rows of absent query heads stay zero; maxima start at -inf
    for (int i = tid; i < (int)(sizeof(wr) / 16); i += 256)
        reinterpret_cast<u32x4 *>(&wr[0][0][0])[i] = zero4;
    for (int i = tid; i < (int)(sizeof(pw) / 16); i += 256)
        reinterpret_cast<u32x4 *>(&pw[0][0][0][0])[i] = zero4;
    for (int i = tid; i < 2 * 2 * 16; i += 256) (&msl[0][0][0])[i] = -INFINITY;
    for (int i = tid; i < HID; i += 256) biask[i] = kb1 ? kb1[i] : 0.f;
    if constexpr (SP)
        for (int i = tid; i < qe - qa; i += 256) ordl[i] = cord_u[qa + i];
    __syncthreads();
    // the stored token (ordinal) behind list position i of this partition,
    // clamped into it; dense: the ordinal itself, clamped to the stored ones
    // (counts mode clamps to the unit's own last token: rows past a sequence's
    // length are not its data)
    const int tlast = cmode ? qe - 1 : Ntm1;
    auto tok_of = [&](int i) -> uint32_t {
        return SP ? (uint32_t)ordl[min(i, qe - 1) - qa] : (uint32_t)min(i, tlast);
    };
    // the last reference row a gathered row may name (counts mode: the unit's
    // own last reference, rows past a sequence's length are not its data)
    const uint32_t rlast_u = (uint32_t)(cmode ? Rt_u : Rt) - 1u;
    // paged layout: logical page of the tile at t0 (its clamped tokens lie in
    // the page of min(t0, tlast)) and the offset, in rows, from a token's
    // ordinal to its pool row
    auto tile_page = [&](int t0) -> int {
        return (int)(((uint64_t)(uint32_t)min(t0, tlast) * pm.mag) >> 40);
    };
    auto page_shift = [&](int lp) -> int {   // (pool page) - lp
        return __builtin_amdgcn_readfirstlane(ptab[lp]) >> (pm.lg + LRB);
    };
    // the last page a loader looked up (lp, its pool page lp + dp) and the
    // row shift from a token's ordinal to its pool row: consecutive tiles
    // mostly stay in one page, so the table is read when the page changes
    struct PgMemo {
        int lp = -1, dp = 0;
        int64_t sh = 0;
    };
    auto tok_shift_memo = [&](PgMemo &m, int t0) -> int64_t {
        const int lp = tile_page(t0);
        if (lp != m.lp) {
            m.lp = lp;
            m.dp = page_shift(lp);
            m.sh = (int64_t)m.dp * pm.npp;
        }
        return m.sh;
    };

    if (w < 2) {
        // ================= score waves =================
        const int src = w;
        bf16x8 wK[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            wK[mb] = as_bf16x8(8 * lq < DC ? ld16(kw1 + (16 * mb + l16) * DC + 8 * lq) : zero4);
        // U = W2K^T q in f16, hidden permuted to match the hK^T operand layout
        f16x8 uA[KJ];
        {
            const bool gl = l16 < G;
            const float *ug = ubuf + ((int64_t)bseq * Hq + h * G + (gl ? l16 : 0)) * kMaxH;
            const float gm = gl ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < KJ; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    uA[j][e] = (_Float16)(gm * ug[32 * j + (e < 4 ? 4 * lq + e : 16 + 4 * lq + (e - 4))]);
        }
        // softmax role: lane (lq, l16) owns token l16 and heads lq + 4 e
        int gh[EG];
        float cqv[EG], m_w[EG], l_run[EG];
#pragma unroll
        for (int e = 0; e < EG; ++e) {
            gh[e] = lq + 4 * e;
            cqv[e] = gh[e] < G ? cq[(int64_t)bseq * Hq + h * G + gh[e]] : 0.f;
            m_w[e] = -INFINITY;
            l_run[e] = 0.f;
        }

        // a tile's inputs: the token's latent row and index rows, and the
        // q.R^K table entries of its K references with their count.  Three
        // slots rotate: the rows of tile i + 2 are requested while tile i is
        // computed and the table entries of tile i + 1 (whose index rows are
        // in by then), so no load of a tile waits inside that tile.
        struct KIn {
            bf16x8 z;
            IdxV ik, iv;
            float qv[EG][KX];
            float kek;
        };
        // rows of token (t0 + 16 src + l16), clamped to a stored token
        PgMemo kmemo;
        auto kload = [&](int t0, KIn &in) {
            const uint32_t tok = tok_of(t0 + TH * src + l16);
            if constexpr (PG) {
                const int64_t sh = tok_shift_memo(kmemo, t0);
                in.z = zrow(klat + sh * DC, kq_u, tok);
                in.ik = *reinterpret_cast<const IdxV *>(at_byte(kidx + sh * KX, tok * (KX * 2)));
                in.iv = *reinterpret_cast<const IdxV *>(at_byte(vidx + sh * KX, tok * (KX * 2)));
            } else {
                in.z = zrow(klat_u, kq_u, tok);
                in.ik = *reinterpret_cast<const IdxV *>(at_byte(kidx_u, tok * (KX * 2)));
                in.iv = *reinterpret_cast<const IdxV *>(at_byte(vidx_u, tok * (KX * 2)));
            }
        };
        // q.R^K of the token's references for the lane's heads (unused slots
        // read the all-zero row Rt)
        auto qload = [&](KIn &in) {
            float kek = 0.f;
#pragma unroll
            for (int i = 0; i < KX; ++i) {
                const uint32_t wv = in.ik[i >> 1];
                const uint32_t j = (i & 1) ? (wv >> 16) : (wv & 0xffffu);
                const bool ok = j != kIdxUnused;
                kek += ok ? 1.f : 0.f;
                const uint32_t row = (ok ? j : (uint32_t)Rt) * (uint32_t)GQ;
#pragma unroll
                for (int e = 0; e < EG; ++e)
                    in.qv[e][i] = *at_byte(qr_u, (row + (uint32_t)min(gh[e], GQ - 1)) * 4u);
            }
            in.kek = kek;
        };

        // one tile: scores, softmax, publish into slot (it & 1).  Also starts
        // the table reads of the next tile (n1, whose rows are in) and the row
        // loads of the tile after it (into n2, at token t2).
        // (4-bit latents with k = 8 read the table at the start of the tile
        // itself: a table slot per ring entry would not fit the registers)
        constexpr bool QPRE = !(Q4 && KX == 8);
        auto ktile = [&](int it, int t0, KIn &in, KIn &n1, int t2, KIn &n2) {
            const int sl = it & 1;
            if constexpr (QPRE) qload(n1);
            else qload(in);
            if constexpr (PGS) {
                // V rows of tile it + 1: slot lq of token l16 of this wave
                const uint32_t wv = n1.iv[lq >> 1];
                const uint32_t j = min((lq & 1) ? (wv >> 16) : (wv & 0xffffu), rlast_u);
                voff[(it + 1) & 1][(TH * src + l16) * KX + lq] = ref_off(j);
            }
            kload(t2, n2);
            // hidden tile and partial scores, 32 hidden units per step; the
            // products of step j + 1 are issued before the GELU of step j, and
            // the bias rows of step j + 2 are read from LDS before that
            f32x4 S = {0.f, 0.f, 0.f, 0.f};
            auto bload = [&](int j, f32x4 &b0, f32x4 &b1) {
                b0 = *reinterpret_cast<const f32x4 *>(&biask[32 * j + 4 * lq]);
                b1 = *reinterpret_cast<const f32x4 *>(&biask[32 * j + 16 + 4 * lq]);
            };
            f32x4 bn0, bn1, bm0, bm1;
            bload(0, bn0, bn1);
            if (KJ > 1) bload(1, bm0, bm1);
            f32x4 cn0 = mfma16_bf16(wK[0], in.z, bn0);
            f32x4 cn1 = mfma16_bf16(wK[1], in.z, bn1);
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const f32x4 c0 = cn0, c1 = cn1;
                if (j + 1 < KJ) {
                    bn0 = bm0;
                    bn1 = bm1;
                    if (j + 2 < KJ) bload(j + 2, bm0, bm1);
                    cn0 = mfma16_bf16(wK[2 * (j + 1)], in.z, bn0);
                    cn1 = mfma16_bf16(wK[2 * (j + 1) + 1], in.z, bn1);
                }
                f16x2 g0, g1, g2, g3;
                gelu4_f16(c0[0], c0[1], c0[2], c0[3], g0, g1);
                gelu4_f16(c1[0], c1[1], c1[2], c1[3], g2, g3);
                const u32x4 hv = {as_u32(g0), as_u32(g1), as_u32(g2), as_u32(g3)};
                S = mfma16_f16(uA[j], as_f16x8(hv), S);
            }
            // S[4 q + r][t] sits in lane 16 q + t, register r.  Move it so that
            // lane (lq, l16) holds head lq + 4 e of token l16: all 64 lanes
            // then carry one (token, head) pair each for G <= 4.
            float sv[EG];
#pragma unroll
            for (int e = 0; e < EG; ++e) {
                const int srcl = 16 * e + l16;
                const float x0 = __shfl(S[0], srcl), x1 = __shfl(S[1], srcl);
                const float x2 = __shfl(S[2], srcl), x3 = __shfl(S[3], srcl);
                sv[e] = lq == 0 ? x0 : lq == 1 ? x1 : lq == 2 ? x2 : x3;
            }
            const bool tok_ok = t0 + TH * src + l16 < qe;
            const float inv_k = __builtin_amdgcn_rcpf(in.kek);
            float s[EG], mref[EG];
            bool up = false;
#pragma unroll
            for (int e = 0; e < EG; ++e) {
                float rs = (in.qv[e][0] + in.qv[e][1]) + (in.qv[e][2] + in.qv[e][3]);
                if constexpr (KX == 8)
                    rs += (in.qv[e][4] + in.qv[e][5]) + (in.qv[e][6] + in.qv[e][7]);
                const float v = scale * (sv[e] + rs * inv_k + cqv[e]);
                s[e] = (tok_ok && gh[e] < G) ? v : -INFINITY;
                if (!SP && logc && tok_ok && gh[e] < G)
                    logc[((int64_t)unit * G + gh[e]) * Nt + (t0 + TH * src + l16)] = v;
                // reference maximum: the larger of the two waves' previous ones
                mref[e] = fmaxf(msl[sl ^ 1][0][gh[e]], msl[sl ^ 1][1][gh[e]]);
                up = up || s[e] > mref[e] + kSlack;
            }
            if (__builtin_amdgcn_ballot_w64(up)) {
                // a score far above the reference: raise it to the maximum over
                // the 16 tokens (the 16 lanes of a row group share the head)
#pragma unroll
                for (int e = 0; e < EG; ++e) {
                    float tm = s[e];
#pragma unroll
                    for (int o = 8; o > 0; o >>= 1) tm = fmaxf(tm, __shfl_xor(tm, o, 16));
                    mref[e] = tm > mref[e] + kSlack ? tm : mref[e];
                }
            }
            bool moved = false;
#pragma unroll
            for (int e = 0; e < EG; ++e) moved = moved || mref[e] != m_w[e];
            if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
                for (int e = 0; e < EG; ++e) {
                    l_run[e] *= mref[e] == -INFINITY ? 1.f : __expf(m_w[e] - mref[e]);
                    m_w[e] = mref[e];
                }
            }
            // publish p (f16, by token), p / k_eff on the token's used V slots
            // (bf16, by (token, slot) row) and the maxima
            // per 32-bit word of the V index entries: which halves are used
            IdxV vmask;
            int nbits = 0;
#pragma unroll
            for (int q = 0; q < KX / 2; ++q) {
                const uint32_t wv = in.iv[q];
                vmask[q] = ((wv & 0xffffu) != kIdxUnused ? 0x0000ffffu : 0u) |
                           ((wv >> 16) != kIdxUnused ? 0xffff0000u : 0u);
                nbits += __builtin_popcount(vmask[q]);
            }
            const float kev = (float)nbits * (1.f / 16.f);
            const float inv_v = __builtin_amdgcn_rcpf(kev);
#pragma unroll
            for (int e = 0; e < EG; ++e) {
                const float p = s[e] == -INFINITY ? 0.f : __expf(s[e] - m_w[e]);
                l_run[e] += p;
                if (gh[e] < G) {
                    pw[sl][src][gh[e]][l16] = (_Float16)p;
                    const uint32_t wb = pack_bf16(p * inv_v, p * inv_v);
                    IdxV wv;
#pragma unroll
                    for (int q = 0; q < KX / 2; ++q) wv[q] = wb & vmask[q];
                    *reinterpret_cast<IdxV *>(&wr[sl][gh[e]][(TH * src + l16) * KX]) = wv;
                    if (l16 == 0) msl[sl][src][gh[e]] = m_w[e];
                }
            }
        };

        KIn X0, X1, X2;
        kload(qa, X0);
        kload(qa + TT, X1);
        if constexpr (QPRE) qload(X0);
        ktile(0, qa, X0, X1, qa + 2 * TT, X2);
        __syncthreads();
        // the value waves' barriers of a tile: one at k = 4, two at k = 8
        // (mid-tile, once the tile's rows are gathered, and end of tile)
        auto tile_sync = [&]() {
            __syncthreads();
            if constexpr (KX == 8) __syncthreads();
        };
        // tiles 1, 2, 3, ... with the slots rotating (tile i in slot i % 3)
        for (int it = 1; it < ntile; it += 3) {
            ktile(it, qa + it * TT, X1, X2, qa + (it + 2) * TT, X0);
            tile_sync();
            if (it + 1 >= ntile) break;
            ktile(it + 1, qa + (it + 1) * TT, X2, X0, qa + (it + 3) * TT, X1);
            tile_sync();
            if (it + 2 >= ntile) break;
            ktile(it + 2, qa + (it + 2) * TT, X0, X1, qa + (it + 4) * TT, X2);
            tile_sync();
        }
        // the value waves run one tile behind: their last tile's barrier
        tile_sync();
        // per-head sums of this wave's tokens
#pragma unroll
        for (int e = 0; e < EG; ++e) {
            float lsum = l_run[e];
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 16);
            if (l16 == 0) {
                lfin[src][gh[e]] = lsum;
                mfin[src][gh[e]] = m_w[e];
            }
        }
        __syncthreads();
    } else {
        // ================= value waves =================
        const int vj = w - 2;
        const int hb = vj * HV, cb = vj * DV;
        bf16x8 wV[NBV];
        f32x4 bV[NBV];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) {
            const int hh = hb + 16 * nb + l16;
            wV[nb] = as_bf16x8(8 * lq < DC ? ld16(vw1 + hh * DC + 8 * lq) : zero4);
            const float bb = vb1 ? vb1[hh] : 0.f;
            bV[nb] = f32x4{bb, bb, bb, bb};
        }
        f32x4 acc_h[NBV], acc_r[NC];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) acc_h[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) acc_r[nc] = f32x4{0.f, 0.f, 0.f, 0.f};
        float macc[4];  // maxima the accumulators are relative to (heads 4 lq + r)
#pragma unroll
        for (int r = 0; r < 4; ++r) macc[r] = -INFINITY;

        // gather addressing: a gather instruction covers RPD rows of 16-byte
        // chunks; this lane's chunk and its swizzled source offsets
        const uint32_t lrow = (uint32_t)(lane / CH);
        const uint32_t c8 = (uint32_t)(lane % CH);
        // source chunk of this lane's LDS slot (rows of a gather instruction
        // start at a multiple of 4, so the row's swizzle is lrow % 4)
        const uint32_t coff = 16u * (c8 ^ (2u * (lrow & 3u)));
        // (counts mode: the unit's own last reference, rows past a sequence's
        // length are not its data)
        const uint32_t rlast = (uint32_t)(cmode ? Rt_u : Rt) - 1u;
        uint32_t gi[NDMA];
        // index entries of this wave's rows of the tile at t0 (k = 4: rows
        // [64 vj, 64 vj + 64) of the tile's buffer; k = 8: the 128 rows of
        // tokens 16 vj .. 16 vj + 15, the whole of this wave's buffer): rows
        // are (token, slot) pairs in order, i.e. consecutive index entries.
        // Buffer loads over the stored tokens' entries: past them they
        // return 0 (reference 0, a stored row) instead of reading on.
        const __amdgpu_buffer_rsrc_t idx_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)vidx_u, (short)0, (int)(Nt * KX * 2), 0x00020000);
        // (the tile offset goes in the per-lane offset, which the range check
        // covers, not in the scalar offset)
        PgMemo gmemo, zmemo;
        auto gload = [&](int t0) {
            if constexpr (PG) {
                // the tile's page as a buffer of its stored rows: offsets
                // relative to the page start, rows past it (or past the stored
                // tokens) read 0
                (void)tok_shift_memo(gmemo, t0);
                const int lp = gmemo.lp;
                const int pstart = lp * pm.npp;
                const int pp = lp + gmemo.dp;
                const int nrec = min(pm.npp, (int)Nt - pstart);
                const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(vidx + (int64_t)pp * pm.npp * KX), (short)0, nrec * (KX * 2),
                    0x00020000);
                const int vbase = (t0 - pstart + TH * vj) * (KX * 2) + (int)(lrow * 2u);
#pragma unroll
                for (int m = 0; m < NDMA; ++m)
                    gi[m] = __builtin_amdgcn_raw_buffer_load_b16(prsrc, vbase + 2 * RPD * m, 0, 0);
            } else if constexpr (SP) {
                // row r = lrow + RPD m is (token r / KX, slot r % KX) of this
                // wave's 16 tokens, looked up through the list
#pragma unroll
                for (int m = 0; m < NDMA; ++m) {
                    const uint32_t r = lrow + (uint32_t)(RPD * m);
                    const uint32_t tok = tok_of(t0 + TH * vj + (int)(r / KX));
                    gi[m] = __builtin_amdgcn_raw_buffer_load_b16(
                        idx_rsrc, (int)(tok * (KX * 2) + (r % KX) * 2u), 0, 0);
                }
            } else {
                const int vbase = (t0 + TH * vj) * (KX * 2) + (int)(lrow * 2u);
#pragma unroll
                for (int m = 0; m < NDMA; ++m)
                    gi[m] = __builtin_amdgcn_raw_buffer_load_b16(idx_rsrc, vbase + 2 * RPD * m, 0, 0);
            }
        };
        // unused slots (0xFFFF) and rows past the stored range read the last
        // stored reference row: finite data under a zero weight.  Tile 0 takes
        // its rows from the index entries in gi (paged: already pool offsets),
        // later tiles from the offsets the score waves left in voff (without
        // them, every tile from gi)
        auto gissue = [&](bf16_t (*dst)[D], int tile) {
#pragma unroll
            for (int m = 0; m < NDMA; ++m) {
                uint32_t pof;
                if (PGS && tile > 0)
                    pof = voff[tile & 1][64 * vj + RPD * m + lrow] + coff;
                else
                    pof = PG ? gi[m] : min(gi[m], rlast) * (uint32_t)(D * 2) + coff;
                __builtin_amdgcn_global_load_lds(
                    (const void *)((const char *)(PG ? vref : vref_u) + pof),
                    (__attribute__((address_space(3))) void *)&dst[(KX == 4 ? 64 * vj : 0) + RPD * m][0], 16, 0, 0);
            }
        };
        // paged: the loaded index entries become byte offsets of their rows
        // in the pool, while the wave waits at the barrier after the loads
        auto gready = [&]() {
            if constexpr (PG) {
#pragma unroll
                for (int m = 0; m < NDMA; ++m) gi[m] = ref_off(min(gi[m], rlast)) + coff;
            }
        };
        auto zload = [&](int t0, bf16x8 (&z)[2]) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const uint32_t tok = tok_of(t0 + 16 * mb + l16);
                z[mb] = zrow(PG ? vlat + tok_shift_memo(zmemo, t0) * DC : vlat_u, vq_u, tok);
            }
        };

        // One tile's value work, without branches (kScl: the two score waves'
        // maxima differ and their weights are scaled by es0, es1).  The
        // products of hidden block nb + 1 are issued before the GELU of block
        // nb, and the reference-row products are spread over the blocks, so
        // matrix and vector work overlap.
        auto vbody = [&](auto kScl, const bf16x8 (&zv)[2], bf16_t (*cur)[D], const f16x4 (&pa)[2],
                         float es0, float es1, int sl) {
            constexpr bool SCL = decltype(kScl)::value;
            const f16x8 pa8 = {pa[0][0], pa[0][1], pa[0][2], pa[0][3],
                               pa[1][0], pa[1][1], pa[1][2], pa[1][3]};
            u32x4 pv = {0u, 0u, 0u, 0u};
            // reference-row step q: rows 64 s2 + 32 ks + 8 lq of score wave
            // s2's tokens, value columns block nc; the steps are spread over
            // the hidden blocks (k = 4: score wave s2, half ks, block nc; k = 8
            // takes them after a barrier instead).  The LDS operands of a
            // block's steps are read one hidden block ahead (rread), so the
            // products (rmma) do not wait for the transposing reads.
            constexpr int NQ = KX == 4 ? 4 * NC : 0;
            constexpr int QPB = NQ / NBV;   // steps per hidden block
            struct RIn {
                u32x4 bv, pw;
            };
            auto rread = [&](int q, RIn &r) {
                const int s2 = q / (2 * NC), ks = (q / NC) & 1, nc = q % NC;
                const int rb = 64 * s2 + 32 * ks + 8 * lq;
                if (nc == 0) r.pw = *reinterpret_cast<const u32x4 *>(&wr[sl][l16][rb]);
                const int c = cb + 16 * nc + 4 * (l16 & 3);
                const int pcol = (((c >> 3) ^ (2 * (l16 >> 2))) << 3) | (c & 7);
                const u32x2 lo = lds_read_tr16(&cur[rb + (l16 >> 2)][pcol]);
                const u32x2 hi = lds_read_tr16(&cur[rb + 4 + (l16 >> 2)][pcol]);
                r.bv = u32x4{lo[0], lo[1], hi[0], hi[1]};
            };
            auto rmma = [&](int q, const RIn &r) {
                const int s2 = q / (2 * NC), nc = q % NC;
                if (nc == 0) {
                    pv = r.pw;
                    if constexpr (SCL) {
                        const float es = s2 ? es1 : es0;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pv[e] = pack_bf16(__uint_as_float(pv[e] << 16) * es,
                                              __uint_as_float(pv[e] & 0xffff0000u) * es);
                    }
                }
                acc_r[nc] = mfma16_bf16(as_bf16x8(pv), as_bf16x8(r.bv), acc_r[nc]);
            };
            RIn rc[QPB > 0 ? QPB : 1], rn[QPB > 0 ? QPB : 1];
#pragma unroll
            for (int i = 0; i < QPB; ++i) rread(i, rc[i]);
            f32x4 hn0 = mfma16_bf16(zv[0], wV[0], bV[0]);
            f32x4 hn1 = mfma16_bf16(zv[1], wV[0], bV[0]);
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const f32x4 c0 = hn0, c1 = hn1;
                if (nb + 1 < NBV) {
                    hn0 = mfma16_bf16(zv[0], wV[nb + 1], bV[nb + 1]);
                    hn1 = mfma16_bf16(zv[1], wV[nb + 1], bV[nb + 1]);
#pragma unroll
                    for (int i = 0; i < QPB; ++i) rread(QPB * (nb + 1) + i, rn[i]);
                }
                f16x2 g0, g1, g2, g3;
                gelu4_f16_short(c0[0], c0[1], c0[2], c0[3], g0, g1);
                gelu4_f16_short(c1[0], c1[1], c1[2], c1[3], g2, g3);
                // one 32-token product: K index 8 lq + i is token 4 lq + i of
                // the first score wave's 16 (i < 4) or of the second's (i >= 4),
                // the order in which pa8 holds the weights
                const u32x4 hh = {as_u32(g0), as_u32(g1), as_u32(g2), as_u32(g3)};
                acc_h[nb] = mfma16_f16(pa8, as_f16x8(hh), acc_h[nb]);
#pragma unroll
                for (int i = 0; i < QPB; ++i) {
                    rmma(QPB * nb + i, rc[i]);
                    rc[i] = rn[i];
                }
            }
        };

        // k = 8: the reference-row products of one tile, rows 32 q8 .. 32 q8 +
        // 31 (tokens of score wave q8 / 4) from the buffer that holds them
        auto racc8 = [&](auto kScl, float es0, float es1, int sl) {
            constexpr bool SCL = decltype(kScl)::value;
#pragma unroll
            for (int q8 = 0; q8 < ROWS / 32; ++q8) {
                const int rb = 32 * q8 + 8 * lq;
                const int s2 = q8 / (ROWS / 64);
                bf16_t (*buf)[D] = s2 == 0 ? vbufA : vbufB;
                const int rl = rb - BROWS * s2;
                u32x4 pv = *reinterpret_cast<const u32x4 *>(&wr[sl][min(l16, WH - 1)][rb]);
                if (l16 >= WH) pv = zero4;
                if constexpr (SCL) {
                    const float es = s2 ? es1 : es0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pv[e] = pack_bf16(__uint_as_float(pv[e] << 16) * es,
                                          __uint_as_float(pv[e] & 0xffff0000u) * es);
                }
#pragma unroll
                for (int nc = 0; nc < NC; ++nc) {
                    const int c = cb + 16 * nc + 4 * (l16 & 3);
                    const int pcol = (((c >> 3) ^ (2 * (l16 >> 2))) << 3) | (c & 7);
                    const u32x2 lo = lds_read_tr16(&buf[rl + (l16 >> 2)][pcol]);
                    const u32x2 hi = lds_read_tr16(&buf[rl + 4 + (l16 >> 2)][pcol]);
                    const u32x4 bv = {lo[0], lo[1], hi[0], hi[1]};
                    acc_r[nc] = mfma16_bf16(as_bf16x8(pv), as_bf16x8(bv), acc_r[nc]);
                }
            }
        };

        auto vtile = [&](int it, const bf16x8 (&zv)[2], bf16_t (*cur)[D]) {
            const int sl = it & 1;
            // maxima the score waves used for this tile
            const f32x4 mn0 = *reinterpret_cast<const f32x4 *>(&msl[sl][0][4 * lq]);
            const f32x4 mn1 = *reinterpret_cast<const f32x4 *>(&msl[sl][1][4 * lq]);
            bool moved = false, split = false;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                moved = moved || mn0[r] != macc[r] || mn1[r] != macc[r];
                split = split || mn0[r] != mn1[r];
            }
            if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float mn = fmaxf(mn0[r], mn1[r]);
                    const float al = mn == -INFINITY ? 1.f : __expf(macc[r] - mn);
                    macc[r] = mn;
#pragma unroll
                    for (int nb = 0; nb < NBV; ++nb) acc_h[nb][r] *= al;
#pragma unroll
                    for (int nc = 0; nc < NC; ++nc) acc_r[nc][r] *= al;
                }
            }
            // P operands (rows = query heads l16), per score wave
            f16x4 pa[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                pa[s2] = *reinterpret_cast<const f16x4 *>(&pw[sl][s2][l16][4 * lq]);
            const bool scl = __builtin_amdgcn_ballot_w64(split) != 0;
            float e0 = 1.f, e1 = 1.f;
            if (!scl) {
                vbody(std::integral_constant<bool, false>{}, zv, cur, pa, 1.f, 1.f, sl);
            } else {
                // the two waves used different maxima: bring the lower one's
                // weights to the larger maximum
                const float a0 = msl[sl][0][l16], a1 = msl[sl][1][l16];
                const float mx = fmaxf(a0, a1);
                e0 = a0 == -INFINITY ? 0.f : __expf(a0 - mx);
                e1 = a1 == -INFINITY ? 0.f : __expf(a1 - mx);
                pa[0] = pa[0] * (_Float16)e0;
                pa[1] = pa[1] * (_Float16)e1;
                vbody(std::integral_constant<bool, true>{}, zv, cur, pa, e0, e1, sl);
            }
            if constexpr (KX == 8) {
                // both value waves' gathers of this tile have landed and are
                // visible: the reference-row products over all 256 rows
                wait_vm_all();
                __syncthreads();
                if (!scl)
                    racc8(std::integral_constant<bool, false>{}, 1.f, 1.f, sl);
                else
                    racc8(std::integral_constant<bool, true>{}, e0, e1, sl);
            }
        };

        bf16x8 zA[2], zB[2];
        if constexpr (KX == 8) {
            // each tile's rows are gathered into both buffers (this wave's
            // tokens into its own) after the previous tile is done with them,
            // under the tile's hidden work
            bf16_t (*own)[D] = vj == 0 ? vbufA : vbufB;
            gload(qa);
            zload(qa, zA);
            wait_vm_all();
            gready();
            __syncthreads();
            for (int it = 0; it < ntile; it += 2) {
                gissue(own, 0);
                zload(qa + (it + 1) * TT, zB);
                gload(qa + (it + 1) * TT);
                vtile(it, zA, own);   // (waits for the index loads mid-tile)
                gready();
                __syncthreads();
                if (it + 1 >= ntile) break;
                gissue(own, 0);
                zload(qa + (it + 2) * TT, zA);
                gload(qa + (it + 2) * TT);
                vtile(it + 1, zB, own);
                gready();
                __syncthreads();
            }
        } else {
        gload(qa);
        gready();
        gissue(vbufA, 0);
        zload(qa, zA);
        wait_vm_all();
        __syncthreads();
        for (int it = 0; it < ntile; it += 2) {
            if (it + 1 < ntile) {
                gissue(vbufB, it + 1);
                zload(qa + (it + 1) * TT, zB);
            }
            vtile(it, zA, vbufA);
            wait_vm_all();
            __syncthreads();
            if (it + 1 >= ntile) break;
            if (it + 2 < ntile) {
                gissue(vbufA, it + 2);
                zload(qa + (it + 2) * TT, zA);
            }
            vtile(it + 1, zB, vbufB);
            wait_vm_all();
            __syncthreads();
        }
        }
        __syncthreads();  // the score waves' sums and maxima are in LDS
        // partial record: accumulators relative to macc; the two waves' sums
        // brought to the same maximum
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int g = 4 * lq + r;
            if (g < G) {
                const float m0 = mfin[0][g], m1 = mfin[1][g];
                const float M = macc[r];
                const float e0 = m0 == -INFINITY ? 0.f : __expf(m0 - M);
                const float e1 = m1 == -INFINITY ? 0.f : __expf(m1 - M);
                float *pg = prec + (int64_t)g * kPStride;
#pragma unroll
                for (int nb = 0; nb < NBV; ++nb) pg[4 + kMaxD + hb + 16 * nb + l16] = acc_h[nb][r];
#pragma unroll
                for (int nc = 0; nc < NC; ++nc) pg[4 + cb + 16 * nc + l16] = acc_r[nc][r];
                if (vj == 0 && l16 == 0) {
                    const float L = lfin[0][g] * e0 + lfin[1][g] * e1;
                    pg[0] = M;
                    pg[1] = L;
                    pg[2] = L;
                }
            }
        }
    }
}

// Per-call extras: the sparse lists (ord == nullptr: a dense call) and the
// optional logit outputs of a dense call (logc [U][G][Nt] by token ordinal,
// logr [U][G][Rt] by reference ordinal; nullptr: not written).
struct SparseArgs {
    const int32_t *ord;
    const int32_t *cnt;
    int nsel;
    float *logc;
    float *logr;
    PageMap pm;   // paged caches (pm.tbl non-null)
};

template <int D, int DC, int HID, int KP>
void launch_mfma_t(const Dims &dm, int Hq, const DecPlan &pl, const CacheArgs &kc,
                   const MlpArgs &kd, const CacheArgs &vc, const MlpArgs &vd, float scale,
                   const float *u, const float *cq, const float *qr, float *part,
                   const SparseArgs &sa, hipStream_t st) {
    const int U = dm.B * dm.H;
    const int G = Hq / dm.H;
    auto kern = sa.ord ? main_mfma_kernel<D, DC, HID, KP, true> : main_mfma_kernel<D, DC, HID, KP, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(pl.P * U)), dim3(256),
                       0, st, U, Hq, G, dm.k, dm.R, dm.N, pl.Rt, pl.Nt, pl.tiles_per_part,
                       (int)pl.Ptok, (int)pl.P, (const bf16_t *)kc.lat, kc.idx,
                       (const bf16_t *)vc.refs, (const bf16_t *)vc.lat, vc.idx,
                       (const bf16_t *)kd.w1, kd.b1, (const bf16_t *)vd.w1, vd.b1, scale, u, cq,
                       qr, part, sa.ord, sa.cnt, sa.nsel, sa.logc, sa.logr);
}

template <int D, int DC, int HID>
void launch_ws_t(const Dims &dm, int Hq, const DecPlan &pl, const CacheArgs &kc,
                 const MlpArgs &kd, const CacheArgs &vc, const MlpArgs &vd, float scale,
                 const float *u, const float *cq, const float *qr, float *part,
                 const SparseArgs &sa, hipStream_t st) {
    const int U = dm.B * dm.H;
    const int G = Hq / dm.H;
    const bool sp = sa.ord != nullptr;
    auto pick = [&](auto q4c) {
        constexpr bool QF = decltype(q4c)::value;
        return dm.k == 4
                   ? (G <= 4 ? (sp ? main_ws_kernel<D, DC, HID, 1, 4, true, QF, false> : main_ws_kernel<D, DC, HID, 1, 4, false, QF, false>)
                             : (sp ? main_ws_kernel<D, DC, HID, 2, 4, true, QF, false> : main_ws_kernel<D, DC, HID, 2, 4, false, QF, false>))
                   : (G <= 4 ? (sp ? main_ws_kernel<D, DC, HID, 1, 8, true, QF, false> : main_ws_kernel<D, DC, HID, 1, 8, false, QF, false>)
                             : (sp ? main_ws_kernel<D, DC, HID, 2, 8, true, QF, false> : main_ws_kernel<D, DC, HID, 2, 8, false, QF, false>));
    };
    auto kern = dm.lat_fmt ? pick(std::true_type()) : pick(std::false_type());
    if (sa.pm.tbl)
        kern = dm.k == 4 ? (G <= 4 ? main_ws_kernel<D, DC, HID, 1, 4, false, false, true>
                                   : main_ws_kernel<D, DC, HID, 2, 4, false, false, true>)
                         : (G <= 4 ? main_ws_kernel<D, DC, HID, 1, 8, false, false, true>
                                   : main_ws_kernel<D, DC, HID, 2, 8, false, false, true>);
    hipLaunchKernelGGL(kern, dim3((unsigned)(pl.P * U)), dim3(256), 0, st,
                       U, Hq, G, dm.R, dm.N, pl.Rt, pl.Nt, pl.tiles_per_part, (int)pl.Ptok,
                       (int)pl.P, (const bf16_t *)kc.lat, kc.idx, (const bf16_t *)vc.refs,
                       (const bf16_t *)vc.lat, vc.idx, (const bf16_t *)kd.w1, kd.b1,
                       (const bf16_t *)vd.w1, vd.b1, scale, u, cq, qr, part, sa.logc, sa.logr,
                       sa.ord, sa.cnt, sa.nsel, sa.pm);
}

// The wave-specialised kernel covers k = 4 or 8 and d_c <= 32.
template <int D>
bool launch_ws_d(const Dims &dm, int Hq, const DecPlan &pl, const CacheArgs &kc,
                 const MlpArgs &kd, const CacheArgs &vc, const MlpArgs &vd, float scale,
                 const float *u, const float *cq, const float *qr, float *part,
                 const SparseArgs &sa, hipStream_t st) {
    if ((dm.k != 4 && dm.k != 8) || dm.dc > 32) return false;
    const bool h256 = kd.hidden == 256;
    if (dm.dc <= 16) {
        if (h256) launch_ws_t<D, 16, 256>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        else launch_ws_t<D, 16, 128>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
    } else {
        if (h256) launch_ws_t<D, 32, 256>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        else launch_ws_t<D, 32, 128>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
    }
    return true;
}

template <int D, int DC>
bool launch_mfma_dc(const Dims &dm, int Hq, const DecPlan &pl, const CacheArgs &kc,
                    const MlpArgs &kd, const CacheArgs &vc, const MlpArgs &vd, float scale,
                    const float *u, const float *cq, const float *qr, float *part,
                    const SparseArgs &sa, hipStream_t st) {
    const bool kp4 = dm.k <= 4;
    if (kd.hidden == 256) {
        if (kp4) launch_mfma_t<D, DC, 256, 4>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        else launch_mfma_t<D, DC, 256, 8>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        return true;
    }
    if (kd.hidden == 128) {
        if (kp4) launch_mfma_t<D, DC, 128, 4>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        else launch_mfma_t<D, DC, 128, 8>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        return true;
    }
    return false;
}

// The matrix-core path covers bf16 storage with GELU decompressors of hidden
// width 128 or 256 (same width for K and V) and d_c <= 64; everything else
// takes the general path.
bool mfma_eligible(const Dims &dm, const MlpArgs &kd, const MlpArgs &vd) {
    return dm.dtype == 1 && kd.hidden == vd.hidden && (kd.hidden == 128 || kd.hidden == 256) &&
           kd.act == 0 && vd.act == 0 && dm.dc <= 64;
}

// 4-bit latents are read by the wave-specialised kernel only
bool ws_eligible(const Dims &dm, const MlpArgs &kd, const MlpArgs &vd) {
    return mfma_eligible(dm, kd, vd) && (dm.k == 4 || dm.k == 8) && dm.dc <= 32;
}

// One decode call; with pos non-null, the sparse call over the listed
// positions pos[B][H][nsel] (the lists are split first, then the same
// kernels walk them).
template <typename T>
hipError_t launch_decode_t(const Dims &dm, int Hq, int64_t T_, const void *q,
                           const CacheArgs &kc, const MlpArgs &kd, const CacheArgs &vc,
                           const MlpArgs &vd, float scale, float *out, void *ws,
                           const int32_t *pos, int nsel, hipStream_t st,
                           float *logc = nullptr, float *logr = nullptr, float *lse = nullptr,
                           uint32_t *hist0 = nullptr, const int32_t *counts = nullptr) {
    const DecPlan pl = plan_decode(dm, Hq, T_, pos ? (int64_t)nsel : -1);
    // paged caches: K and V share one block table (entries clamped into the
    // smaller pool)
    PageMap pm;
    if (dm.pr) {
        pm = page_map(dm, kc);
        pm.npages = (int32_t)std::min(kc.npages, vc.npages);
    }
    const int G = Hq / dm.H;
    char *w = (char *)ws;
    float *u = (float *)(w + pl.off_u);
    float *cq = (float *)(w + pl.off_cq);
    float *qr = (float *)(w + pl.off_qr);
    float *part = (float *)(w + pl.off_part);
    SparseArgs sa{nullptr, counts, 0, logc, logr, pm};
    int32_t *ord = nullptr, *cnt = nullptr;
    if (pos) {
        ord = (int32_t *)(w + pl.off_ord);
        cnt = (int32_t *)(w + pl.off_cnt);
        sa = SparseArgs{ord, cnt, nsel, nullptr, nullptr, PageMap{}};
    }
    // the query-side tables, and for a sparse call the list split (one more
    // block per unit)
    const int nrb = (int)((qr_rows(pl.Rt) + 255) / 256);
    hipLaunchKernelGGL((dm.pr ? prep_kernel<T, true> : prep_kernel<T, false>),
                       dim3((unsigned)(nrb + G + (pos ? 1 : 0)), dm.H, dm.B),
                       dim3(256), 0, st, (const T *)q, Hq, G, dm.d, (const T *)kc.refs, dm.R,
                       pl.Rt, nrb, (const T *)kd.w2, kd.hidden, kd.b2, u, cq, qr, pos, nsel, T_,
                       dm.s, ord, cnt, pm);
    bool done = false;
    if constexpr (sizeof(T) == 2) {
        if (mfma_eligible(dm, kd, vd)) {
            done = dm.d == 128
                       ? launch_ws_d<128>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st)
                       : launch_ws_d<64>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
        }
        if (!done && !dm.lat_fmt && mfma_eligible(dm, kd, vd)) {
            if (dm.d == 128) {
                if (dm.dc == 16) done = launch_mfma_dc<128, 16>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
                else if (dm.dc == 32) done = launch_mfma_dc<128, 32>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
                else done = launch_mfma_dc<128, 64>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
            } else {
                if (dm.dc == 16) done = launch_mfma_dc<64, 16>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
                else if (dm.dc == 32) done = launch_mfma_dc<64, 32>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
                else done = launch_mfma_dc<64, 64>(dm, Hq, pl, kc, kd, vc, vd, scale, u, cq, qr, part, sa, st);
            }
        }
    }
    if (!done && (dm.lat_fmt || dm.pr)) return hipErrorInvalidValue;  // (rejected before any launch)
    if (!done)
        hipLaunchKernelGGL(main_kernel<T>, dim3((unsigned)pl.P, dm.H, dm.B), dim3(256), 0, st, Hq,
                           G, dm.d, dm.dc, dm.k, dm.s, dm.R, dm.N, pl.Rt, pl.Nt, pl.Ptok,
                           (int64_t)pl.tiles_per_part * kTileTok, (const T *)kc.refs,
                           (const T *)kc.lat, kc.idx, (const T *)vc.refs, (const T *)vc.lat,
                           vc.idx, (const T *)kd.w1, kd.b1, kd.hidden, kd.act, (const T *)vd.w1,
                           vd.b1, vd.hidden, vd.act, scale, u, cq, qr, part, sa.ord, sa.cnt,
                           sa.nsel, sa.logc, sa.logr);
    hipLaunchKernelGGL(combine2_kernel<T>, dim3(Hq, dm.B), dim3(kCombThreads), 0, st, Hq, G, dm.d, dm.H,
                       pl.P, part, (const T *)vd.w2, vd.hidden, vd.b2, out, lse, hist0);
    return hipGetLastError();
}

}  // namespace

size_t decode_ws_bytes(const Dims &dm, int Hq, int64_t T) { return plan_decode(dm, Hq, T).total; }

// Dims of n_win exact rows [B][H][n_win][d] seen as a stride-1 cache: every
// row is a reference (attended verbatim), nothing is compressed.
static Dims window_dims(const Dims &dm, int64_t n_win) {
    Dims w = dm;
    w.s = 1;
    w.cap = n_win;
    w.R = n_win;
    w.N = 0;
    w.lat_fmt = 0;
    w.pr = 0;   // the window rows are one contiguous array
    return w;
}

// Workspace of a decode call with a window: the compressed cache's call, the
// window's call, then each one's output and per-head log-sum-exp.
struct WinPlan {
    size_t off_w, off_o1, off_l1, off_o2, off_l2, total;
};
static WinPlan plan_window(const Dims &dm, int Hq, int64_t T, int64_t n_win) {
    WinPlan p;
    size_t off = align_up(plan_decode(dm, Hq, T).total);
    p.off_w = off;
    off += align_up(plan_decode(window_dims(dm, n_win), Hq, n_win).total);
    const size_t ob = align_up((size_t)dm.B * Hq * dm.d * 4), lb = align_up((size_t)dm.B * Hq * 4);
    p.off_o1 = off;
    off += ob;
    p.off_l1 = off;
    off += lb;
    p.off_o2 = off;
    off += ob;
    p.off_l2 = off;
    off += lb;
    p.total = off;
    return p;
}

size_t decode_window_ws_bytes(const Dims &dm, int Hq, int64_t T, int64_t n_win) {
    return plan_window(dm, Hq, T, n_win).total;
}

hipError_t launch_decode_window(const Dims &dm, int Hq, int64_t T, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, const void *kwin, const void *vwin,
                                int64_t n_win, float scale, float *out, void *ws, size_t ws_bytes,
                                hipStream_t st) {
    (void)ws_bytes;
    const WinPlan wp = plan_window(dm, Hq, T, n_win);
    char *w = (char *)ws;
    float *o1 = (float *)(w + wp.off_o1), *l1 = (float *)(w + wp.off_l1);
    float *o2 = (float *)(w + wp.off_o2), *l2 = (float *)(w + wp.off_l2);
    const Dims dw = window_dims(dm, n_win);
    const CacheArgs kw{const_cast<void *>(kwin), nullptr, nullptr, nullptr};
    const CacheArgs vw{const_cast<void *>(vwin), nullptr, nullptr, nullptr};
    hipError_t e;
    if (dm.dtype == 0) {
        e = launch_decode_t<float>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, o1, ws, nullptr, 0, st,
                                   nullptr, nullptr, l1);
        if (e == hipSuccess)
            e = launch_decode_t<float>(dw, Hq, n_win, q, kw, kdec, vw, vdec, scale, o2,
                                       w + wp.off_w, nullptr, 0, st, nullptr, nullptr, l2);
    } else {
        e = launch_decode_t<bf16_t>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, o1, ws, nullptr, 0,
                                    st, nullptr, nullptr, l1);
        if (e == hipSuccess)
            e = launch_decode_t<bf16_t>(dw, Hq, n_win, q, kw, kdec, vw, vdec, scale, o2,
                                        w + wp.off_w, nullptr, 0, st, nullptr, nullptr, l2);
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge2_kernel, dim3((unsigned)(dm.B * Hq)), dim3(kMaxD), 0, st, o1, l1, o2,
                       l2, dm.d, out);
    return hipGetLastError();
}

// A batch of sequences of different lengths on the wave-specialised kernel:
// counts[unit] = (compressed tokens, references) of the unit's sequence,
// nmax the longest sequence (the partition plan's length).
bool decode_counts_supported(const Dims &dm, const MlpArgs &kdec, const MlpArgs &vdec) {
    return ws_eligible(dm, kdec, vdec);
}

size_t decode_counts_ws_bytes(const Dims &dm, int Hq, int64_t nmax) {
    return plan_decode(dm, Hq, nmax).total;
}

hipError_t launch_decode_counts(const Dims &dm, int Hq, int64_t nmax, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, const int32_t *counts, float scale,
                                float *out, void *ws, hipStream_t st) {
    return launch_decode_t<bf16_t>(dm, Hq, nmax, q, kc, kdec, vc, vdec, scale, out, ws, nullptr,
                                   0, st, nullptr, nullptr, nullptr, nullptr, counts);
}

bool decode_q4_supported(const Dims &dm, const MlpArgs &kdec, const MlpArgs &vdec) {
    return ws_eligible(dm, kdec, vdec);
}

size_t decode_sparse_ws_bytes(const Dims &dm, int Hq, int64_t T, int nsel) {
    return plan_decode(dm, Hq, T, nsel).total;
}

// Workspace of a decode call with token selection: the dense call's, then the
// logits (by token and by reference ordinal), the per-head log-sum-exp and the
// selection keys.
struct SelPlan {
    DecPlan dec;
    size_t off_logc, off_logr, off_lse, off_keys, off_hist, off_cnt, total;
};
SelPlan plan_select(const Dims &dm, int Hq, int64_t T) {
    SelPlan p;
    p.dec = plan_decode(dm, Hq, T);
    const size_t U = (size_t)dm.B * dm.H, G = (size_t)(Hq / dm.H);
    size_t off = p.dec.total;
    p.off_logc = off;
    off += align_up(U * G * (size_t)p.dec.Nt * 4);
    p.off_logr = off;
    off += align_up(U * G * (size_t)p.dec.Rt * 4);
    p.off_lse = off;
    off += align_up((size_t)dm.B * Hq * 4);
    p.off_keys = off;
    off += align_up(U * (size_t)keys_stride(T) * 4);
    p.off_hist = off;
    off += align_up(U * kSelHist * 4);
    p.off_cnt = off;
    off += align_up(U * (size_t)((T + kSelSlice - 1) / kSelSlice) * 2 * 4);
    p.total = off;
    return p;
}

size_t decode_select_ws_bytes(const Dims &dm, int Hq, int64_t T) { return plan_select(dm, Hq, T).total; }

hipError_t launch_decode_select(const Dims &dm, int Hq, int64_t T, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, float scale, float *out, int n_keep,
                                int32_t *positions, float *scores, void *ws, size_t ws_bytes,
                                hipStream_t st) {
    (void)ws_bytes;
    const SelPlan sp = plan_select(dm, Hq, T);
    char *w = (char *)ws;
    float *logc = (float *)(w + sp.off_logc);
    float *logr = (float *)(w + sp.off_logr);
    float *lse = (float *)(w + sp.off_lse);
    uint32_t *keys = (uint32_t *)(w + sp.off_keys);
    uint32_t *hist0 = (uint32_t *)(w + sp.off_hist);
    const hipError_t e =
        dm.dtype == 0
            ? launch_decode_t<float>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, nullptr, 0,
                                     st, logc, logr, lse, hist0)
            : launch_decode_t<bf16_t>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, nullptr,
                                      0, st, logc, logr, lse, hist0);
    if (e != hipSuccess) return e;
    const unsigned U = (unsigned)(dm.B * dm.H);
    hipLaunchKernelGGL(select_keys_kernel,
                       dim3((unsigned)((T + 256 * kKeyPer - 1) / (256 * kKeyPer)), U), dim3(256), 0,
                       st, logc, logr, lse, Hq, Hq / dm.H, dm.H, T, sp.dec.Nt, sp.dec.Rt, dm.s,
                       keys, scores, hist0);
    const dim3 sg((unsigned)((T + kSelSlice - 1) / kSelSlice), U);
    for (int pass = 1; pass < 4; ++pass)
        hipLaunchKernelGGL(select_hist_kernel, sg, dim3(256), 0, st, keys, hist0, T, n_keep, pass);
    uint32_t *cnt = (uint32_t *)(w + sp.off_cnt);
    hipLaunchKernelGGL(select_count_kernel, sg, dim3(256), 0, st, keys, hist0, T, n_keep, cnt);
    hipLaunchKernelGGL(select_write_kernel, sg, dim3(256), 0, st, keys, hist0, cnt, T, n_keep,
                       positions);
    return hipGetLastError();
}

hipError_t launch_decode(const Dims &dm, int Hq, int64_t T, const void *q, const CacheArgs &kc,
                         const MlpArgs &kdec, const CacheArgs &vc, const MlpArgs &vdec,
                         float scale, float *out, void *ws, size_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;
    if (dm.dtype == 0)
        return launch_decode_t<float>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, nullptr,
                                      0, st);
    return launch_decode_t<bf16_t>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, nullptr, 0,
                                   st);
}

hipError_t launch_decode_sparse(const Dims &dm, int Hq, int64_t T, const void *q,
                                const CacheArgs &kc, const MlpArgs &kdec, const CacheArgs &vc,
                                const MlpArgs &vdec, const int32_t *pos, int nsel, float scale,
                                float *out, void *ws, size_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;
    if (dm.dtype == 0)
        return launch_decode_t<float>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, pos,
                                      nsel, st);
    return launch_decode_t<bf16_t>(dm, Hq, T, q, kc, kdec, vc, vdec, scale, out, ws, pos, nsel,
                                   st);
}

}  // namespace dk
