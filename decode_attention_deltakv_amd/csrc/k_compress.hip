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
#include "dk_mfma.h"

#include <limits.h>

#include <algorithm>
#include <type_traits>

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

// Matrix-core path (bf16 storage, hidden width 128 or 256, d_c <= 64).
// A block walks tiles of 32 tokens of one unit.  Per tile the residual tile
// (x - mean of the chosen reference rows, fp32, rounded to bf16) is formed in
// LDS; the 4 waves split the hidden units: h^T = act(W1 r^T + b1) on bf16
// MFMA (hidden x tokens), then each wave's share of the second product
// W2 h^T is summed across waves in LDS, b2 added, and the latent rounded to
// bf16.  The hidden tile never leaves registers (its MFMA output layout is
// the B operand of the second product, with the hidden index permuted
// consistently in W2's operand).
//
// The global loads run ahead of the products in a three-stage pipeline: the
// index lists two tiles ahead, the token rows and the chosen reference rows
// (whose addresses those lists give) one tile ahead, so neither the
// index-then-gather dependence nor HBM latency sits between two tiles.
// Each thread owns NI 16-byte chunks (token t, columns 8 c8 .. 8 c8 + 7) of
// every tile.  KX: largest k (4 or 8).  Q4: latents stored as 4-bit codes
// with a per-row bf16 shift and scale (d_c / 4 lanes per row quantise it).
// The body of one block (bidx: the block's index over units x tile groups),
// shared by the kernel over a range of one cache and the batched-append kernel
// over one token of several caches, so both compute the same bits.  PG: a
// paged cache (appends only: the range [q0, q0 + nq) lies in one page), whose
// index and latent rows are found through pm once and whose reference rows are
// looked up by ordinal.
template <int D, int HID, int DC, int KX, bool GELU, bool Q4, bool PG = false>
__device__ __forceinline__ void compress_mfma_body(
    int bidx, const bf16_t *__restrict__ x, int64_t t0, int64_t nrows, int s, int k,
    const bf16_t *__restrict__ refs, int64_t Rcap, const uint16_t *__restrict__ idx,
    int64_t Ncap, int64_t q0, int64_t nq, int U, int tiles_per_block,
    const bf16_t *__restrict__ w1, const float *__restrict__ b1, const bf16_t *__restrict__ w2,
    const float *__restrict__ b2, bf16_t *__restrict__ lat, PageMap pm = PageMap{}) {
    constexpr int TT = 32;
    constexpr int HW = HID / 4;
    constexpr int MT = HW / 16;
    constexpr int KSD = D / 32;
    constexpr int KJ = HW / 32;
    constexpr int MD = DC / 16;
    constexpr int CH = D / 8;
    constexpr int NI = (TT * CH) / 256;
    static_assert(HW % 32 == 0 && DC % 16 == 0, "unsupported shape");
    __shared__ __attribute__((aligned(16))) bf16_t dl[TT][D + 8];
    __shared__ float zp[4][DC][TT + 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int unit = bidx % U;
    const int blk = bidx / U;
    const int hb = w * HW;
    const int64_t qend = q0 + nq;
    static_assert(!(PG && Q4), "paged caches hold bf16 latents");
    const bf16_t *urefs = refs + (int64_t)unit * Rcap * D;
    const bf16_t *ux = x + (int64_t)unit * nrows * D;
    // (paged: the offset, in rows, from token ordinal q to its pool row in the
    // page that holds the range)
    const int64_t tsh = PG ? pg_tok_row(pm, unit, q0) - q0 : 0;
    const uint16_t *uidx = PG ? idx + tsh * k : idx + (int64_t)unit * Ncap * k;

    bf16x8 a1[MT][KSD];
    f32x4 bias1[MT];
    // W2 operand: bf16 for the identity activation, f16 after the GELU (whose
    // packed-f16 output then feeds an f16 product without a conversion)
    using A2 = typename std::conditional<GELU, f16x8, bf16x8>::type;
    A2 a2[MD][KJ];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
            a1[m][ks] = as_bf16x8(ld16(w1 + (int64_t)(hb + 16 * m + l16) * D + 32 * ks + 8 * lq));
#pragma unroll
        for (int r = 0; r < 4; ++r) bias1[m][r] = b1 ? b1[hb + 16 * m + 4 * lq + r] : 0.f;
    }
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const bf16_t *wr = w2 + (int64_t)(16 * md + l16) * HID + hb + 32 * j + 4 * lq;
            const uint2 lo = *reinterpret_cast<const uint2 *>(wr);
            const uint2 hi = *reinterpret_cast<const uint2 *>(wr + 16);
            u32x4 v = {lo.x, lo.y, hi.x, hi.y};
            if constexpr (GELU) {
                f16x8 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * e] = (_Float16)__uint_as_float(v[e] << 16);
                    h[2 * e + 1] = (_Float16)__uint_as_float(v[e] & 0xffff0000u);
                }
                a2[md][j] = h;
            } else {
                a2[md][j] = as_bf16x8(v);
            }
        }

    const int ntile = (int)min((int64_t)tiles_per_block,
                               (qend - q0 + TT - 1) / TT - (int64_t)blk * tiles_per_block);
    // token ordinals and positions fit in 32 bits (the cache holds fewer
    // than 2^31 rows per unit)
    const uint32_t qlast = (uint32_t)(qend - 1);
    const uint32_t sm1 = (uint32_t)(s - 1);
    auto tile_q = [&](int it) {
        return (uint32_t)(q0 + ((int64_t)blk * tiles_per_block + it) * TT);
    };
    // token ordinal of chunk m in the tile at qt (clamped to the range)
    auto chunk_q = [&](uint32_t qt, int m) { return min(qt + (uint32_t)((tid + 256 * m) / CH), qlast); };
    // index lists and reference rows through buffer resources: every load
    // is issued (no branch, so the wait counts stay exact) and a read past a
    // resource's end returns zeros (the index rows end at the range's last
    // token: the slots past k of that token are masked where used)
    const __amdgpu_buffer_rsrc_t idx_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)uidx, (short)0, (int)(qend * k * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t ref_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)urefs, (short)0, (int)(Rcap * D * 2), 0x00020000);

    // latents of the range [q0, qend) of this unit; stores past qend drop.
    // Q4: the unit's code rows, then its (shift, scale) words
    uint8_t *lat_q4 = reinterpret_cast<uint8_t *>(lat) + (int64_t)unit * Ncap * (DC / 2 + 4);
    const __amdgpu_buffer_rsrc_t lat_rsrc =
        Q4 ? __builtin_amdgcn_make_buffer_rsrc((void *)lat_q4, (short)0, (int)(qend * (DC / 2)),
                                               0x00020000)
           : __builtin_amdgcn_make_buffer_rsrc(
                 (void *)(PG ? lat + tsh * DC : lat + (int64_t)unit * Ncap * DC), (short)0,
                 (int)(qend * DC * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t par_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(lat_q4 + Ncap * (DC / 2)), (short)0, (int)(qend * 4), 0x00020000);
    // Q4: b2 of the four latent columns this thread quantises
    float bias4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int o = 4 * (tid % (DC / 4)) + e;
        bias4[e] = (Q4 && b2) ? b2[o] : 0.f;
    }
    // b2 of the two latent columns this thread stores (fixed across tiles)
    float bias2[2];
    {
        const int o = 2 * (tid % (DC / 2));
        bias2[0] = b2 ? b2[o] : 0.f;
        bias2[1] = b2 ? b2[o + 1] : 0.f;
    }

    uint32_t jn[NI][KX];  // index lists, two tiles ahead
    u32x4 xv[NI];         // token chunks, one tile ahead
    u32x4 rv[NI][KX];     // chosen reference chunks (zeros for unused slots)
    float inv[NI];        // 1 / k_eff of those tokens

    auto stage_idx = [&](uint32_t qt) {
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            const uint32_t base = chunk_q(qt, m) * (uint32_t)k * 2u;
            // slots r >= k read the next entries (or zeros); they are
            // masked where used, so nothing waits for these loads here
#pragma unroll
            for (int r = 0; r < KX; ++r)
                jn[m][r] = __builtin_amdgcn_raw_buffer_load_b16(idx_rsrc, base + 2u * r, 0, 0);
        }
    };
    auto stage_rows = [&](uint32_t qt) {
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            const uint32_t c8 = (uint32_t)((tid + 256 * m) % CH);
            const uint32_t q = chunk_q(qt, m);
            const uint32_t pos = (q / sm1) * (uint32_t)s + q % sm1 + 1u;
            xv[m] = ld16(ux + ((int64_t)pos - t0) * D + 8 * c8);
            int keff = 0;
#pragma unroll
            for (int r = 0; r < KX; ++r) {
                const bool used = r < k && jn[m][r] != kIdxUnused;
                keff += used ? 1 : 0;
                if constexpr (PG) {
                    const int64_t row = pg_ref_row(pm, unit, used ? jn[m][r] : 0u);
                    const u32x4 v = ld16(refs + row * D + 8 * c8);
                    rv[m][r] = used ? v : u32x4{0u, 0u, 0u, 0u};
                } else {
                    const uint32_t off = used ? (jn[m][r] * D + 8u * c8) * 2u : 0x80000000u;
                    rv[m][r] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(ref_rsrc, off, 0, 0));
                }
            }
            // 1 / k_eff (exact for 1, 2, 4, 8; within an ulp otherwise,
            // far below the bf16 rounding of the residual)
            inv[m] = __builtin_amdgcn_rcpf((float)keff);
        }
    };
    // the sum of the chosen rows per coordinate with bf16 dot products: one
    // byte permute pairs coordinate c of two rows, one v_dot2 adds both
    // (products by one are exact; fp32 sums), then x - sum / k_eff
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
    auto dot_ones = [&](uint32_t pair, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), one2, acc, false);
    };
    auto residual = [&]() {
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            const int item = tid + 256 * m;
            const int t = item / CH, c8 = item % CH;
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int r = 0; r + 1 < KX; r += 2) {
                    // [row r, row r + 1] of the low, then the high coordinate
                    const uint32_t lo = __builtin_amdgcn_perm(rv[m][r + 1][e], rv[m][r][e], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(rv[m][r + 1][e], rv[m][r][e], 0x07060302u);
                    s0 = dot_ones(lo, s0);
                    s1 = dot_ones(hi, s1);
                }
                const float d0 = __builtin_fmaf(-s0, inv[m], __uint_as_float(xv[m][e] << 16));
                const float d1 = __builtin_fmaf(-s1, inv[m], __uint_as_float(xv[m][e] & 0xffff0000u));
                o[e] = pack_bf16(d0, d1);
            }
            *reinterpret_cast<u32x4 *>(&dl[t][8 * c8]) = o;
        }
    };

    if (ntile > 0) {
        stage_idx(tile_q(0));
        stage_rows(tile_q(0));
        stage_idx(tile_q(min(1, ntile - 1)));
    }
    for (int it = 0; it < ntile; ++it) {
        const int64_t qt = (int64_t)tile_q(it);
        // ---- residual tile from the staged rows, then the next loads
        residual();
        // issued on every tile (the last tiles load the final one again), so
        // the loop body has no branch around its loads
        // (in this order: the next residual then waits only for the rows)
        __builtin_amdgcn_sched_barrier(0);
        stage_rows(tile_q(min(it + 1, ntile - 1)));
        __builtin_amdgcn_sched_barrier(0);
        stage_idx(tile_q(min(it + 2, ntile - 1)));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // ---- hidden tile and the wave's share of the latent
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            bf16x8 bd[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks)
                bd[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&dl[16 * nt + l16][32 * ks + 8 * lq]));
            f32x4 c[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                c[m] = bias1[m];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) c[m] = mfma16_bf16(a1[m][ks], bd[ks], c[m]);
            }
            f32x4 zc[MD];
#pragma unroll
            for (int md = 0; md < MD; ++md) zc[md] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                u32x4 hv;
                if constexpr (GELU) {
                    // packed-f16 GELU, two pairs per call
                    f16x2 g0, g1, g2, g3;
                    gelu4_f16(c[2 * j][0], c[2 * j][1], c[2 * j][2], c[2 * j][3], g0, g1);
                    gelu4_f16(c[2 * j + 1][0], c[2 * j + 1][1], c[2 * j + 1][2], c[2 * j + 1][3], g2, g3);
                    hv = u32x4{as_u32(g0), as_u32(g1), as_u32(g2), as_u32(g3)};
#pragma unroll
                    for (int md = 0; md < MD; ++md)
                        zc[md] = mfma16_f16(a2[md][j], as_f16x8(hv), zc[md]);
                } else {
                    hv = u32x4{pack_bf16(c[2 * j][0], c[2 * j][1]), pack_bf16(c[2 * j][2], c[2 * j][3]),
                               pack_bf16(c[2 * j + 1][0], c[2 * j + 1][1]),
                               pack_bf16(c[2 * j + 1][2], c[2 * j + 1][3])};
#pragma unroll
                    for (int md = 0; md < MD; ++md)
                        zc[md] = mfma16_bf16(a2[md][j], as_bf16x8(hv), zc[md]);
                }
            }
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int r = 0; r < 4; ++r) zp[w][16 * md + 4 * lq + r][16 * nt + l16] = zc[md][r];
        }
        __syncthreads();
        if constexpr (Q4) {
            // ---- sum the waves' shares, add b2, round to bf16, quantise the
            // row: d_c / 4 consecutive lanes per token, four columns each
            constexpr int TPT = DC / 4;
            static_assert(256 / TPT >= TT, "one pass over the tile's rows");
            const int t = tid / TPT, j = tid % TPT;
            const int tc = t < TT ? t : TT - 1;  // lanes past the tile repeat its last row
            float z[4];
            float zmin = INFINITY, zmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = 4 * j + e;
                const float v = zp[0][o][tc] + zp[1][o][tc] + zp[2][o][tc] + zp[3][o][tc] + bias4[e];
                z[e] = __uint_as_float(pack_bf16(v, v) << 16);  // the stored (bf16) value
                zmin = fminf(zmin, z[e]);
                zmax = fmaxf(zmax, z[e]);
            }
#pragma unroll
            for (int o = 1; o < TPT; o <<= 1) {
                zmin = fminf(zmin, __shfl_xor(zmin, o, TPT));
                zmax = fmaxf(zmax, __shfl_xor(zmax, o, TPT));
            }
            // the format is defined in IEEE fp64: scale = bf16(fl64(fl64(max -
            // min) / 15)) rounded once from fp64, code = rint(fl64(fl64(z -
            // min) / scale)) clamped to 0..15 (correctly rounded divisions)
            const double lo = (double)zmin;
            const double scale64 = bf16_grid_f64(((double)zmax - lo) / 15.0);
            const float scale = (float)scale64;  // exact: a bf16 value (or +inf)
            uint32_t nib = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                double c = scale64 > 0.0 ? rint(((double)z[e] - lo) / scale64) : 0.0;
                c = fmin(fmax(c, 0.0), 15.0);
                nib |= (uint32_t)c << (4 * e);
            }
            // lanes j, j + 1 (j even) make one 32-bit word of eight codes
            const uint32_t hi = __shfl_down(nib, 1, TPT);
            if (t < TT && (j & 1) == 0)
                __builtin_amdgcn_raw_buffer_store_b32(nib | (hi << 16), lat_rsrc,
                                                      ((uint32_t)qt + t) * (DC / 2) + 2u * j, 0, 0);
            if (t < TT && j == 0)
                __builtin_amdgcn_raw_buffer_store_b32(
                    (pack_bf16(zmin, zmin) & 0xffffu) | (pack_bf16(scale, scale) << 16), par_rsrc,
                    ((uint32_t)qt + t) * 4u, 0, 0);
            continue;
        }
        // ---- sum the waves' shares, add b2, round, store (pairs of latent
        // values; rows past the range fall outside the store resource)
        static_assert((TT * DC / 2) % 256 == 0, "whole store passes");
#pragma unroll
        for (int n = 0; n < TT * DC / 512; ++n) {
            const int i = tid + 256 * n;
            const int t = i / (DC / 2), o = 2 * (i % (DC / 2));
            const float z0 = zp[0][o][t] + zp[1][o][t] + zp[2][o][t] + zp[3][o][t] + bias2[0];
            const float z1 = zp[0][o + 1][t] + zp[1][o + 1][t] + zp[2][o + 1][t] + zp[3][o + 1][t] +
                             bias2[1];
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16(z0, z1), lat_rsrc,
                                                  (((uint32_t)qt + t) * DC + o) * 2u, 0, 0);
        }
    }
}

template <int D, int HID, int DC, int KX, bool GELU, bool Q4>
__global__ __launch_bounds__(256, 2) void compress_mfma_kernel(
    const bf16_t *__restrict__ x, int64_t t0, int64_t nrows, int s, int k,
    const bf16_t *__restrict__ refs, int64_t Rcap, const uint16_t *__restrict__ idx,
    int64_t Ncap, int64_t q0, int64_t nq, int U, int tiles_per_block,
    const bf16_t *__restrict__ w1, const float *__restrict__ b1, const bf16_t *__restrict__ w2,
    const float *__restrict__ b2, bf16_t *__restrict__ lat) {
    compress_mfma_body<D, HID, DC, KX, GELU, Q4>(blockIdx.x, x, t0, nrows, s, k, refs, Rcap, idx,
                                                 Ncap, q0, nq, U, tiles_per_block, w1, b1, w2, b2,
                                                 lat);
}

// Batched appends: the one token t (ordinal q) of every unit of cache
// blockIdx.y of the set.  grid (U, n).
template <int D, int HID, int DC, int KX, bool GELU, bool Q4, bool PG = false>
__global__ __launch_bounds__(256, 2) void compress_append_kernel(AppendSet set, int64_t t, int s,
                                                                 int k, int64_t Rcap,
                                                                 int64_t Ncap, int64_t q, int U,
                                                                 PageMap pg) {
    const int item = blockIdx.y;
    compress_mfma_body<D, HID, DC, KX, GELU, Q4, PG>(
        blockIdx.x, (const bf16_t *)set.x[item], t, 1, s, k, (const bf16_t *)set.refs[item],
        Rcap, set.idx[item], Ncap, q, 1, U, 1, (const bf16_t *)set.w1[item], set.b1[item],
        (const bf16_t *)set.w2[item], set.b2[item], (bf16_t *)set.lat[item],
        PG ? item_pages(pg, set, item) : PageMap{});
}

template <int D, int HID, int DC>
void launch_cappend_t(const Dims &dm, int64_t t, int n, const AppendSet &set, int act,
                      hipStream_t st) {
    const int U = dm.B * dm.H;
    const int64_t q = t - refs_upto(t + 1, dm.s);
    auto kern = dm.k <= 4 ? (act == 0 ? compress_append_kernel<D, HID, DC, 4, true, false>
                                      : compress_append_kernel<D, HID, DC, 4, false, false>)
                          : (act == 0 ? compress_append_kernel<D, HID, DC, 8, true, false>
                                      : compress_append_kernel<D, HID, DC, 8, false, false>);
    if constexpr (DC <= 32) {
        if (dm.lat_fmt)
            kern = dm.k <= 4 ? (act == 0 ? compress_append_kernel<D, HID, DC, 4, true, true>
                                         : compress_append_kernel<D, HID, DC, 4, false, true>)
                             : (act == 0 ? compress_append_kernel<D, HID, DC, 8, true, true>
                                         : compress_append_kernel<D, HID, DC, 8, false, true>);
    }
    if (dm.pr)
        kern = dm.k <= 4
                   ? (act == 0 ? compress_append_kernel<D, HID, DC, 4, true, false, true>
                               : compress_append_kernel<D, HID, DC, 4, false, false, true>)
                   : (act == 0 ? compress_append_kernel<D, HID, DC, 8, true, false, true>
                               : compress_append_kernel<D, HID, DC, 8, false, false, true>);
    hipLaunchKernelGGL(kern, dim3((unsigned)U, (unsigned)n), dim3(256), 0, st, set, t, dm.s, dm.k,
                       dm.R, dm.N, q, U, set_pages(dm));
}

template <int D, int HID>
void launch_cappend_dc(const Dims &dm, int64_t t, int n, const AppendSet &set, int act,
                       hipStream_t st) {
    switch (dm.dc) {
        case 16: launch_cappend_t<D, HID, 16>(dm, t, n, set, act, st); break;
        case 32: launch_cappend_t<D, HID, 32>(dm, t, n, set, act, st); break;
        default: launch_cappend_t<D, HID, 64>(dm, t, n, set, act, st); break;
    }
}

template <int D, int HID, int DC>
void launch_cmfma_t(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0, int64_t nq,
                    const MlpArgs &m, const CacheArgs &c, hipStream_t st) {
    const int U = dm.B * dm.H;
    const int64_t tiles = (nq + 31) / 32;
    const int tpb = (int)std::max<int64_t>(1, std::min<int64_t>(16, (tiles * U + 1023) / 1024));
    const int64_t nblk = (tiles + tpb - 1) / tpb;
    auto kern = dm.k <= 4 ? (m.act == 0 ? compress_mfma_kernel<D, HID, DC, 4, true, false>
                                        : compress_mfma_kernel<D, HID, DC, 4, false, false>)
                          : (m.act == 0 ? compress_mfma_kernel<D, HID, DC, 8, true, false>
                                        : compress_mfma_kernel<D, HID, DC, 8, false, false>);
    if constexpr (DC <= 32) {
        if (dm.lat_fmt)
            kern = dm.k <= 4 ? (m.act == 0 ? compress_mfma_kernel<D, HID, DC, 4, true, true>
                                           : compress_mfma_kernel<D, HID, DC, 4, false, true>)
                             : (m.act == 0 ? compress_mfma_kernel<D, HID, DC, 8, true, true>
                                           : compress_mfma_kernel<D, HID, DC, 8, false, true>);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(nblk * U)), dim3(256), 0, st, (const bf16_t *)x, t0,
                       t1 - t0, dm.s, dm.k, (const bf16_t *)c.refs, dm.R, c.idx, dm.N, q0, nq, U,
                       tpb, (const bf16_t *)m.w1, m.b1, (const bf16_t *)m.w2, m.b2,
                       (bf16_t *)c.lat);
}

template <int D, int HID>
bool launch_cmfma_dc(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                     int64_t nq, const MlpArgs &m, const CacheArgs &c, hipStream_t st) {
    switch (dm.dc) {
        case 16: launch_cmfma_t<D, HID, 16>(dm, x, t0, t1, q0, nq, m, c, st); return true;
        case 32: launch_cmfma_t<D, HID, 32>(dm, x, t0, t1, q0, nq, m, c, st); return true;
        case 64: launch_cmfma_t<D, HID, 64>(dm, x, t0, t1, q0, nq, m, c, st); return true;
    }
    return false;
}

bool launch_compress_mfma(const Dims &dm, const void *x, int64_t t0, int64_t t1, int64_t q0,
                          int64_t nq, const MlpArgs &m, const CacheArgs &c, hipStream_t st) {
    if (dm.dtype != 1 || (m.hidden != 128 && m.hidden != 256)) return false;
    // the index lists and reference rows of a unit are read through buffer
    // resources with 31-bit byte ranges
    if (dm.N * dm.k * 2 > INT32_MAX || dm.R * dm.d * 2 > INT32_MAX ||
        dm.N * dm.dc * 2 > INT32_MAX)
        return false;
    if (dm.d == 128)
        return m.hidden == 256 ? launch_cmfma_dc<128, 256>(dm, x, t0, t1, q0, nq, m, c, st)
                               : launch_cmfma_dc<128, 128>(dm, x, t0, t1, q0, nq, m, c, st);
    return m.hidden == 256 ? launch_cmfma_dc<64, 256>(dm, x, t0, t1, q0, nq, m, c, st)
                           : launch_cmfma_dc<64, 128>(dm, x, t0, t1, q0, nq, m, c, st);
}

}  // namespace

bool append_batched_supported(const Dims &dm, const MlpArgs &comp) {
    // the matrix-core Compressor's conditions (launch_compress_mfma), and the
    // 16-bit reference ordinals that the split scan writes
    return dm.dtype == 1 && (comp.hidden == 128 || comp.hidden == 256) &&
           (dm.dc == 16 || dm.dc == 32 || dm.dc == 64) && dm.N * dm.k * 2 <= INT32_MAX &&
           dm.R * dm.d * 2 <= INT32_MAX && dm.N * dm.dc * 2 <= INT32_MAX;
}

size_t append_ws_bytes(const Dims &dm, int64_t t, int n) {
    // the batched search's split lists for one launch set of up to kAppendMax
    // caches, or a per-cache compress of one token; at a reference position
    // (nothing to compress) the next position's size, so that the size never
    // decreases with t
    const int64_t tt = (dm.s > 1 && t % dm.s == 0) ? t + 1 : t;
    return std::max(append_select_ws_bytes(dm, tt, std::min(n, kAppendMax)),
                    compress_ws_bytes(dm, tt, tt + 1));
}

hipError_t launch_append_compress(const Dims &dm, int64_t t, int n, const AppendSet &set,
                                  int hidden, int act, hipStream_t st) {
    if (dm.d == 128) {
        if (hidden == 256) launch_cappend_dc<128, 256>(dm, t, n, set, act, st);
        else launch_cappend_dc<128, 128>(dm, t, n, set, act, st);
    } else {
        if (hidden == 256) launch_cappend_dc<64, 256>(dm, t, n, set, act, st);
        else launch_cappend_dc<64, 128>(dm, t, n, set, act, st);
    }
    return hipGetLastError();
}

bool compress_q4_supported(const Dims &dm, const MlpArgs &comp) {
    // the matrix-core Compressor is the one that writes 4-bit rows: its
    // conditions (launch_compress_mfma), with d_c 16 or 32
    return dm.dtype == 1 && (dm.dc == 16 || dm.dc == 32) &&
           (comp.hidden == 128 || comp.hidden == 256) && dm.N * dm.k * 2 <= INT32_MAX &&
           dm.R * dm.d * 2 <= INT32_MAX && dm.N * dm.dc * 2 <= INT32_MAX;
}

// Workspace of one compress call (bf16 path): a 256-byte header holding the
// fallback counter, then one 8-byte fallback-list entry per compressed token
// of the range and unit, then (when the top-k search splits its reference
// ranges) each split's candidate lists and largest reference norms.
size_t compress_ws_bytes(const Dims &dm, int64_t t0, int64_t t1) {
    if (dm.pr) return paged_compress_ws_bytes(dm, t0, t1);
    if (dm.dtype != 1) return 0;
    const int64_t nq = toks_upto(t1, dm.s) - toks_upto(t0, dm.s);
    const size_t flist = ((size_t)nq * dm.B * dm.H * sizeof(uint64_t) + 255) & ~(size_t)255;
    // fallback list, then the search's split lists, whose space the split
    // exact scan of the fallback list reuses
    return std::max<size_t>(
        256 + flist + std::max(topk_split_ws_bytes(dm, t1, nq),
                               exact_list_ws_bytes(dm, t1, nq * dm.B * dm.H)),
        select_split_ws_bytes(dm, t0, t1));
}

hipError_t launch_compress(const Dims &dm, const void *x, int64_t t0, int64_t t1,
                           const MlpArgs &comp, const CacheArgs &c, void *ws, size_t ws_bytes,
                           uint32_t *stats, hipStream_t st) {
    if (dm.pr) return launch_compress_paged(dm, x, t0, t1, comp, c, ws, ws_bytes, stats, st);
    const int64_t q0 = toks_upto(t0, dm.s);
    const int64_t nq = toks_upto(t1, dm.s) - q0;
    if (nq <= 0) return hipSuccess;
    hipError_t e;
    if (dm.dtype == 1 && nq > kSmallRange) {
        uint32_t *fcount = (uint32_t *)ws;
        uint64_t *flist = (uint64_t *)((char *)ws + 256);
        e = launch_select_mfma(dm, x, t0, t1, q0, nq, c, flist, fcount, stats, st);
    } else if (dm.dtype == 1) {
        // a few tokens (a streaming append): exact, references split over blocks
        e = launch_select_split(dm, x, t0, t1, q0, nq, c, ws, st);
    } else {
        // fp32 storage, or a few tokens: exact scan
        e = launch_select_exact(dm, x, t0, t1, q0, nq, c, nullptr, nullptr, 0, nullptr, 0, st);
    }
    if (e != hipSuccess) return e;
    if (launch_compress_mfma(dm, x, t0, t1, q0, nq, comp, c, st)) return hipGetLastError();
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
