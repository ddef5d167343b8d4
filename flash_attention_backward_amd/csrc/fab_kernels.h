// Kernels of the flash-attention backward (gfx950, wave64, fp16 MFMA with fp32 accumulate).
//
// Row order inside a KV head hk: r = i*G + g for query row i of head h = hk*G + g, so the G
// heads that share a K/V head sit in the same row tiles and share every K/V tile.
//
// Launch sequence (all on one stream):
//   absmax   per-tensor max |q|, max |dO|           -> power-of-two prescale exponents
//   prep     q, dO -> power-of-two-scaled fp16 rows in the workspace
//   maskcls  class of every (32-row block, 64-key tile) of the mask (only with a mask)
//   qpass<0> walk 1 over keys: online softmax max/sum and delta numerator per row
//   merge    fixed-order merge of the key-range splits -> LSE, delta (packed output)
//   qpass<1> walk 2 over keys: dS = P (dP - delta), dQ += dS K
//   dqreduce fixed-order sum of per-split dQ (only when the keys were split)
//   kvpass   per 128-key tile: dV += P^T dO, dK += dS^T Q over every row of the group
#pragma once

#include "fab_common.h"
#include "fab_tiles.h"

namespace fab {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453;

// ----------------------------------------------------------------------------- absmax

__global__ __launch_bounds__(kThreads) void absmax_kernel(Params p) {
    __shared__ float red[2][kWaves];
    float mq = 0.0f, md = 0.0f;
    const int rows = p.N * p.H;
    // kThreads / D rows per step (D <= kThreads), each thread one element of one of them; four
    // steps' loads are issued before any is used
    const int rpi = kThreads / p.D, c = threadIdx.x % p.D, sub = threadIdx.x / p.D;
    const int stride = gridDim.x * rpi;
    for (int row0 = blockIdx.x * rpi + sub; row0 < rows; row0 += 4 * stride) {
        float xq[4], xd[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // q row (i, h) and dO row (h, i) for the same linear index
            const int row = row0 + u * stride;
            xq[u] = xd[u] = 0.0f;
            if (row < rows) {
                const int i = row / p.H, h = row - (row / p.H) * p.H;
                xq[u] = load_scalar(p.q + c * p.q_nb0 + i * p.q_nb1 + h * p.q_nb2, p.q_type);
                xd[u] = load_scalar(p.d + c * p.d_nb0 + h * p.d_nb1 + i * p.d_nb2, p.d_type);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            mq = fmaxf(mq, fabsf(xq[u]));
            md = fmaxf(md, fabsf(xd[u]));
        }
    }
    mq = wave_max(mq);
    md = wave_max(md);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = mq;
        red[1][threadIdx.x >> 6] = md;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0][0], b = red[1][0];
        for (int w = 1; w < kWaves; ++w) {
            a = fmaxf(a, red[0][w]);
            b = fmaxf(b, red[1][w]);
        }
        p.absmax_part[blockIdx.x] = a;
        p.absmax_part[p.npart + blockIdx.x] = b;
    }
}

// ----------------------------------------------------------------------------- prep

// One workgroup per (hk, 32-row block): q and dO rows, scaled by the power-of-two prescale
// (q also by the sign of the scale), rounded to fp16 and written row-major in the row order
// r = i*G + g (padding rows are 0).
template <int D>
__global__ __launch_bounds__(kThreads) void prep_kernel(Params p) {
    __shared__ float red[2][kWaves];

    // exponents from the absmax partials (every block reduces them identically)
    float aq = 0.0f, ad = 0.0f;
    for (int t = threadIdx.x; t < p.npart; t += kThreads) {
        aq = fmaxf(aq, p.absmax_part[t]);
        ad = fmaxf(ad, p.absmax_part[p.npart + t]);
    }
    aq = wave_max(aq);
    ad = wave_max(ad);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = aq;
        red[1][threadIdx.x >> 6] = ad;
    }
    __syncthreads();
    aq = red[0][0];
    ad = red[1][0];
    for (int w = 1; w < kWaves; ++w) {
        aq = fmaxf(aq, red[0][w]);
        ad = fmaxf(ad, red[1][w]);
    }
    const int eq = prescale_exponent(aq), edo = prescale_exponent(ad);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        p.scal[0] = eq;
        p.scal[1] = edo;
    }
    // q rows also take the sign of the scale, so every score product uses |scale|
    const float fq = p.scale < 0.0f ? -ldexpf(1.0f, eq) : ldexpf(1.0f, eq), fd = ldexpf(1.0f, edo);

    const int hk = blockIdx.x / p.RB, rb = blockIdx.x - (blockIdx.x / p.RB) * p.RB;
    constexpr int GR = D / 8;
    for (int item = threadIdx.x; item < 32 * GR; item += kThreads) {
        const int rr = item / GR, grp = item - (item / GR) * GR;
        const int r = rb * 32 + rr;
        f16x8 vq, vd;
        if (r < p.R) {
            const int i = r / p.G, g = r - (r / p.G) * p.G;
            const int h = hk * p.G + g;
            const char* qrow = p.q + (int64_t)i * p.q_nb1 + (int64_t)h * p.q_nb2;
            const char* drow = p.d + (int64_t)h * p.d_nb1 + (int64_t)i * p.d_nb2;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int c = 8 * grp + t;
                vq[t] = (_Float16)(load_scalar(qrow + c * p.q_nb0, p.q_type) * fq);
                vd[t] = (_Float16)(load_scalar(drow + c * p.d_nb0, p.d_type) * fd);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) vq[t] = vd[t] = (_Float16)0.0f;
        }
        const int64_t off = (((int64_t)hk * p.RB + rb) * 32 + rr) * D + 8 * grp;
        *(f16x8*)(p.qr + off) = vq;
        *(f16x8*)(p.dr + off) = vd;
    }
}

// ----------------------------------------------------------------------------- helpers

// dS exponent of KV head hk (for the key side, which sums dS over every row of the head):
// every wave reduces the head's bound partials of the merge. It ends in a wave-wide reduction,
// so every lane of the wave must call it (never from a lane-divergent branch).
FAB_DEV int head_ds_exponent(const Params& p, int hk) {
    float b = 0.0f;
    const float* bp = p.bound_part + (int64_t)hk * p.nbound;
    for (int t = threadIdx.x & 63; t < p.nbound; t += 64) b = fmaxf(b, bp[t]);
    return ds_exponent(wave_max(b));
}

// q_i . c for query row i of head h (K centre c of its KV head), fp64, fixed-order wave sum;
// every lane of the wave must call it and gets the sum.
FAB_DEV double q_dot_kcen(const Params& p, int h, int i, int lane) {
    const float* cen = p.kcen + (int64_t)(h / p.G) * p.D;
    double s = 0.0;
    for (int c = lane; c < p.D; c += 64)
        s = fma((double)load_scalar(p.q + (int64_t)c * p.q_nb0 + (int64_t)i * p.q_nb1 + (int64_t)h * p.q_nb2, p.q_type),
                (double)cen[c], s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
}

// ----------------------------------------------------------------------------- mask classes

// Class of every (32-row block, 64-key tile) of the mask, so the passes can skip tiles no row
// sees and skip mask reads where every entry is 0. Rows past N and keys past M are ignored.
// Grid: x = Hc * RB (Hc = 1 when the mask is shared by all heads), y = tile groups of 16.
constexpr int kClassTilesPerBlock = 16;

// ESZ: bytes per mask entry (2: F16, 4: F32). With one mask head the mask row depends on the
// query row i only, and the G rows r = i*G + g share it: a thread whose row repeats the previous
// row's i reads nothing (its entries count as both 0 and -inf, neutral for the all-lanes tests).
template <int ESZ>
__global__ __launch_bounds__(kThreads) void maskclass_kernel(Params p) {
    __shared__ unsigned int red[kClassTilesPerBlock][kWaves];
    const int hc = blockIdx.x / p.RB, rb = blockIdx.x - (blockIdx.x / p.RB) * p.RB;
    const int wave = threadIdx.x >> 6;
    const int rr = threadIdx.x >> 3, kg = threadIdx.x & 7;
    const int r = rb * 32 + rr;
    const int i = r / p.G, gh = r - (r / p.G) * p.G;
    const bool repeat = p.Hm == 1 && rr > 0 && (r - 1) / p.G == i;
    const bool row_ok = r < p.R && !repeat;
    const char* mrow = p.mask + (int64_t)i * p.m_nb1 + (int64_t)(p.Hm == 1 ? 0 : hc * p.G + gh) * p.m_nb2;
    const int tb = blockIdx.y * kClassTilesPerBlock;
    const int te = min(p.KT, tb + kClassTilesPerBlock);
    constexpr int esz = ESZ;
    // 16-byte loads of 8 consecutive entries when the rows allow them
    const bool vec = (((uintptr_t)p.mask | (uintptr_t)p.m_nb1 | (uintptr_t)p.m_nb2) & 15) == 0;
    // entries of this thread in every tile: keys t*64 + 8*kg .. +7; all loads issued first
    u32x4 raw[kClassTilesPerBlock][ESZ / 2];
#pragma unroll
    for (int k = 0; k < kClassTilesPerBlock; ++k) {
        const int t = tb + k;
        const int j = t * kQTileKeys + 8 * kg;
#pragma unroll
        for (int h = 0; h < ESZ / 2; ++h) raw[k][h] = u32x4{0u, 0u, 0u, 0u};
        if (row_ok && t < te && vec && j + 8 <= p.M) {
#pragma unroll
            for (int h = 0; h < ESZ / 2; ++h) raw[k][h] = *(const u32x4*)(mrow + (int64_t)j * esz + 16 * h);
        }
    }
#pragma unroll
    for (int k = 0; k < kClassTilesPerBlock; ++k) {
        const int t = tb + k;
        const int j = t * kQTileKeys + 8 * kg;
        bool all0 = true, allinf = true;
        if (row_ok && t < te) {
            if (vec && j + 8 <= p.M) {
                if constexpr (ESZ == 2) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const unsigned int x = raw[k][0][w];
                        // fp16 zero: bits 0x0000 or 0x8000; fp16 -inf: 0xfc00
                        all0 = all0 && ((x & 0x7fff7fffu) == 0u);
                        allinf = allinf && (x == 0xfc00fc00u);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const unsigned int x = raw[k][w >> 2][w & 3];
                        all0 = all0 && ((x & 0x7fffffffu) == 0u);
                        allinf = allinf && (x == (unsigned int)kNegInfBits);
                    }
                }
            } else {
                for (int e = 0; e < 8; ++e) {
                    if (j + e >= p.M) break;
                    const float x = p.m_type == FA_BACK_F16 ? (float)*(const _Float16*)(mrow + 2 * (int64_t)(j + e))
                                                             : *(const float*)(mrow + 4 * (int64_t)(j + e));
                    all0 = all0 && (x == 0.0f);
                    allinf = allinf && (x == neg_inf());
                }
            }
        }
        const bool w0 = __all(all0), winf = __all(allinf);
        if ((threadIdx.x & 63) == 0) red[k][wave] = (w0 ? 1u : 0u) | (winf ? 2u : 0u);
    }
    __syncthreads();
    if (threadIdx.x < kClassTilesPerBlock && tb + (int)threadIdx.x < te) {
        unsigned int f = 3u;
        for (int w = 0; w < kWaves; ++w) f &= red[threadIdx.x][w];
        p.mcls[((int64_t)hc * p.RB + rb) * p.KT + tb + threadIdx.x] =
            (unsigned char)((f & 2u) ? kMaskDead : ((f & 1u) ? kMaskZero : kMaskMixed));
    }
}

// The same classes with one mask head, reading each distinct query row of a block once: the
// rows r = i*G + g of a 32-row block share the mask row of query i. Wave w, lane l: key chunk
// kc = l & 7 (8 keys), tile ts = (l >> 3) + 8 (w & 1) of the block's 16, row group w >> 1 (the
// block's query rows i_lo, i_lo + 2, ... or i_lo + 1, i_lo + 3, ...). A tile's 8 chunk lanes
// meet in a ballot, its two row groups in LDS. Rows past R and keys past M are ignored; a tile
// with no row left is dead, as in maskclass_kernel.
template <int ESZ>
__global__ __launch_bounds__(kThreads) void maskclass_rows_kernel(Params p) {
    __shared__ unsigned int red[kClassTilesPerBlock][2];
    const int rb = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int kc = lane & 7, ts = (lane >> 3) + 8 * (wave & 1), rg = wave >> 1;
    const int r0 = rb * 32, r1 = min(p.R, r0 + 32);
    const int i_lo = r0 / p.G, i_hi = r1 > r0 ? (r1 - 1) / p.G : i_lo - 1;
    const int t = blockIdx.y * kClassTilesPerBlock + ts;
    const int j = t * kQTileKeys + 8 * kc;
    const bool vec = (((uintptr_t)p.mask | (uintptr_t)p.m_nb1) & 15) == 0;
    bool all0 = true, allinf = true;
    if (t < p.KT) {
#pragma unroll 4
        for (int i = i_lo + rg; i <= i_hi; i += 2) {
            const char* mrow = p.mask + (int64_t)i * p.m_nb1;
            if (vec && j + 8 <= p.M) {
                u32x4 raw[ESZ / 2];
#pragma unroll
                for (int h = 0; h < ESZ / 2; ++h) raw[h] = *(const u32x4*)(mrow + (int64_t)j * ESZ + 16 * h);
                if constexpr (ESZ == 2) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const unsigned int x = raw[0][w];
                        all0 = all0 && ((x & 0x7fff7fffu) == 0u);
                        allinf = allinf && (x == 0xfc00fc00u);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const unsigned int x = raw[w >> 2][w & 3];
                        all0 = all0 && ((x & 0x7fffffffu) == 0u);
                        allinf = allinf && (x == (unsigned int)kNegInfBits);
                    }
                }
            } else {
                for (int e = 0; e < 8; ++e) {
                    if (j + e >= p.M) break;
                    const float x = p.m_type == FA_BACK_F16 ? (float)*(const _Float16*)(mrow + 2 * (int64_t)(j + e))
                                                             : *(const float*)(mrow + 4 * (int64_t)(j + e));
                    all0 = all0 && (x == 0.0f);
                    allinf = allinf && (x == neg_inf());
                }
            }
        }
    }
    const unsigned long long m0 = __ballot(all0), mi = __ballot(allinf);
    if (kc == 0) {
        const int sh = lane & ~7;
        const unsigned int g0 = ((m0 >> sh) & 0xffull) == 0xffull ? 1u : 0u;
        const unsigned int gi = ((mi >> sh) & 0xffull) == 0xffull ? 2u : 0u;
        red[ts][rg] = g0 | gi;
    }
    __syncthreads();
    if (threadIdx.x < kClassTilesPerBlock) {
        const int tt = blockIdx.y * kClassTilesPerBlock + (int)threadIdx.x;
        if (tt < p.KT) {
            const unsigned int f = red[threadIdx.x][0] & red[threadIdx.x][1];
            p.mcls[(int64_t)rb * p.KT + tt] = (unsigned char)((f & 2u) ? kMaskDead : ((f & 1u) ? kMaskZero : kMaskMixed));
        }
    }
}

// The class without a stored mask: no mask (kMaskZero), or the causal tail, where query row i
// sees keys j <= M - N + i; the block's rows r < R hold query rows ilo..ihi and the tile keys
// j0..j1 < M: the class the stored mask would get.
FAB_DEV int mask_class_implicit(const Params& p, int rb, int t) {
    if (p.m_type == FA_BACK_NONE) return kMaskZero;
    const int ilo = (32 * rb) / p.G, ihi = min(32 * rb + 31, p.R - 1) / p.G;
    const int j0 = t * kQTileKeys, j1 = min(j0 + kQTileKeys - 1, p.M - 1);
    const int off = p.M - p.N;
    if (j0 > off + ihi) return kMaskDead;
    if (j1 <= off + ilo) return kMaskZero;
    return kMaskMixed;
}

// Class of (32-row block rb, 64-key tile t): none or causal-tail masks from the indices, stored
// masks from the class table.
FAB_DEV int mask_class(const Params& p, int hk, int rb, int t) {
    if (p.m_type == FA_BACK_NONE || p.m_type == FA_BACK_CAUSAL_TAIL) return mask_class_implicit(p, rb, t);
    const int hc = p.Hm == 1 ? 0 : hk;
    return p.mcls[((int64_t)hc * p.RB + rb) * p.KT + t];
}

// mask_class for wave-uniform arguments: a stored class is read through the scalar cache (the
// load counts on lgkmcnt, so waiting for it leaves the wave's vector loads and copies in flight).
// The dword read may cover up to 3 bytes past the table, which the workspace still holds.
FAB_DEV int mask_class_s(const Params& p, int hk, int rb, int t) {
    if (p.m_type == FA_BACK_NONE || p.m_type == FA_BACK_CAUSAL_TAIL) return mask_class_implicit(p, rb, t);
    const int hc = p.Hm == 1 ? 0 : hk;
    const int64_t o = ((int64_t)hc * p.RB + rb) * p.KT + t;
    typedef const __attribute__((address_space(4))) unsigned int cu32;
    const unsigned int w = *(cu32*)(uintptr_t)(p.mcls + (o & ~(int64_t)3));
    return (int)((w >> (8 * (int)(o & 3))) & 0xffu);
}

FAB_DEV float mask_at(const char* mrow, int type, int j) {
    return type == FA_BACK_F16 ? (float)*(const _Float16*)(mrow + 2 * (int64_t)j)
                               : *(const float*)(mrow + 4 * (int64_t)j);
}

// Mask entry of key j for query row i (whose stored mask row is mrow, if any).
FAB_DEV float mask_value(const Params& p, const char* mrow, int i, int j) {
    if (p.m_type == FA_BACK_CAUSAL_TAIL) return j <= p.M - p.N + i ? 0.0f : neg_inf();
    return mask_at(mrow, p.m_type, j);
}

// ----------------------------------------------------------------------------- product loops

// Two interleaved 32x32 products over d (two independent accumulator chains, so the matrix
// core never waits for its own previous result), first operands read from LDS PF steps
// ahead of their use:  sa += A1 * B1,  pa += A2 * B2, where the A operands are frag_rows reads
// of tiles t1 and t2 (rows m1 .. m1+31, m2a ..) and the B operands come from `b1` / `b2` in
// registers or, if b2 is null, from frag_rows reads of tile t2b (rows m2b .. m2b+31).
template <int D, int PF>
FAB_DEV void mfma_pair_d(const _Float16* t1, int m1, const f16x8* b1, const _Float16* t2, int m2a,
                         const f16x8* b2, const _Float16* t2b, int m2b, f32x16& sa, f32x16& pa,
                         int lane, const Swz& z) {
    constexpr int KS = D / 16;
    constexpr int NB = PF + 1;
    f16x8 r1[NB], r2[NB], r3[NB];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        r1[k] = frag_rows<D>(t1, m1, k, lane, z);
        r2[k] = frag_rows<D>(t2, m2a, k, lane, z);
        if (!b2) r3[k] = frag_rows<D>(t2b, m2b, k, lane, z);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) {
            r1[(ks + PF) % NB] = frag_rows<D>(t1, m1, ks + PF, lane, z);
            r2[(ks + PF) % NB] = frag_rows<D>(t2, m2a, ks + PF, lane, z);
            if (!b2) r3[(ks + PF) % NB] = frag_rows<D>(t2b, m2b, ks + PF, lane, z);
        }
        sa = mfma32(r1[ks % NB], b1[ks], sa);
        pa = mfma32(r2[ks % NB], b2 ? b2[ks] : r3[ks % NB], pa);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// acc[md] += A(md, rh) * b[rh] over md = 0 .. D/32-1 and rh = 0, 1, with A the frag_cols read
// (contraction over 32 rows kbase .. kbase+31 of tile t) fetched PF products ahead; the
// accumulator changes between consecutive products.
template <int D, int PF>
FAB_DEV void mfma_cols(const _Float16* t, int kbase, const f16x8 b[2], f32x16* acc, int lane,
                       const Swz& z) {
    constexpr int MD = D / 32;
    constexpr int NP = 2 * MD;                       // products, index n = rh*MD + md
    constexpr int NB = PF + 1;
    f16x8 r[NB];
#pragma unroll
    for (int n = 0; n < PF; ++n) r[n] = frag_cols<D>(t, n % MD, kbase + 16 * (n / MD), lane, z);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        if (n + PF < NP) r[(n + PF) % NB] = frag_cols<D>(t, (n + PF) % MD, kbase + 16 * ((n + PF) / MD), lane, z);
        acc[n % MD] = mfma32(r[n % NB], b[n / MD], acc[n % MD]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ----------------------------------------------------------------------------- query side

// Workgroup: one KV head, 4 row blocks of 32 rows, one key-range split, and 8 waves:
//   S waves (0..3)  one row block each; q and dO fragments in registers. For every 32-key
//                   sub-tile: S^T = K Q^T and dP^T = V dO^T, then walk 1 updates the online
//                   softmax statistics, walk 2 forms dS = P (dP - delta) and hands it over
//                   through LDS. They also queue the DMA of the raw q8_0 / q4_0 bytes of
//                   sub-tile s+2.
//   K waves (4..7)  decode K and V of sub-tile s+1 into LDS while the S waves compute s; in
//                   walk 2 each also holds the dQ accumulators of one row block and consumes
//                   the dS of sub-tile s-1: dQ^T += K^T dS^T.
// A slot holds the K and V tiles of one sub-tile; three slots rotate (S waves at s, decode at
// s+1, dQ at s-1), the staged bytes and the dS exchange are double-buffered; one barrier per
// sub-tile. Every wave stays within 256 registers, so each SIMD runs an S wave and a K wave.
// S^T = K Q^T puts one query row per lane column and 16 keys per lane; lanes l and l^32
// together hold a row's 32 keys.
constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * kWave;
constexpr int kSubKeys = 32;

// With the decoded image of the cache (IMG), the S waves copy whole slots from it two sub-tiles
// ahead: four slots rotate and nothing is staged.
template <int D, bool IMG = false>
struct QLds {
    static constexpr int kTile = kSubKeys * D * 2;                 // bytes of a K or V sub-tile
    static constexpr int kSlot = 2 * kTile;                        // K tile then V tile
    static constexpr int kRaw = RawTile<D, kSubKeys>::kBytes;      // block bytes of one sub-tile
    static constexpr int kSlots = IMG ? 4 : 3;
    static constexpr int kOffSlot = 0;
    static constexpr int kOffRaw = kOffSlot + kSlots * kSlot;      // [2][K, V] staged bytes
    static constexpr int kOffEx = kOffRaw + (IMG ? 0 : 4 * kRaw);  // [2][4 row blocks] dS, 2 KB
    static constexpr int kOffCls = kOffEx + 2 * 4 * 2048;          // [2][4 row blocks] mask class
    static constexpr int kBytes = kOffCls + 16;
};

// How the K waves decode a sub-tile: both K and V q8_0, both block types (q8_0 / q4_0), or
// anything else (F32/F16/BF16 rows read from global memory, possibly centred). Each is a
// kernel of its own, so that no decode holds registers in another's loop. kDecImg decodes
// nothing: the slots are copied from the image kvimage_kernel wrote (the same decode, done
// once per sub-tile instead of once per workgroup).
constexpr int kDecQ8 = 0;
constexpr int kDecBlk = 1;
constexpr int kDecGen = 2;
constexpr int kDecImg = 3;

// Byte offset of head hk's first row from a 16-byte boundary (q8_0 rows with fixed strides).
FAB_DEV int q8_misalign(const char* base, int64_t nb2, int hk) {
    return (int)((uintptr_t)(base + (int64_t)hk * nb2) & 15);
}

// Decode K and V of sub-tile s (keys 32s ..) of head hk into the swizzled fp16 tiles tk, tv:
// from the bytes staged in rk, rv for the block types, from global memory for the others
// (centred where a centre is given); keys >= M become 0. kw is this wave among the 4 decoding
// waves and `last` the bound of its q8_0 items. The query-side walks and kvimage_kernel both
// decode through here, so the image holds exactly the walks' own tiles.
template <int D, int DEC>
FAB_DEV void decode_sub(const Params& p, int hk, bool fixed16, const Q8Fixed<D>& qf, int s,
                        const unsigned char* rk, const unsigned char* rv, _Float16* tk, _Float16* tv,
                        int kw, int lane, int last) {
    const char* kh = p.k + (int64_t)hk * p.k_nb2;
    const char* vh = p.v + (int64_t)hk * p.v_nb2;
    const int j0 = s * kSubKeys;
    if constexpr (DEC == kDecQ8) {
        if (fixed16)
            qf.decode(j0, p.M, rk, rv, (unsigned char*)tk, (unsigned char*)tv, kw, last);
        else
            decode_blk_pair32<D, true>(kh, p.k_nb1, p.k_type, vh, p.v_nb1, p.v_type, j0, p.M,
                                       rk, rv, tk, tv, kw, last, lane);
    } else if constexpr (DEC == kDecBlk) {
        decode_blk_pair32<D, false>(kh, p.k_nb1, p.k_type, vh, p.v_nb1, p.v_type, j0, p.M,
                                    rk, rv, tk, tv, kw, last, lane);
    } else {
        const int ktid = kw * 64 + lane;
        decode_tile<D, kSubKeys, 256>(p.k, p.k_type, p.k_nb1, p.k_nb2, hk, j0, p.M, rk, tk, ktid,
                                      p.kcen ? p.kcen + (int64_t)hk * D : nullptr);
        decode_tile<D, kSubKeys, 256>(p.v, p.v_type, p.v_nb1, p.v_nb2, hk, j0, p.M, rv, tv, ktid,
                                      p.vcen ? p.vcen + (int64_t)hk * D : nullptr);
    }
}

// Walk-1 statistics of one query row over the keys seen so far (the lane's half of the row's
// entries): running max m of the scaled scores (log2 units), l = sum exp2(s - m) and
// d' = sum exp2(s - m) dp carried in fp64, and max |dp|.
struct W1Row {
    float m;
    double l, d;
    float b;
};

FAB_DEV void w1_init(W1Row& w) {
    w.m = neg_inf();
    w.l = 0.0;
    w.d = 0.0;
    w.b = 0.0f;
}

// Folds the 32 keys j0 .. j0+31 of one 32-row block into the row's statistics: sa holds the
// products q.k (prescaled; sc2 takes them to log2 units), pa the products dO.v, in the lane's
// 16 entries of the 32 x 32 result. fast: every entry visible (no mask term, no ragged edge);
// otherwise the mask (class cls) and the bounds decide per entry, and an entry with mask 0 gets
// exactly the arithmetic of the fast path.
FAB_DEV void w1_fold(const Params& p, W1Row& w, const f32x16& sa, const f32x16& pa, bool fast, int cls,
                     bool row_ok, const char* mrow, int i, int j0, int g, float sc2) {
    if (fast) {
        // every entry visible: the scale is positive, so max(s) = sc2 * max(sa)
        float tm = sa[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) tm = fmaxf(tm, sa[v]);
        tm = max_halves(tm);
        const float mnew = fmaxf(w.m, tm * sc2);
        const float alpha = fast_exp2(w.m - mnew);
        float ls = 0.0f, ds = 0.0f, bm = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float e = fast_exp2(fmaf(sa[v], sc2, -mnew));
            ls += e;
            ds = fmaf(e, pa[v], ds);
            bm = fmaxf(bm, fabsf(pa[v]));
        }
        w.l = fma(w.l, (double)alpha, (double)ls);
        w.d = fma(w.d, (double)alpha, (double)ds);
        w.m = mnew;
        w.b = fmaxf(w.b, bm);
        return;
    }
    float madd[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int key = j0 + crow(v, g);
        float mv = 0.0f;
        if (!row_ok || key >= p.M) mv = neg_inf();
        else if (cls == kMaskMixed) mv = mask_value(p, mrow, i, key) * kLog2e;
        madd[v] = mv;
    }
    float tmax = neg_inf();
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (madd[v] != neg_inf()) tmax = fmaxf(tmax, fmaf(sa[v], sc2, madd[v]));
    tmax = max_halves(tmax);
    const float mnew = fmaxf(w.m, tmax);
    if (mnew != neg_inf()) {
        const float alpha = fast_exp2(w.m - mnew);
        float ls = 0.0f, ds = 0.0f, bm = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            if (madd[v] == neg_inf()) continue;
            const float e = fast_exp2(fmaf(sa[v], sc2, madd[v] - mnew));
            ls += e;
            ds = fmaf(e, pa[v], ds);
            bm = fmaxf(bm, fabsf(pa[v]));
        }
        w.l = fma(w.l, (double)alpha, (double)ls);
        w.d = fma(w.d, (double)alpha, (double)ds);
        w.m = mnew;
        w.b = fmaxf(w.b, bm);
    }
}

// The row's record for key-range split `split`: the two lane halves' sums, carried in fp64,
// rounded once to fp32.
FAB_DEV void w1_record(const Params& p, const W1Row& w, int split, int ridx, int g) {
    const double lo = w.l + __shfl_xor(w.l, 32);
    const double dd = w.d + __shfl_xor(w.d, 32);
    const float bb = fmaxf(w.b, __shfl_xor(w.b, 32));
    if (g == 0)
        p.part_rec[(int64_t)split * p.Hkv * p.RB * 32 + ridx] = f32x4{w.m, (float)lo, (float)dd, bb};
}

template <int D, bool GRAD, int DEC>
__global__ __launch_bounds__(kQThreads, 1) void qpass_kernel(Params p) {
    constexpr bool IMG = DEC == kDecImg;
    using L = QLds<D, IMG>;
    // The K waves decode whole sub-tiles. (Handing the V half to the S waves was measured: with
    // the DMA queued from the S waves, they are the busier role.)
    constexpr bool kSplitDecode = false;
    constexpr int KS = D / 16;     // 16-deep steps of a contraction over d
    constexpr int MD = D / 32;     // 32-wide d blocks of dQ
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l32 = lane & 31, g = lane >> 5;
    const int role = wave >> 2, w4 = wave & 3;
    const int hk = blockIdx.x % p.Hkv;
    const int rt = blockIdx.x / p.Hkv;
    const int split = blockIdx.y;
    const int rb = rt * kWaves + w4;
    const bool active = rb < p.RB;
    const int rowsHK = p.RB * 32;
    const int r = rb * 32 + l32;
    const int i = r / p.G, gh = r - (r / p.G) * p.G;
    const int h = hk * p.G + gh;
    const bool row_ok = active && r < p.R;
    const int ridx = hk * rowsHK + r;
    const int NS = (p.M + kSubKeys - 1) / kSubKeys;
    const int tps = GRAD ? p.tiles_per_split : p.w1_tps;    // walk 1 has key ranges of its own
    const int s_begin = 2 * split * tps;
    const int s_end = min(NS, 2 * min(p.KT, (split + 1) * tps));
    const int eq = p.scal[0], edo = p.scal[1];

    auto slot = [&](int s) { return lds + L::kOffSlot + (s % L::kSlots) * L::kSlot; };
    auto rawK = [&](int s) { return lds + L::kOffRaw + ((s & 1) * 2 + 0) * L::kRaw; };
    auto rawV = [&](int s) { return lds + L::kOffRaw + ((s & 1) * 2 + 1) * L::kRaw; };
    auto exch = [&](int s) { return lds + L::kOffEx + ((s & 1) * 4 + w4) * 2048; };
    auto wclass = [&](int s) { return active ? mask_class(p, hk, rb, s >> 1) : kMaskDead; };
    // the class of sub-tile s for row block w4, passed from the K waves (which load it from
    // HBM one sub-tile ahead) to the S waves
    unsigned char* clsx = lds + L::kOffCls;

    if (role == 0) {
        // ================= S waves
        f16x8 bq[KS], bd[KS];
        if (active) {
            const _Float16* rq = p.qr + ((int64_t)hk * rowsHK + r) * D;
            const _Float16* rd = p.dr + ((int64_t)hk * rowsHK + r) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bq[ks] = *(const f16x8*)(rq + 16 * ks + 8 * g);
                bd[ks] = *(const f16x8*)(rd + 16 * ks + 8 * g);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < 8; ++t) bq[ks][t] = bd[ks][t] = (_Float16)0.0f;
        }
        const bool has_mask = p.m_type != FA_BACK_NONE;
        const char* mrow = (has_mask && row_ok)
            ? p.mask + (int64_t)i * p.m_nb1 + (int64_t)(p.Hm == 1 ? 0 : h) * p.m_nb2 : nullptr;
        // q rows carry the sign of the scale (prep), so the score scale is positive here
        const float sc2 = fabsf(p.scale) * ldexpf(1.0f, -eq) * kLog2e;
        const bool full_rows = active && (rb + 1) * 32 <= p.R;
        W1Row w1;   // walk 1 state
        w1_init(w1);
        // walk 2 state: p * 2^-ks = exp2(s2 - lse2 - ks), lse2 stored less the image exponent
        float lse2 = pos_inf(), dlt = 0.0f, lse2k = 0.0f;
        if (GRAD) {
            if (row_ok) {
                lse2 = p.row_lse2[ridx];
                dlt = p.row_dlt[ridx];
            }
            lse2k = lse2 + (float)((row_ok ? p.row_ks[ridx] : 0) + kPScaleLog2);
        }
        const bool dead = (lse2 == pos_inf());
        const RowWalk<D> rw = make_row_walk<D>(lane);

        const bool sdec = kSplitDecode && is_block_type(p.k_type) && is_block_type(p.v_type);
        const char* kh = p.k + (int64_t)hk * p.k_nb2;
        const char* vh = p.v + (int64_t)hk * p.v_nb2;
        // the V half of sub-tile t, staged by the K waves
        auto sdecode = [&](int t) {
            decode_blk_pair32<D, false>(kh, p.k_nb1, p.k_type, vh, p.v_nb1, p.v_type, t * kSubKeys, p.M, rawK(t), rawV(t),
                                (_Float16*)slot(t), (_Float16*)(slot(t) + L::kTile),
                                Q8Pair<D>::UPT + w4, Q8Pair<D>::U, lane);
        };
        // block bytes are staged by these waves: the LDS reads that follow the DMA here are
        // plain loads, which the compiler does not hold back for the DMA in flight (it makes
        // transpose reads wait for it)
        RawDma<D, kSubKeys, 256> dk, dv;
        if constexpr (!IMG) {
            dk.init(kh, p.k_nb1, block_row_bytes(p.k_type, D), s_begin * kSubKeys, w4 * 64 + lane);
            dv.init(vh, p.v_nb1, block_row_bytes(p.v_type, D), s_begin * kSubKeys, w4 * 64 + lane);
        }
        // image: the slot of sub-tile t is one contiguous run of kSlot bytes; each S wave copies
        // a quarter of it in 1 KB pieces (hidden from the compiler: the copies stay in flight
        // across the products, and the block barrier below waits for them by count)
        constexpr int NI = L::kSlot / (4 * 1024);
        const unsigned char* img = IMG ? p.kvimg + (int64_t)hk * p.img_ns * L::kSlot : nullptr;
        auto sdma = [&](int t) {
            if constexpr (IMG) {
                const unsigned char* src = img + (int64_t)t * L::kSlot + w4 * (NI * 1024);
                const uint32_t dst = lds_addr(slot(t)) + (uint32_t)(w4 * (NI * 1024));
#pragma unroll
                for (int it = 0; it < NI; ++it) dma16_hidden(src + it * 1024, 16u * lane, dst + it * 1024);
            } else {
                if (is_block_type(p.k_type)) dk.issue(rawK(t), p.M, w4);
                if (is_block_type(p.v_type)) dv.issue(rawV(t), p.M, w4);
            }
        };
        // prologue: sub-tile s_begin staged and decoded (V half here, K half by the K waves),
        // the bytes of s_begin+1 on their way; from the image, the first two slots on their way
        if constexpr (IMG) {
            // the q and dO fragments are in registers before the first copy is queued: a wait
            // for them left inside the loop would wait for the copies in flight as well
            wait_all_mem();
        }
        if constexpr (IMG) {
            // the K waves copy the slots from the image
            lds_barrier();
        } else {
            if (s_begin < s_end) sdma(s_begin);
            wait_all_mem();
            __syncthreads();
            if (s_begin + 1 < s_end) sdma(s_begin + 1);
        }
        if (sdec && s_begin < s_end) sdecode(s_begin);
        for (int s = s_begin; s <= s_end; ++s) {
            wait_all_mem();
            __syncthreads();   // sub-tile s decoded or copied and its class posted; exchange slot s free
            if (s == s_end) break;
            if (!IMG && s + 2 < s_end) sdma(s + 2);
            const int cls = __builtin_amdgcn_readfirstlane(clsx[(s & 1) * 4 + w4]);
            if (cls == kMaskDead) {
                if (sdec && s + 1 < s_end) sdecode(s + 1);
                continue;
            }
            f32x16 sa, pa;
#pragma unroll
            for (int v = 0; v < 16; ++v) sa[v] = pa[v] = 0.0f;
            // both roles' products at raised priority: whichever wave has products to issue goes
            // ahead of the other's exponentials
            mfma_prio_hi();
            pair_rows<D, 2>(slot(s), bq, bd, sa, pa, rw);
            mfma_prio_lo();
            const int j0 = s * kSubKeys;
            const bool fast = full_rows && cls == kMaskZero && j0 + kSubKeys <= p.M;
            if (!GRAD) {
                w1_fold(p, w1, sa, pa, fast, cls, row_ok, mrow, i, j0, g, sc2);
            } else {
                f16x8 bs[2];
                if (fast) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float pv = fast_exp2(fmaf(sa[v], sc2, -lse2k));
                        bs[v >> 3][v & 7] = ds_f16(pv, pa[v], dlt);
                    }
                } else {
                    // masked or ragged sub-tile, same arithmetic as above for mask-0 entries
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = j0 + crow(v, g);
                        float mv = 0.0f;
                        if (!row_ok || key >= p.M) mv = neg_inf();
                        else if (cls == kMaskMixed) mv = mask_value(p, mrow, i, key) * kLog2e;
                        const float pv = (dead || mv == neg_inf()) ? 0.0f : fast_exp2(fmaf(sa[v], sc2, mv - lse2k));
                        bs[v >> 3][v & 7] = ds_f16(pv, pa[v], dlt);
                    }
                }
                unsigned char* ex = exch(s);
                *(f16x8*)(ex + lane * 16) = bs[0];
                *(f16x8*)(ex + 1024 + lane * 16) = bs[1];
            }
            if (sdec && s + 1 < s_end) sdecode(s + 1);
        }
        if (!GRAD && active) w1_record(p, w1, split, ridx, g);
        return;
    }

    // ================= K waves
    const int kw = wave - 4;                          // 0..3, uniform
    // q8_0 with row strides that are multiples of 16 bytes: offsets formed once
    const bool fixed16 = DEC == kDecQ8 && ((p.k_nb1 | p.v_nb1) & 15) == 0;
    Q8Fixed<D> qf;
    if constexpr (DEC == kDecQ8) {
        if (fixed16) qf.init(kw, q8_misalign(p.k, p.k_nb2, hk), q8_misalign(p.v, p.v_nb2, hk), lane);
    }
    auto kdecode = [&](int s) {
        constexpr int last = kSplitDecode ? Q8Pair<D>::UPT : Q8Pair<D>::U;
        if constexpr (!IMG)
            decode_sub<D, DEC>(p, hk, fixed16, qf, s, rawK(s), rawV(s), (_Float16*)slot(s),
                               (_Float16*)(slot(s) + L::kTile), kw, lane, last);
    };
    // image: the slot of sub-tile t is one contiguous run of kSlot bytes; each K wave copies a
    // quarter of it in 1 KB pieces (hidden from the compiler: the copies stay in flight across
    // the transpose reads, and the block barrier waits for them by count)
    constexpr int NI = L::kSlot / (4 * 1024);
    auto kdma = [&](int t) {
        if constexpr (IMG) {
            const unsigned char* src = p.kvimg + ((int64_t)hk * p.img_ns + t) * L::kSlot + kw * (NI * 1024);
            const uint32_t dst = lds_addr(slot(t)) + (uint32_t)(kw * (NI * 1024));
#pragma unroll
            for (int it = 0; it < NI; ++it) dma16_hidden(src + it * 1024, 16u * lane, dst + it * 1024);
        }
    };
    // the class of sub-tile s; with the image a scalar load, so that waiting for it leaves the
    // copies in flight
    auto kclass = [&](int s) {
        if constexpr (IMG) return active ? mask_class_s(p, hk, rb, s >> 1) : kMaskDead;
        else return wclass(s);
    };
    // prologue: the S waves stage sub-tile s_begin (or the K waves copy the first two slots);
    // its class is posted
    int cls_cur = s_begin < s_end ? kclass(s_begin) : kMaskDead;    // class of sub-tile s
    if (lane == 0) clsx[(s_begin & 1) * 4 + kw] = (unsigned char)cls_cur;
    if constexpr (IMG) {
        // the class loads are done before the first copy is queued
        wait_all_mem();
        if (s_begin < s_end) kdma(s_begin);
        if (s_begin + 1 < s_end) kdma(s_begin + 1);
        lds_barrier();   // the copies stay in flight: the first block barrier waits for them
    } else {
        __syncthreads();
    }
    if (s_begin < s_end) kdecode(s_begin);

    f32x16 dqacc[GRAD ? MD : 1];
    if (GRAD) {
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int v = 0; v < 16; ++v) dqacc[md][v] = 0.0f;
    }
    const ColWalk<D> cw = make_col_walk<D>(lane);
    int cls_last = kMaskDead;                                        // class of sub-tile s-1
    int cls_nx = s_begin + 1 < s_end ? kclass(s_begin + 1) : kMaskDead;   // s+1, in flight
    for (int s = s_begin; s <= s_end; ++s) {
        if (IMG && s + 1 < s_end) {
            dma_barrier<NI>();   // slot s+1 landed (needed next); the copies of s+2 stay in flight
        } else {
            wait_all_mem();
            __syncthreads();   // sub-tile s decoded and dS of s-1 exchanged
        }
        const int cls_prev = cls_last;
        cls_last = cls_cur;
        cls_cur = cls_nx;                                            // class of sub-tile s+1
        if (lane == 0 && s + 1 < s_end) clsx[((s + 1) & 1) * 4 + kw] = (unsigned char)cls_cur;
        cls_nx = s + 2 < s_end ? kclass(s + 2) : kMaskDead;          // in flight during sub-tile s
        if (IMG && s + 2 < s_end) kdma(s + 2);
        // the decode (vector ALU work) first, beside the S waves' products; then the dQ products,
        // beside the S waves' exponentials
        if (s + 1 < s_end) kdecode(s + 1);
        if (GRAD && s > s_begin && cls_prev != kMaskDead) {
            const unsigned char* ex = exch(s - 1);
            const f16x8 bb[2] = {*(const f16x8*)(ex + lane * 16), *(const f16x8*)(ex + 1024 + lane * 16)};
            mfma_prio_hi();
            cols_acc<D>(slot(s - 1), bb, dqacc, cw);
            mfma_prio_lo();
        }
        if (s == s_end) break;
    }
    if (GRAD && row_ok) {
        const int ksx = p.row_ks[ridx];   // the row's dS exponent
        const bool direct = p.splits == 1;
        const float fac = direct ? p.scale * ldexpf(1.0f, ksx - edo) : 1.0f;
        float* dst = direct ? p.dq + ((int64_t)h * p.N + i) * D
                            : p.dq_part + ((int64_t)split * p.Hkv * rowsHK + ridx) * D;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f32x4 o = {dqacc[md][4 * b] * fac, dqacc[md][4 * b + 1] * fac,
                           dqacc[md][4 * b + 2] * fac, dqacc[md][4 * b + 3] * fac};
                *(f32x4*)(dst + 32 * md + 8 * b + 4 * g) = o;
            }
    }
}

// ----------------------------------------------------------------------------- cache image

// The decoded cache for the query-side walks when several of their workgroups would decode each
// sub-tile: for every KV head and 32-key sub-tile, the LDS slot a walk decodes (swizzled fp16 K
// tile, then V tile, keys >= M zero), written out once to img [Hkv][img_ns][slot bytes]. A
// workgroup of 4 waves stages one sub-tile, decodes it with the walks' own decode and copies
// the slot out; the walks then copy slots instead of decoding (qpass_kernel<.., kDecImg>).
constexpr int kImgThreads = 256;

template <int D, int DEC>
__global__ __launch_bounds__(kImgThreads) void kvimage_kernel(Params p) {
    using L = QLds<D>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kSlot + 2 * L::kRaw];
    unsigned char* rk = lds + L::kSlot;
    unsigned char* rv = rk + L::kRaw;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int s = blockIdx.x, hk = blockIdx.y;
    const char* kh = p.k + (int64_t)hk * p.k_nb2;
    const char* vh = p.v + (int64_t)hk * p.v_nb2;
    RawDma<D, kSubKeys, kImgThreads> dk, dv;
    dk.init(kh, p.k_nb1, block_row_bytes(p.k_type, D), s * kSubKeys, threadIdx.x);
    dv.init(vh, p.v_nb1, block_row_bytes(p.v_type, D), s * kSubKeys, threadIdx.x);
    if (is_block_type(p.k_type)) dk.issue(rk, p.M, wave);
    if (is_block_type(p.v_type)) dv.issue(rv, p.M, wave);
    const bool fixed16 = DEC == kDecQ8 && ((p.k_nb1 | p.v_nb1) & 15) == 0;
    Q8Fixed<D> qf;
    if constexpr (DEC == kDecQ8) {
        if (fixed16) qf.init(wave, q8_misalign(p.k, p.k_nb2, hk), q8_misalign(p.v, p.v_nb2, hk), lane);
    }
    wait_all_mem();
    __syncthreads();
    decode_sub<D, DEC>(p, hk, fixed16, qf, s, rk, rv, (_Float16*)lds, (_Float16*)(lds + L::kTile),
                       wave, lane, Q8Pair<D>::U);
    __syncthreads();
    unsigned char* dst = p.kvimg + ((int64_t)hk * p.img_ns + s) * L::kSlot;
#pragma unroll
    for (int o = 16 * (int)threadIdx.x; o < L::kSlot; o += 16 * kImgThreads)
        *(uint4*)(dst + o) = *(const uint4*)(lds + o);
}

// ----------------------------------------------------------------------------- walk 1 by rows over the image

// Walk 1 with the rows owned, reading K and V from the decoded image: a workgroup takes one KV
// head, 8 row blocks of 32 rows (one per wave, its q and dO fragments in registers) and a key
// range. The image slots (32 keys each) are copied into LDS two at a time by all 8 waves (an
// eighth each, one pair ahead), and every wave forms S and dP of its rows against each slot
// and folds them into its rows' statistics. So all 8 waves issue products, two per SIMD, where
// the query-side kernel's walk 1 leaves half of its waves to the tile copies. The per-row
// arithmetic (w1_fold, w1_record) and the key ranges are those of the query-side kernel's
// walk 1, so both give the same records.
constexpr int kR1Waves = 8;
constexpr int kR1Threads = kR1Waves * kWave;

template <int D>
struct R1Lds {
    static constexpr int kSlot = 2 * kSubKeys * D * 2;   // K sub-tile, then V sub-tile (the image's slot)
    // two image slots per step (one barrier each; against one per step with three steps held:
    // 3.30 against 3.44 ms at N2048/M75520/D256), the next step copied during this one
    static constexpr int kSub = 2;                       // image slots per step
    static constexpr int kSteps = 2;                     // steps held in LDS
    static constexpr int kAhead = kSteps - 1;            // steps copied ahead of the one in use
    static constexpr int kBytes = kSteps * kSub * kSlot;
};

template <int D>
__global__ __launch_bounds__(kR1Threads, 1) void walk1_rows_kernel(Params p) {
    using L = R1Lds<D>;
    constexpr int KS = D / 16;
    constexpr int NI = L::kSlot / (kR1Waves * 1024);  // 1 KB copies per wave per slot
    static_assert(NI >= 1 && L::kSlot == NI * kR1Waves * 1024, "a slot splits into 1 KB copies per wave");
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l32 = lane & 31, g = lane >> 5;
    const int hk = blockIdx.x % p.Hkv;
    const int rt = blockIdx.x / p.Hkv;
    const int split = blockIdx.y;
    const int rb = rt * kR1Waves + wave;
    const bool active = rb < p.RB;
    const int rowsHK = p.RB * 32;
    const int r = rb * 32 + l32;
    const int i = r / p.G, gh = r - (r / p.G) * p.G;
    const int h = hk * p.G + gh;
    const bool row_ok = active && r < p.R;
    const int ridx = hk * rowsHK + r;
    const int NS = (p.M + kSubKeys - 1) / kSubKeys;
    const int s_begin = 2 * split * p.w1_tps;
    const int s_end = min(NS, 2 * min(p.KT, (split + 1) * p.w1_tps));

    f16x8 bq[KS], bd[KS];
    if (active) {
        const _Float16* rq = p.qr + ((int64_t)hk * rowsHK + r) * D;
        const _Float16* rd = p.dr + ((int64_t)hk * rowsHK + r) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bq[ks] = *(const f16x8*)(rq + 16 * ks + 8 * g);
            bd[ks] = *(const f16x8*)(rd + 16 * ks + 8 * g);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < 8; ++t) bq[ks][t] = bd[ks][t] = (_Float16)0.0f;
    }
    const bool has_mask = p.m_type != FA_BACK_NONE;
    const char* mrow = (has_mask && row_ok)
        ? p.mask + (int64_t)i * p.m_nb1 + (int64_t)(p.Hm == 1 ? 0 : h) * p.m_nb2 : nullptr;
    // q rows carry the sign of the scale (prep), so the score scale is positive here
    const float sc2 = fabsf(p.scale) * ldexpf(1.0f, -p.scal[0]) * kLog2e;
    const bool full_rows = active && (rb + 1) * 32 <= p.R;
    const RowWalk<D> rw = make_row_walk<D>(lane);

    // step t covers image slots s_begin + kSub*t .. + kSub - 1 (those below s_end)
    const int nsteps = (s_end - s_begin + L::kSub - 1) / L::kSub;
    auto ring = [&](int t) { return lds + (t % L::kSteps) * (L::kSub * L::kSlot); };
    const unsigned char* img = p.kvimg + (int64_t)hk * p.img_ns * L::kSlot;
    // the copies are hidden from the compiler (dma16_hidden): they stay in flight across the
    // products, and the step barrier waits for them by count. Every step copies kSub slots, so
    // that the counts are the same for every step: past s_end the last slot is copied again.
    auto copy = [&](int t) {
#pragma unroll
        for (int u = 0; u < L::kSub; ++u) {
            const int sl = min(s_begin + L::kSub * t + u, s_end - 1);
            const unsigned char* src = img + (int64_t)sl * L::kSlot + wave * (NI * 1024);
            const uint32_t dst = lds_addr(ring(t) + u * L::kSlot) + (uint32_t)(wave * (NI * 1024));
#pragma unroll
            for (int it = 0; it < NI; ++it) dma16_hidden(src + it * 1024, 16u * lane, dst + it * 1024);
        }
    };
    constexpr int NS1 = L::kSub * NI;                 // copies per wave per step

    // All 8 waves form their products right after the step barrier and fold them right after.
    // (Measured and not kept: the two waves of a SIMD half a slot apart, and a slot's fold
    // spread over the next slot's product steps; both slower.)
    W1Row w1;
    w1_init(w1);
    wait_all_mem();   // the fragments are in registers before the first copy is queued
#pragma unroll
    for (int t = 0; t < L::kAhead; ++t)
        if (t < nsteps) copy(t);
    for (int t = 0; t < nsteps; ++t) {
        // step t has landed for every wave (the copies of later steps stay in flight); the
        // slots of step t-1, which step t+kAhead reuses, are read by no wave any more
        const int later = min(L::kAhead - 1, nsteps - 1 - t);
        if (later >= 2) dma_barrier<(L::kAhead >= 3 ? 2 : 0) * NS1>();
        else if (later == 1) dma_barrier<(L::kAhead >= 2 ? 1 : 0) * NS1>();
        else dma_barrier<0>();
        if (t + L::kAhead < nsteps) copy(t + L::kAhead);
#pragma unroll
        for (int u = 0; u < L::kSub; ++u) {
            const int s = s_begin + L::kSub * t + u;
            if (s >= s_end) break;
            // a scalar load: waiting for it leaves the copies in flight
            const int cls = active ? mask_class_s(p, hk, rb, s >> 1) : kMaskDead;
            if (cls == kMaskDead) continue;
            f32x16 sa, pa;
#pragma unroll
            for (int v = 0; v < 16; ++v) sa[v] = pa[v] = 0.0f;
            mfma_prio_hi();
            pair_rows<D, 2>(ring(t) + u * L::kSlot, bq, bd, sa, pa, rw);
            mfma_prio_lo();
            const int j0 = s * kSubKeys;
            const bool fast = full_rows && cls == kMaskZero && j0 + kSubKeys <= p.M;
            w1_fold(p, w1, sa, pa, fast, cls, row_ok, mrow, i, j0, g, sc2);
        }
    }
    wait_all_mem();   // no copy is left in flight when the wave ends
    if (active) w1_record(p, w1, split, ridx, g);
}

// ----------------------------------------------------------------------------- walk 1 by keys

// Walk 1 with the keys owned (used when the cache is long next to the rows): a workgroup takes
// one KV head, 256 keys (8 waves x 32 keys) and a range of 32-row blocks. The K and V fragments
// of a wave's keys are decoded once into its registers; per row block (q/dO rows DMA'd into
// LDS, double-buffered) each wave computes S^T = K Q^T and dP^T = V dO^T and, per query row over
// its 32 keys, the max m, l = sum exp2(s - m) and d' = sum exp2(s - m) dp (fp32) and max |dp|.
// One block later the 8 waves' values of a row are merged in wave order and written as the
// row's record for this 256-key tile; the merge kernel combines a row's records in tile
// order. Rows no key of the tile sees get an empty record.
constexpr int kW1Waves = 8;
constexpr int kW1Threads = kW1Waves * kWave;
constexpr int kW1Keys = kW1Waves * 32;

template <int D>
struct W1Lds {
    static constexpr int kBlk = 32 * D * 2;                              // bytes of a 32-row block
    static constexpr int kBuf = 2 * kBlk;                                // q, dO
    static constexpr int kRec = kW1Waves * 32 * 16;                      // [wave][row] {m, l, d, b}
    static constexpr int kWork = 2 * kBuf + 3 * kRec;
    static constexpr int kRaw = RawTile<D, kQTileKeys>::kBytes;
    static constexpr int kSetup = 2 * kQTileKeys * D * 2 + 4 * kRaw;     // K, V 64-key tiles + [2][K, V] bytes
    static constexpr int kMaxRB = 2048;                                  // row blocks per workgroup
    static constexpr int kTiles = kW1Keys / kQTileKeys;                  // 64-key class tiles
    static constexpr int kList = 4 * kMaxRB + 16;                        // needed blocks, count
    static constexpr int kBytes = (kSetup > kWork + kList ? kSetup : kWork + kList) + kTiles * kMaxRB;
};

template <int D>
__global__ __launch_bounds__(kW1Threads, 1) void walk1_keys_kernel(Params p) {
    using L = W1Lds<D>;
    constexpr int KS = D / 16;
    constexpr int NI = L::kBlk / 1024;                // 64-lane x 16-byte DMA instructions per tensor
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];
    unsigned char* work = lds;
    unsigned char* recs = work + 2 * L::kBuf;                         // [3][wave][row] x 16 B
    unsigned char* cls = lds + L::kBytes - L::kTiles * L::kMaxRB;     // [tile][row block - rb0]
    // the needed row blocks in order, entry = (rb - rb0) | class of 64-key tile t << (16 + 2t);
    // built after the setup, in its region past the row-block buffers and records
    uint32_t* list = (uint32_t*)(work + L::kWork);
    int* nlist = (int*)(list + L::kMaxRB);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l32 = lane & 31, g = lane >> 5;
    const int hk = blockIdx.x % p.Hkv;
    const int kt = blockIdx.x / p.Hkv;
    const int key0 = kt * kW1Keys;
    const int wkey0 = key0 + 32 * wave;
    const int mytile = wave / 2;                      // 64-key class tile of this wave
    const int rb0 = blockIdx.y * p.w1_rbs;
    const int rb1 = min(p.RB, rb0 + p.w1_rbs);
    const int nloc = rb1 > rb0 ? rb1 - rb0 : 0;
    const int rowsHK = p.RB * 32;
    const int64_t total = (int64_t)p.Hkv * rowsHK;
    const int64_t rec0 = (int64_t)kt * total + (int64_t)hk * rowsHK;   // record index of row 0

    // ---- setup: K and V fragments of the wave's 32 keys into registers (keys >= M are 0)
    f16x8 bk[KS], bv[KS];
    {
        _Float16* sK = (_Float16*)work;
        _Float16* sV = sK + kQTileKeys * D;
        unsigned char* raw0 = work + 2 * kQTileKeys * D * 2;          // [2][K, V] staged bytes
        auto rawK = [&](int qt) { return raw0 + ((qt & 1) * 2 + 0) * L::kRaw; };
        auto rawV = [&](int qt) { return raw0 + ((qt & 1) * 2 + 1) * L::kRaw; };
        auto stage = [&](int qt) {
            const int j0 = key0 + qt * kQTileKeys;
            if (is_block_type(p.k_type))
                dma_raw_tile<D, kQTileKeys, kW1Threads>(p.k, p.k_nb1, p.k_nb2, hk, j0, p.M,
                                                        block_row_bytes(p.k_type, D), rawK(qt), threadIdx.x);
            if (is_block_type(p.v_type))
                dma_raw_tile<D, kQTileKeys, kW1Threads>(p.v, p.v_nb1, p.v_nb2, hk, j0, p.M,
                                                        block_row_bytes(p.v_type, D), rawV(qt), threadIdx.x);
        };
        // the bytes of quarter qt+1 are on their way while quarter qt is decoded
        stage(0);
#pragma unroll 1
        for (int qt = 0; qt < L::kTiles; ++qt) {
            const int j0 = key0 + qt * kQTileKeys;
            wait_all_mem();
            __syncthreads();   // bytes of qt landed; the decoded tiles of qt-1 are read
            if (qt + 1 < L::kTiles) stage(qt + 1);
            decode_tile<D, kQTileKeys, kW1Threads>(p.k, p.k_type, p.k_nb1, p.k_nb2, hk, j0, p.M, rawK(qt), sK,
                                                   threadIdx.x, p.kcen ? p.kcen + (int64_t)hk * D : nullptr);
            decode_tile<D, kQTileKeys, kW1Threads>(p.v, p.v_type, p.v_nb1, p.v_nb2, hk, j0, p.M, rawV(qt), sV,
                                                   threadIdx.x, p.vcen ? p.vcen + (int64_t)hk * D : nullptr);
            __syncthreads();
            if (mytile == qt) {
                const Swz z = make_swz<D>(lane);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    bk[ks] = frag_rows<D>(sK, 32 * (wave & 1), ks, lane, z);
                    bv[ks] = frag_rows<D>(sV, 32 * (wave & 1), ks, lane, z);
                }
            }
        }
        wait_all_mem();
        __syncthreads();
        // mask classes of (row block, 64-key tile) for the workgroup's row blocks and tiles
        for (int idx = threadIdx.x; idx < L::kTiles * nloc; idx += kW1Threads) {
            const int t = idx / nloc, lr = idx - (idx / nloc) * nloc;
            const int tile = key0 / kQTileKeys + t;
            cls[t * L::kMaxRB + lr] = (unsigned char)(tile < p.KT ? mask_class(p, hk, rb0 + lr, tile) : kMaskDead);
        }
        __syncthreads();   // the setup region becomes the row-block buffers
    }
    auto tcls = [&](int rbx, int t) -> int { return cls[t * L::kMaxRB + (rbx - rb0)]; };
    auto needed = [&](int rbx) -> bool {
#pragma unroll
        for (int t = 0; t < L::kTiles; ++t)
            if (tcls(rbx, t) != kMaskDead) return true;
        return false;
    };
    // empty records for the rows of blocks no key of this tile sees
    for (int idx = threadIdx.x; idx < 32 * nloc; idx += kW1Threads) {
        const int rbx = rb0 + idx / 32;
        if (needed(rbx)) continue;
        p.part_rec[rec0 + (int64_t)rb0 * 32 + idx] = f32x4{neg_inf(), 0.0f, 0.0f, 0.0f};
    }

    if (wave == 0) {
        int cnt = 0;
        for (int b0 = 0; b0 < nloc; b0 += 64) {
            const int lr = b0 + lane;
            uint32_t code = (uint32_t)lr;
            bool need = false;
            if (lr < nloc) {
#pragma unroll
                for (int t = 0; t < L::kTiles; ++t) {
                    const uint32_t c = cls[t * L::kMaxRB + lr];
                    code |= c << (16 + 2 * t);
                    need = need || c != (uint32_t)kMaskDead;
                }
            }
            const unsigned long long m = __ballot(need);
            if (need) list[cnt + __popcll(m & ((1ull << lane) - 1ull))] = code;
            cnt += __popcll(m);
        }
        if (lane == 0) *nlist = cnt;
    }
    __syncthreads();
    const int n = __builtin_amdgcn_readfirstlane(*nlist);

    const char* qbase = (const char*)(p.qr + (int64_t)hk * rowsHK * D);
    const char* dbase = (const char*)(p.dr + (int64_t)hk * rowsHK * D);
    // nw waves issue it; wi is this wave's index among them (both uniform)
    auto dma_block = [&](int rbx, int b, int nw, int wi) {
        unsigned char* base = work + b * L::kBuf;
        const int64_t blk = (int64_t)rbx * L::kBlk;
#pragma unroll
        for (int k = 0; k < 2 * NI; ++k) {
            const int ins = wi + nw * k;     // uniform
            if (ins >= 2 * NI) break;
            const int ten = ins / NI, ii = ins - (ins / NI) * NI;
            const int P = ii * 64 + lane;
            const int row = P / (D / 8), pc = P - (P / (D / 8)) * (D / 8);
            const int off = (row * D + 8 * swz_chunk<D>(row, pc)) * 2;
            dma16((ten ? dbase : qbase) + blk + off, base + ten * L::kBlk + ii * 1024);
        }
    };
    // The same copy by the late waves (wl = 0 .. 3 among them) in the loop. Instruction
    // ins = wl + 4k moves 1 KB piece ii = ins % NI of tensor ins / NI; the swizzle repeats every
    // IP = D/32 pieces, so a lane's source offset is that of ii % IP, one of the two computed
    // here once, and the rest of the address is a uniform 16-row step on the base. The copies
    // are hidden from the compiler (dma16_hidden); the block barrier waits for them.
    constexpr int IP = D / 32;
    const int wl = (wave - kW1Waves / 2) & 3;
    uint32_t doff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int P = ((wl + 4 * h) % IP) * 64 + lane;
        const int row = P / (D / 8), pc = P - (P / (D / 8)) * (D / 8);
        doff[h] = (uint32_t)((row * D + 8 * swz_chunk<D>(row, pc)) * 2);
    }
    auto dma_block_late = [&](int rbx, int b) {
        const uint32_t base = lds_addr(work + b * L::kBuf);
        const int64_t blk = (int64_t)rbx * L::kBlk;
#pragma unroll
        for (int k = 0; k < 2 * NI / 4; ++k) {
            const int ins = wl + 4 * k;     // uniform
            const int ten = ins / NI, ii = ins - (ins / NI) * NI;
            const char* sb = (ten ? dbase : qbase) + blk + (int64_t)(ii / IP) * (16 * D * 2);
            dma16_hidden(sb, doff[IP > 4 ? (k & 1) : 0], base + ten * L::kBlk + ii * 1024);
        }
    };
    // the 8 records of a row of a finished block are merged in wave order; waves 0..3 (which
    // finish their products first) take 8 rows each, one per lane
    auto merge_block = [&](int rbx, const unsigned char* rec, int l32) {
        const f32x4* rr = (const f32x4*)rec;
        float mx = neg_inf(), bb = 0.0f;
#pragma unroll
        for (int w = 0; w < kW1Waves; ++w) {
            const f32x4 x = rr[w * 32 + l32];
            mx = fmaxf(mx, x[0]);
            bb = fmaxf(bb, x[3]);
        }
        // eight partial sums of 32 keys each: combined in fp32 (the row's records of all key
        // tiles are combined in fp64 by the merge kernel)
        float ls = 0.0f, ds = 0.0f;
        if (mx != neg_inf()) {
#pragma unroll
            for (int w = 0; w < kW1Waves; ++w) {
                const f32x4 x = rr[w * 32 + l32];
                const float f = x[0] == neg_inf() ? 0.0f : fast_exp2(x[0] - mx);   // 1 at the max
                ls = fmaf(x[1], f, ls);
                ds = fmaf(x[2], f, ds);
            }
        }
        p.part_rec[rec0 + (int64_t)rbx * 32 + l32] = f32x4{mx, ls, ds, bb};
    };

    const float sc2 = fabsf(p.scale) * ldexpf(1.0f, -p.scal[0]) * kLog2e;   // q carries the sign
    const bool has_mask = p.m_type != FA_BACK_NONE;
    const RowWalk<D> rw = make_row_walk<D>(lane);

    // statistics of one row block from its S^T (sa) and dP^T (pa) over this wave's 32 keys when a
    // mask or a ragged edge is involved
    auto stats_slow = [&](int rbx, int c, const f32x16& sa, const f32x16& pa) -> f32x4 {
        float m = neg_inf(), l = 0.0f, d = 0.0f, b = 0.0f;
        const int r = 32 * rbx + l32;
        const bool row_ok = r < p.R;
        const char* mrow = nullptr;
        const int i = r / p.G;
        const bool use_mask = has_mask && row_ok && c == kMaskMixed;
        if (use_mask) {
            const int gh = r - (r / p.G) * p.G;
            mrow = p.mask + (int64_t)i * p.m_nb1 + (int64_t)(p.Hm == 1 ? 0 : hk * p.G + gh) * p.m_nb2;
        }
        float madd[16];
        float tm = neg_inf();
        const int kbase = opaque(wkey0);   // keeps per-key offsets out of the loop preheader
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = kbase + crow(v, g);
            float mv = 0.0f;
            if (!row_ok || key >= p.M) mv = neg_inf();
            else if (use_mask) mv = mask_value(p, mrow, i, key) * kLog2e;
            madd[v] = mv;
            if (mv != neg_inf()) tm = fmaxf(tm, fmaf(sa[v], sc2, mv));
        }
        m = max_halves(tm);
        if (m != neg_inf()) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (madd[v] == neg_inf()) continue;
                const float e = fast_exp2(fmaf(sa[v], sc2, madd[v] - m));
                l += e;
                d = fmaf(e, pa[v], d);
                b = fmaxf(b, fabsf(pa[v]));
            }
        }
        l = sum_halves(l);
        d = sum_halves(d);
        b = max_halves(b);
        return f32x4{m, l, d, b};
    };
    auto fast_ok = [&](int rbx, int c) { return c == kMaskZero && wkey0 + 32 <= p.M && (rbx + 1) * 32 <= p.R; };

    // the same statistics without products to overlap (last block, or the next one is dead)
    auto stats_fast = [&](const f32x16& sa, const f32x16& pa) -> f32x4 {
        float tm = neg_inf(), l = 0.0f, d = 0.0f, b = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) tm = fmaxf(tm, sa[v]);
        const float m = max_halves(tm) * sc2;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float e = fast_exp2(fmaf(sa[v], sc2, -m));
            l += e;
            d = fmaf(e, pa[v], d);
            b = fmaxf(b, fabsf(pa[v]));
        }
        l = sum_halves(l);
        d = sum_halves(d);
        b = max_halves(b);
        return f32x4{m, l, d, b};
    };
    auto put_rec = [&](int bufx, const f32x4& rec) {
        if (g == 0) *(f32x4*)(recs + bufx * L::kRec + (wave * 32 + l32) * 16) = rec;
    };
    auto stats = [&](int rbx, int c, const f32x16& sa, const f32x16& pa) -> f32x4 {
        if (c == kMaskDead) return f32x4{neg_inf(), 0.0f, 0.0f, 0.0f};
        return fast_ok(rbx, c) ? stats_fast(sa, pa) : stats_slow(rbx, c, sa, pa);
    };

    // Iteration i takes the needed blocks c0 = b_i and cp = b_(i-1). On each SIMD the two waves
    // run half an iteration apart: a late wave (4..7) forms the products of c0 and then their
    // statistics; an early wave (0..3) first forms the statistics of cp from the products it
    // kept in registers (and merges the records of b_(i-2)), then the products of c0. So one
    // wave's exponentials overlap the other's matrix products. The DMA of b_(i+1) goes into the
    // buffer of cp, which no wave reads any more; the records of block b sit in buffer b%3.
    const bool early = wave < kW1Waves / 2;
    auto eblock = [&](uint32_t e) { return rb0 + (int)(e & 0xffffu); };
    auto eclass = [&](uint32_t e) { return (int)(e >> (16 + 2 * mytile)) & 3; };
    const uint32_t e0 = n > 0 ? __builtin_amdgcn_readfirstlane(list[0]) : 0u;
    int c0 = n > 0 ? eblock(e0) : -1;
    int k0 = n > 0 ? eclass(e0) : kMaskDead;   // this wave's class of c0
    if (c0 >= 0) dma_block(c0, 0, kW1Waves, wave);
    int cp = -1, cpp = -1, kp = kMaskDead;
    f32x16 ha, hp;   // early waves: products of cp
#pragma unroll
    for (int v = 0; v < 16; ++v) ha[v] = hp[v] = 0.0f;
    for (int i = 0;; ++i) {
        wait_all_mem();
        __syncthreads();   // c0 landed; the records of cpp are complete
        // the list entry of the next block: read by the early waves under their statistics, by
        // the late waves after their products (not held across the products)
        const int inext = i + 1 < n ? i + 1 : 0;
        uint32_t e1 = 0;
        if (early) {
            const uint32_t e1v = list[inext];
            if (cp >= 0) put_rec((i + 2) % 3, stats(cp, kp, ha, hp));
            if (cpp >= 0 && lane < 8) merge_block(cpp, recs + ((i + 1) % 3) * L::kRec, 8 * wave + lane);
            e1 = __builtin_amdgcn_readfirstlane(e1v);
        }
        if (c0 < 0 && cp < 0) break;
        int c1 = -1, k1 = kMaskDead;
        if (c0 >= 0) {
            const int c = k0;
            // the products of a block that is dead for this wave's keys are formed too (stats
            // gives it the empty record): no zero fill, and no copy of the early waves' products
            f32x16 sa, pa;
            mfma_prio_hi();
            pair_rows_t<D, 2, L::kBlk, true>(work + (i & 1) * L::kBuf, bk, bv, sa, pa, rw);
            mfma_prio_lo();
            if (!early) e1 = __builtin_amdgcn_readfirstlane(list[inext]);
            if (i + 1 < n) {
                c1 = eblock(e1);
                k1 = eclass(e1);
            }
            // the next block's DMA is queued by the late waves after their products (queued by
            // all waves at the barrier, the later ones stall behind the earlier ones' copies)
            if (c1 >= 0 && !early) dma_block_late(c1, (i + 1) & 1);
            if (early) {
                ha = sa;
                hp = pa;
            } else {
                put_rec(i % 3, stats(c0, c, sa, pa));
            }
        }
        cpp = cp;
        cp = c0;
        kp = k0;
        c0 = c1;
        k0 = k1;
    }
}

// ----------------------------------------------------------------------------- merge

// Merge of the walk-1 records of every row (one record per key-range split or key tile), then
// LSE, delta and the row's dS exponent. Grid (blocks, Hkv): a block takes 64 consecutive rows of
// one KV head at a time; wave w takes records w, w+4, ... of each row (16-byte loads coalesced
// across the rows), and the four partial results meet in LDS in wave order. Each block also
// leaves max(max|dp| + |delta|) over its rows in bound_part[hk][block], for the head's exponent.
constexpr int kMergeRows = 64;
constexpr int kMergeMaxBlocks = 1024;   // blocks per KV head

__global__ __launch_bounds__(kThreads) void merge_kernel(Params p) {
    __shared__ float smax[kWaves][kMergeRows];
    __shared__ double sl[kWaves][kMergeRows], sd[kWaves][kMergeRows];
    __shared__ float sb[kWaves][kMergeRows];
    const int rowsHK = p.RB * 32;
    const int64_t total = (int64_t)p.Hkv * rowsHK;
    const int hk = blockIdx.y;
    const int lr = threadIdx.x & 63, grp = threadIdx.x >> 6;
    float bound = 0.0f;
    for (int base = blockIdx.x * kMergeRows; base < rowsHK; base += gridDim.x * kMergeRows) {
        const int r = base + lr;
        const int64_t ridx = (int64_t)hk * rowsHK + r;
        const bool ok = r < rowsHK;
        float mx = neg_inf();
        if (ok) {
#pragma unroll 8
            for (int s = grp; s < p.nparts; s += kWaves) mx = fmaxf(mx, p.part_rec[s * total + ridx][0]);
        }
        smax[grp][lr] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(smax[0][lr], smax[1][lr]), fmaxf(smax[2][lr], smax[3][lr]));
        double Ls = 0.0, Ds = 0.0;
        float b = 0.0f;
        if (ok && mx != neg_inf()) {
#pragma unroll 4
            for (int s = grp; s < p.nparts; s += kWaves) {
                const f32x4 rec = p.part_rec[s * total + ridx];
                b = fmaxf(b, rec[3]);
                if (rec[0] != neg_inf()) {
                    const double f = (double)fast_exp2(rec[0] - mx);   // 1 for the record holding the max
                    Ls = fma((double)rec[1], f, Ls);
                    Ds = fma((double)rec[2], f, Ds);
                }
            }
        }
        sl[grp][lr] = Ls;
        sd[grp][lr] = Ds;
        sb[grp][lr] = b;
        __syncthreads();
        if (grp == 0 && ok) {
            float lse2 = pos_inf();   // dead or padding row
            double dl = 0.0, lnat = 0.0;
            int ks = 0;
            if (mx != neg_inf()) {
                const double L = ((sl[0][lr] + sl[1][lr]) + sl[2][lr]) + sl[3][lr];
                const double Dd = ((sd[0][lr] + sd[1][lr]) + sd[2][lr]) + sd[3][lr];
                const double l2 = (double)mx + log2(L);
                lse2 = (float)(l2 - kPScaleLog2);   // stored less the P image exponent
                lnat = l2 * kLn2;
                dl = Dd / L;
                const float br = fmaxf(fmaxf(sb[0][lr], sb[1][lr]), fmaxf(sb[2][lr], sb[3][lr])) + fabsf((float)dl);
                ks = ds_exponent(br);
                bound = fmaxf(bound, br);
            }
            p.row_lse2[ridx] = lse2;
            p.row_dlt[ridx] = (float)dl;
            p.row_ks[ridx] = ks;
            if (r < p.R) {
                const int i = r / p.G, g = r - (r / p.G) * p.G;
                const int h = hk * p.G + g;
                p.lse[(int64_t)h * p.N + i] = (mx == neg_inf()) ? neg_inf() : (float)lnat;
                p.delta[(int64_t)h * p.N + i] = (float)ldexp(dl, -p.scal[1]);
            }
        }
        __syncthreads();   // the LDS rows are reused by the next chunk
    }
    if (grp != 0) return;
    bound = wave_max(bound);
    if (lr == 0) p.bound_part[hk * gridDim.x + blockIdx.x] = bound;
}

// ----------------------------------------------------------------------------- saved statistics

// With the forward's LSE and O supplied (fa_back_run_saved), the row statistics come from them
// instead of from walk 1 and the merge. delta = rowsum(dO o O) is the definition of delta the
// pages give ("The math in fattn_back_q": delta is rowsum(dO o O), computed there without O);
// the dS prescale needs a bound of |dp - delta| that walk 1 would have measured, taken here
// as sum_c |dO_c| * max |v| + |delta| (Hoelder), which holds for every key.

// Partial max |v| over the cache: for q8_0 / q4_0 the block scale times 128 / 8, otherwise
// every element (less the centre when V is centred). Grid-stride over V rows; partial per block.
static __global__ __launch_bounds__(kThreads) void vmax_kernel(Params p) {
    float vm = 0.0f;
    const int64_t rows = (int64_t)p.M * p.Hkv;
    if (is_block_type(p.v_type)) {
        // |d| times the largest |code| (128 for q8_0, 8 for q4_0, 15 for q4_1, 16 for q5_0,
        // 31 for q5_1), plus |m| for the types with a minimum
        const int bsz = block_bytes(p.v_type);
        const float qmax = p.v_type == FA_BACK_Q8_0 ? 128.0f : p.v_type == FA_BACK_Q4_0 ? 8.0f
                         : p.v_type == FA_BACK_Q4_1 ? 15.0f : p.v_type == FA_BACK_Q5_0 ? 16.0f : 31.0f;
        const bool has_m = p.v_type == FA_BACK_Q4_1 || p.v_type == FA_BACK_Q5_1;
        const int bpr = p.D / 32;
        const int64_t n = rows * bpr;
        for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads) {
            const int64_t row = e / bpr;
            const int b = (int)(e - row * bpr);
            const int hk = (int)(row / p.M), j = (int)(row - (int64_t)hk * p.M);
            const char* blk = p.v + (int64_t)hk * p.v_nb2 + (int64_t)j * p.v_nb1 + bsz * b;
            float bound = fabsf((float)*(const _Float16*)blk) * qmax;
            if (has_m) bound += fabsf((float)*(const _Float16*)(blk + 2));
            vm = fmaxf(vm, bound);
        }
    } else {
        const int64_t n = rows * p.D;
        const int es = p.v_type == FA_BACK_F32 ? 4 : 2;
        for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads) {
            const int64_t row = e / p.D;
            const int c = (int)(e - row * p.D);
            const int hk = (int)(row / p.M), j = (int)(row - (int64_t)hk * p.M);
            const float x = load_scalar(p.v + (int64_t)hk * p.v_nb2 + (int64_t)j * p.v_nb1 + (int64_t)c * es, p.v_type);
            vm = fmaxf(vm, fabsf(p.vcen ? x - p.vcen[(int64_t)hk * p.D + c] : x));
        }
    }
    __shared__ float red[kWaves];
    vm = wave_max(vm);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = vm;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0];
        for (int w = 1; w < kWaves; ++w) a = fmaxf(a, red[w]);
        p.vmax_part[blockIdx.x] = a;
    }
}

// Row statistics from the saved LSE and O, one wave per row (rows r = i*G + g of each KV head,
// padding rows past R included): the log2-LSE less the P image exponent (+inf for a fully
// masked or padding row), delta in the dO-scaled units of the products, the row's dS exponent,
// the LSE and delta outputs, and per block the max of the dS bound over its rows. Grid
// (blocks, Hkv), like the merge.
static __global__ __launch_bounds__(kThreads) void saved_rows_kernel(Params p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rowsHK = p.RB * 32;
    const int hk = blockIdx.y;
    const int edo = p.scal[1];
    float vmax = 0.0f;
    for (int t = lane; t < p.nvpart; t += 64) vmax = fmaxf(vmax, p.vmax_part[t]);
    vmax = wave_max(vmax) * 1.001f;   // the fp16 rounding of the products' V values
    float bound = 0.0f;
    for (int r = blockIdx.x * kWaves + wave; r < rowsHK; r += gridDim.x * kWaves) {
        const int64_t ridx = (int64_t)hk * rowsHK + r;
        float lse2 = pos_inf(), dlt = 0.0f;
        int ks = 0;
        if (r < p.R) {
            const int i = r / p.G, g = r - (r / p.G) * p.G;
            const int h = hk * p.G + g;
            const float lse = p.lse_in[(int64_t)h * p.N + i];
            double dl = 0.0, dc = 0.0;   // dO . O, and dO . (O - c) for the products' delta
            float l1 = 0.0f;
            if (lse != neg_inf()) {
                const float* orow = p.o_in + ((int64_t)h * p.N + i) * p.D;
                const float* cen = p.vcen ? p.vcen + (int64_t)hk * p.D : nullptr;
                for (int c = lane; c < p.D; c += 64) {
                    const float x = load_scalar(p.d + (int64_t)c * p.d_nb0 + (int64_t)h * p.d_nb1 + (int64_t)i * p.d_nb2,
                                                p.d_type);
                    dl = fma((double)x, (double)orow[c], dl);
                    dc = fma((double)x, (double)orow[c] - (cen ? (double)cen[c] : 0.0), dc);
                    l1 += fabsf(x);
                }
                // fixed-order wave sums
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    dl += __shfl_xor(dl, o);
                    dc += __shfl_xor(dc, o);
                    l1 += __shfl_xor(l1, o);
                }
                // with K centred, the products see the centred scores: their LSE is the given
                // one less scale * q . c
                const double lc = p.kcen ? (double)lse - (double)p.scale * q_dot_kcen(p, h, i, lane) : (double)lse;
                lse2 = (float)(lc * (1.0 / kLn2) - kPScaleLog2);
                dlt = (float)ldexp(dc, edo);
                const float br = ldexpf(l1, edo) * vmax + fabsf(dlt);
                ks = ds_exponent(br);
                bound = fmaxf(bound, br);
            }
            if (lane == 0) {
                p.lse[(int64_t)h * p.N + i] = lse;
                p.delta[(int64_t)h * p.N + i] = (float)dl;
            }
        }
        if (lane == 0) {
            p.row_lse2[ridx] = lse2;
            p.row_dlt[ridx] = dlt;
            p.row_ks[ridx] = ks;
        }
    }
    __shared__ float red[kWaves];
    bound = wave_max(bound);
    if (lane == 0) red[wave] = bound;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0];
        for (int w = 1; w < kWaves; ++w) a = fmaxf(a, red[w]);
        p.bound_part[hk * gridDim.x + blockIdx.x] = a;
    }
}

// ----------------------------------------------------------------------------- dQ reduce

// ----------------------------------------------------------------------------- centred K and V

// The centre of each KV head's K or V columns (ISK: K): the fp64 mean of its first
// min(M, kCentreKeys) keys, summed in key order. Any constant would leave the results unchanged
// in exact arithmetic; one near the values keeps the difference small, so its fp16 rounding is
// small too. Grid: one block per KV head.
constexpr int kCentreKeys = 256;
template <bool ISK>
static __global__ __launch_bounds__(kThreads) void centre_kernel(Params p) {
    const int hk = blockIdx.x;
    const int n = p.M < kCentreKeys ? p.M : kCentreKeys;
    const int type = ISK ? p.k_type : p.v_type;
    const int es = type == FA_BACK_F32 ? 4 : 2;
    const char* th = (ISK ? p.k + (int64_t)hk * p.k_nb2 : p.v + (int64_t)hk * p.v_nb2);
    const int64_t nb1 = ISK ? p.k_nb1 : p.v_nb1;
    float* cen = ISK ? p.kcen : p.vcen;
    for (int c = threadIdx.x; c < p.D; c += kThreads) {
        double s = 0.0;
#pragma unroll 8
        for (int j = 0; j < n; ++j) s += (double)load_scalar(th + (int64_t)j * nb1 + (int64_t)c * es, type);
        cen[(int64_t)hk * p.D + c] = n ? (float)(s / n) : 0.0f;
    }
}

// The outputs of centred runs, one wave per row (h, i); rows whose LSE is -inf (fully masked)
// keep LSE = -inf and delta = 0.
//   V centred: the products give delta' = delta - dO . c; dO . c is added back.
//   K centred: the products give the LSE of the centred scores, lse - scale * q . c; the shift
//   is added back.
static __global__ __launch_bounds__(kThreads) void centre_out_kernel(Params p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t rows = (int64_t)p.H * p.N;
    for (int64_t r = (int64_t)blockIdx.x * kWaves + wave; r < rows; r += (int64_t)gridDim.x * kWaves) {
        const int h = (int)(r / p.N), i = (int)(r - (int64_t)h * p.N);
        if (p.lse[r] == neg_inf()) continue;   // wave-uniform
        if (p.vcen) {
            const float* cen = p.vcen + (int64_t)(h / p.G) * p.D;
            double s = 0.0;
            for (int c = lane; c < p.D; c += 64) {
                const float x = load_scalar(p.d + (int64_t)c * p.d_nb0 + (int64_t)h * p.d_nb1 + (int64_t)i * p.d_nb2,
                                            p.d_type);
                s = fma((double)x, (double)cen[c], s);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
            if (lane == 0) p.delta[r] = (float)((double)p.delta[r] + s);
        }
        if (p.kcen) {
            const double s = q_dot_kcen(p, h, i, lane);
            if (lane == 0) p.lse[r] = (float)((double)p.lse[r] + (double)p.scale * s);
        }
    }
}

// One lane per 16 bytes of output; launched with kDqThreads per block. The split partials are
// added in split order; their loads go out eight at a time.
constexpr int kDqThreads = 64;

template <int D>
__global__ __launch_bounds__(kDqThreads) void dqreduce_kernel(Params p) {
    const int rowsHK = p.RB * 32;
    const int64_t total = (int64_t)p.Hkv * rowsHK;
    const int64_t n4 = total * (D / 4);
    for (int64_t e = (int64_t)blockIdx.x * kDqThreads + threadIdx.x; e < n4; e += (int64_t)gridDim.x * kDqThreads) {
        const int64_t ridx = e / (D / 4);
        const int c4 = (int)(e - ridx * (D / 4));
        const int hk = (int)(ridx / rowsHK), r = (int)(ridx - (ridx / rowsHK) * rowsHK);
        if (r >= p.R) continue;
        const float* src = p.dq_part + ridx * D + 4 * c4;
        const int64_t step = total * D;
        f32x4 acc = *(const f32x4*)src;
        int s = 1;
        for (; s + 8 <= p.splits; s += 8) {
            f32x4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = *(const f32x4*)(src + (int64_t)(s + u) * step);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += x[u];
        }
        for (; s < p.splits; ++s) acc += *(const f32x4*)(src + (int64_t)s * step);
        const int i = r / p.G, g = r - (r / p.G) * p.G;
        const int h = hk * p.G + g;
        const float fac = p.scale * ldexpf(1.0f, p.row_ks[ridx] - p.scal[1]);   // the row's dS exponent
        *(f32x4*)(p.dq + ((int64_t)h * p.N + i) * D + 4 * c4) = acc * fac;
    }
}

// ----------------------------------------------------------------------------- dQ from stored dS

// dQ = scale dS K from the dS tiles the key side stored (Params::dsbuf), instead of walk 2's
// recomputation of S and dP. A workgroup takes one KV head, 8 row blocks of 32 rows (one per
// wave, its dQ accumulators in registers) and a key range. Per step of two 32-key sub-tiles the
// 8 waves copy the two K tiles from the image into LDS (an eighth each) and every wave copies
// its own row block's two dS tiles; after the step barrier each wave forms dQ^T += K^T dS^T
// with both operands read from LDS by transpose reads: K^T as walk 2 reads it, dS^T from the
// tile as the key side's registers held it (lane = key, 16 rows), so that each lane gets its
// row's 8 keys in the order of the K^T operand. The next step is copied during this one.

// Position of lane l's 16 bytes in half hh of a stored dS tile: lanes 32..63 rotated by 4 and
// the second half by 8, so that the dQ pass's transpose reads of a tile meet no bank twice.
FAB_DEV int ds_pos(int hh, int l) {
    const int p0 = l < 32 ? l : 32 + ((l - 28) & 31);
    return (8 * hh + p0) & 63;
}

constexpr int kQsWaves = 8;
constexpr int kQsThreads = kQsWaves * kWave;

template <int D>
struct QsLds {
    static constexpr int kKTile = kSubKeys * D * 2;           // a K sub-tile: the first half of an image slot
    static constexpr int kSlot = 2 * kKTile;                  // an image slot
    static constexpr int kDsTile = 2048;                      // a stored 32 x 32 dS tile
    static constexpr int kSub = 2;                            // sub-tiles per step
    static constexpr int kStepK = kSub * kKTile;
    static constexpr int kStepDs = kQsWaves * kSub * kDsTile;
    static constexpr int kSteps = 2;
    static constexpr int kBytes = kSteps * (kStepK + kStepDs);
};

// The B operand dS^T of one 16-key step (keys kstep*16 ..) of the stored tile at t: lane l gets
// row l%32 and the keys 16*kstep + crow(j, l/32), j = 0..7, from two transpose reads. In each
// 16-lane group, lane 4a+b takes element b of the 8-byte reads of lanes a, a+4, a+8, a+12: so
// reading lane r = a' + 4i reads key k0 + i of the rows 4a'..4a'+3 of its group's half, where
// the row n of the stored layout sits in half n/16, lane-half (n/4)%2, elements 4((n/8)%2) ...
FAB_DEV f16x8 ds_frag(const unsigned char* t, int kstep, int lane) {
    const int q16 = lane >> 4, r = lane & 15, a = r & 3, i = r >> 2;
    const int hh = q16 & 1, g = q16 >> 1;
    f16x8 out;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int k0 = 16 * kstep + 8 * jj + 4 * g;
        const unsigned char* pa = t + hh * 1024 + 16 * ds_pos(hh, k0 + i + 32 * (a & 1)) + 8 * (a >> 1);
        const f16x4 h = tr_read(pa);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * jj + e] = h[e];
    }
    return out;
}

template <int D>
__global__ __launch_bounds__(kQsThreads, 1) void dq_stored_kernel(Params p) {
    using L = QsLds<D>;
    constexpr int MD = D / 32;
    constexpr int NKW = L::kStepK / (kQsWaves * 1024);       // K copies per wave per step
    static_assert(NKW >= 1 && L::kStepK == NKW * kQsWaves * 1024, "a step's K tiles split into 1 KB copies per wave");
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l32 = lane & 31, g = lane >> 5;
    const int hk = blockIdx.x % p.Hkv;
    const int rt = blockIdx.x / p.Hkv;
    const int split = blockIdx.y;
    const int rb = rt * kQsWaves + wave;
    const bool active = rb < p.RB;
    const int rbc = active ? rb : p.RB - 1;                   // an existing row block's tiles for the idle copies
    const int rowsHK = p.RB * 32;
    const int r = rb * 32 + l32;
    const int i = r / p.G, gh = r - (r / p.G) * p.G;
    const int h = hk * p.G + gh;
    const bool row_ok = active && r < p.R;
    const int ridx = hk * rowsHK + r;
    const int NS = (p.M + kSubKeys - 1) / kSubKeys;
    const int s_begin = 2 * split * p.tiles_per_split;
    const int s_end = min(NS, 2 * min(p.KT, (split + 1) * p.tiles_per_split));
    const int nsteps = (s_end - s_begin + L::kSub - 1) / L::kSub;

    auto ringK = [&](int t) { return lds + (t % L::kSteps) * (L::kStepK + L::kStepDs); };
    auto ringDs = [&](int t) { return ringK(t) + L::kStepK + wave * (L::kSub * L::kDsTile); };
    const unsigned char* img = p.kvimg + (int64_t)hk * p.img_ns * L::kSlot;
    const unsigned char* dsb = (const unsigned char*)p.dsbuf + ((int64_t)hk * p.RB + rbc) * p.ds_kb * L::kDsTile;
    // copies hidden from the compiler (dma16_hidden), waited for by count at the step barrier;
    // the same number in every step (past s_end the last sub-tile again)
    auto copy = [&](int t) {
#pragma unroll
        for (int c = 0; c < NKW; ++c) {
            const int piece = wave + kQsWaves * c;                    // 1 KB piece of the step's K tiles
            const int u = piece / (L::kKTile / 1024), o = piece - u * (L::kKTile / 1024);
            const int sl = min(s_begin + L::kSub * t + u, s_end - 1);
            dma16_hidden(img + (int64_t)sl * L::kSlot + o * 1024, 16u * lane,
                         lds_addr(ringK(t)) + (uint32_t)(u * L::kKTile + o * 1024));
        }
#pragma unroll
        for (int u = 0; u < L::kSub; ++u) {
            const int sl = min(s_begin + L::kSub * t + u, s_end - 1);
#pragma unroll
            for (int o = 0; o < L::kDsTile / 1024; ++o)
                dma16_hidden(dsb + (int64_t)sl * L::kDsTile + o * 1024, 16u * lane,
                             lds_addr(ringDs(t)) + (uint32_t)(u * L::kDsTile + o * 1024));
        }
    };

    f32x16 dqacc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) dqacc[md][v] = 0.0f;
    const ColWalk<D> cw = make_col_walk<D>(lane);

    if (nsteps > 0) copy(0);
    for (int t = 0; t < nsteps; ++t) {
        // step t has landed for every wave; the slots of step t-1, which step t+1 reuses, are
        // read by no wave any more
        dma_barrier<0>();
        if (t + 1 < nsteps) copy(t + 1);
#pragma unroll
        for (int u = 0; u < L::kSub; ++u) {
            const int s = s_begin + L::kSub * t + u;
            if (s >= s_end) break;
            // a scalar load: waiting for it leaves the copies in flight
            const int cls = active ? mask_class_s(p, hk, rb, s >> 1) : kMaskDead;
            if (cls == kMaskDead) continue;
            const unsigned char* dt = ringDs(t) + u * L::kDsTile;
            const f16x8 bb[2] = {ds_frag(dt, 0, lane), ds_frag(dt, 1, lane)};
            mfma_prio_hi();
            cols_acc<D>(ringK(t) + u * L::kKTile, bb, dqacc, cw);
            mfma_prio_lo();
        }
    }
    wait_all_mem();   // no copy is left in flight when the wave ends
    // the key side's dS carries the head's exponent (a reduction over the wave: every lane takes
    // part, before the branch on the lane's row)
    const int ksx = head_ds_exponent(p, hk);
    if (row_ok) {
        // a split's partial is taken to the row's exponent, which the reduction applies (an exact
        // power-of-two factor)
        const bool direct = p.splits == 1;
        const float fac = direct ? p.scale * ldexpf(1.0f, ksx - p.scal[1]) : ldexpf(1.0f, ksx - p.row_ks[ridx]);
        float* dst = direct ? p.dq + ((int64_t)h * p.N + i) * D
                            : p.dq_part + ((int64_t)split * p.Hkv * rowsHK + ridx) * D;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f32x4 o = {dqacc[md][4 * b] * fac, dqacc[md][4 * b + 1] * fac,
                           dqacc[md][4 * b + 2] * fac, dqacc[md][4 * b + 3] * fac};
                *(f32x4*)(dst + 32 * md + 8 * b + 4 * g) = o;
            }
    }
}

// ----------------------------------------------------------------------------- key side

// Workgroup: one KV head, 128 keys in 4 blocks of 32, and 8 waves: one pair per key block kb,
// both waves of a pair on the same SIMD.
//   X wave (w = kb)      K fragments of its 32 keys in registers. Per 32-row block: S = Q K^T,
//                        P = exp(S - lse) in fp32 (its image p*2^15 goes to LDS in fp32 for the
//                        Y wave), then dV^T += dO^T P from its own fp16 image.
//   Y wave (w = 4 + kb)  V fragments in registers. Per row block: dK^T += Q^T dS of the previous
//                        block (its dS kept in registers, its q rows still in their buffer),
//                        dP = dO V^T (kept in registers across the mid-block barrier); then,
//                        with P from the X wave, dS = P (dP - delta) in fp32.
// Two barriers per row block. Neither wave waits for the other's products: the X wave's
// exponentials run beside the Y wave's dK and dP products, the Y wave's dS arithmetic beside
// the X wave's dV products. The q and dO row blocks (fp16, row-major, with their lse/delta) are
// copied HBM -> LDS by DMA once per workgroup through three buffers, each two blocks ahead.
// Every wave stays within 256 registers.
// S = Q K^T puts one key per lane column and 16 rows per lane: the layout of the second
// operand of the dK/dV products, whose first operands are transpose reads of the row blocks.
// With DSOUT the Y waves also store each block's dS tile (fp16, as their registers hold it) for
// the dQ pass from stored dS.
constexpr int kKVWaves = 8;
constexpr int kKVThreads = kKVWaves * kWave;

template <int D>
struct KVLds {
    static constexpr int kBlk = 32 * D * 2;                              // bytes of a 32-row block
    static constexpr int kBuf = 2 * kBlk + 256;                          // q, dO, 32 lse, 32 delta
    static constexpr int kExF = 4 * 4096;                                // [kb][4][lane] P image, fp32
    static constexpr int kWork = 3 * kBuf + kExF;
    static constexpr int kRaw = RawTile<D, kQTileKeys>::kBytes;
    static constexpr int kSetup = 2 * kQTileKeys * D * 2 + 2 * kRaw;     // K, V half tiles + bytes
    static constexpr int kMaxRB = 2048;                                  // row blocks listed per workgroup
    static constexpr int kTail = 6 * kMaxRB + 16;                        // list, two class rows, count
    static constexpr int kBytes = (kSetup > kWork ? kSetup : kWork) + kTail;
};

template <int D, bool DSOUT>
__global__ __launch_bounds__(kKVThreads, 1) void kvpass_kernel(Params p) {
    using L = KVLds<D>;
    constexpr int KS = D / 16;
    constexpr int MD = D / 32;
    constexpr int NI = L::kBlk / 1024;                // 64-lane x 16-byte DMA instructions per tensor
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];
    unsigned char* work = lds;                        // setup scratch, then buffers + exchange
    unsigned char* exF = work + 3 * L::kBuf;             // P images from the X to the Y waves
    uint32_t* sched = (uint32_t*)(lds + L::kBytes - L::kTail);          // needed row blocks of a chunk
    unsigned char* clsA = (unsigned char*)(sched + L::kMaxRB);         // class of (row block, first 64 keys)
    unsigned char* clsB = clsA + L::kMaxRB;                             // class of (row block, last 64 keys)
    int* nsched = (int*)(clsB + L::kMaxRB);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l32 = lane & 31, g = lane >> 5;
    const int role = wave >> 2, kb = wave & 3;        // role 0: A (S, dK), role 1: B (dP, dV)
    // tile and row range: the tiles of the last, partial round of workgroups are split by rows
    const int wg = blockIdx.x;
    const bool split = wg >= p.kv_full;
    const int tile = split ? p.kv_full + (wg - p.kv_full) / p.kv_split : wg;
    const int part = split ? (wg - p.kv_full) % p.kv_split : 0;
    const int nsplit = split ? p.kv_split : 1;
    const int rb_lo = (int)((int64_t)p.RB * part / nsplit);
    const int rb_hi = (int)((int64_t)p.RB * (part + 1) / nsplit);
    const int hk = tile % p.Hkv;
    const int kvt = tile / p.Hkv;
    const int key0 = kvt * kKVKeys;
    const int myj = key0 + 32 * kb + l32;
    const bool key_ok = myj < p.M;
    const int rowsHK = p.RB * 32;

    // ---- setup: K (A waves) or V (B waves) fragments of the wave's 32 keys into registers
    f16x8 bkv[KS];
    {
        _Float16* sK = (_Float16*)work;
        _Float16* sV = sK + kQTileKeys * D;
        unsigned char* rawK = work + 2 * kQTileKeys * D * 2;
        unsigned char* rawV = rawK + L::kRaw;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j0 = key0 + half * kQTileKeys;
            __syncthreads();
            if (is_block_type(p.k_type))
                dma_raw_tile<D, kQTileKeys, kKVThreads>(p.k, p.k_nb1, p.k_nb2, hk, j0, p.M,
                                                        block_row_bytes(p.k_type, D), rawK, threadIdx.x);
            if (is_block_type(p.v_type))
                dma_raw_tile<D, kQTileKeys, kKVThreads>(p.v, p.v_nb1, p.v_nb2, hk, j0, p.M,
                                                        block_row_bytes(p.v_type, D), rawV, threadIdx.x);
            wait_all_mem();
            __syncthreads();
            decode_tile<D, kQTileKeys, kKVThreads>(p.k, p.k_type, p.k_nb1, p.k_nb2, hk, j0, p.M, rawK, sK,
                                                   threadIdx.x, p.kcen ? p.kcen + (int64_t)hk * D : nullptr);
            decode_tile<D, kQTileKeys, kKVThreads>(p.v, p.v_type, p.v_nb1, p.v_nb2, hk, j0, p.M, rawV, sV,
                                                   threadIdx.x, p.vcen ? p.vcen + (int64_t)hk * D : nullptr);
            __syncthreads();
            if ((kb >> 1) == half) {
                const Swz z = make_swz<D>(lane);
                const _Float16* src = role == 0 ? sK : sV;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) bkv[ks] = frag_rows<D>(src, 32 * (kb & 1), ks, lane, z);
            }
        }
        __syncthreads();   // the setup region becomes the row-block buffers
    }

    // DMA of row block rbx (q, dO and their 32 lse / 32 delta values) into buffer b by all 8
    // waves. The LDS copy is swizzled by choosing each lane's source chunk; those choices are
    // the same for every block, so they are computed once.
    const char* qbase = (const char*)(p.qr + (int64_t)hk * rowsHK * D);
    const char* dbase = (const char*)(p.dr + (int64_t)hk * rowsHK * D);
    // nw waves issue it; wi is this wave's index among them (both uniform). The copies are
    // hidden from the compiler (dma16_hidden), so the transpose reads of the products do not
    // wait for them; every wave waits for its own copies before the block barrier.
    // Instruction ii covers rows 64*ii/(D/8) ..; the swizzle repeats every 16 rows, i.e. every
    // IP = D/32 instructions, so a lane's source offset is that of ii % IP plus a uniform
    // 16-row step added to the base.
    constexpr int IP = D / 32;
    auto dma_block = [&](int rbx, int b, int nw, int wi) {
        const uint32_t base = lds_addr(work + b * L::kBuf);
        const int64_t blk = (int64_t)rbx * L::kBlk;
        if (wi == nw - 1 && lane < 16) {
            // first in the batch: lanes 0-7 copy the 32 lse values, lanes 8-15 the 32 delta values
            const float* lb = p.row_lse2 + (int64_t)hk * rowsHK + rbx * 32;
            const float* db = p.row_dlt + (int64_t)hk * rowsHK + rbx * 32;
            if (lane < 8) dma16_hidden(lb, 16 * lane, base + 2 * L::kBlk);
            else dma16_hidden(db, 16 * (lane - 8), base + 2 * L::kBlk);
        }
#pragma unroll
        for (int k = 0; k < 2 * NI; ++k) {
            const int ins = wi + nw * k;             // uniform
            if (ins >= 2 * NI) break;
            const int ten = ins / NI, ii = ins - (ins / NI) * NI;
            const int i0 = ii % IP;
            const int P = i0 * 64 + lane;
            const int row = P / (D / 8), pc = P - (P / (D / 8)) * (D / 8);
            const uint32_t off = (uint32_t)((row * D + 8 * swz_chunk<D>(row, pc)) * 2);
            const char* sb = (ten ? dbase : qbase) + blk + (int64_t)(ii / IP) * (16 * D * 2);
            dma16_hidden(sb, off, base + ten * L::kBlk + ii * 1024);
        }
    };

    const int eq = p.scal[0], edo = p.scal[1];
    const int ksx = head_ds_exponent(p, hk);   // one dS exponent for every row of the head

    f32x16 acc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[md][v] = 0.0f;
    const RowWalkX rw0 = make_row_walk_x<D>(lane);
    const ColWalkX cw0 = make_col_walk_x<D>(lane);
    unsigned char* myF = exF + kb * 4096;             // the pair's P image in fp32 [4][lane] x 16 B

    // ---- the needed row blocks (those with a 64-key half not fully masked) are listed in order
    // in LDS with both classes, entry = (rb - rb_lo) | class(first 64 keys) << 24 |
    // class(last 64 keys) << 28, so that a wave finds its next block with one early LDS read
    // instead of searching the class rows before each barrier. The host splits the rows of a
    // tile so that no workgroup has more than kMaxRB row blocks (a longer range would be cut).
    {
    const int c0 = rb_lo;
    const int c1 = min(rb_hi, c0 + L::kMaxRB);
    for (int rbx = c0 + (int)threadIdx.x; rbx < c1; rbx += kKVThreads) {
        clsA[rbx - c0] = (unsigned char)mask_class(p, hk, rbx, 2 * kvt);
        clsB[rbx - c0] = (unsigned char)(2 * kvt + 1 < p.KT ? mask_class(p, hk, rbx, 2 * kvt + 1) : kMaskDead);
    }
    __syncthreads();
    if (wave == 0) {
        int cnt = 0;
        for (int b0 = c0; b0 < c1; b0 += 64) {
            const int rbx = b0 + lane;
            const uint32_t ca = rbx < c1 ? clsA[rbx - c0] : (uint32_t)kMaskDead;
            const uint32_t cb = rbx < c1 ? clsB[rbx - c0] : (uint32_t)kMaskDead;
            const bool need = ca != (uint32_t)kMaskDead || cb != (uint32_t)kMaskDead;
            const unsigned long long m = __ballot(need);
            if (need) sched[cnt + __popcll(m & ((1ull << lane) - 1ull))] = (uint32_t)(rbx - c0) | (ca << 24) | (cb << 28);
            cnt += __popcll(m);
        }
        if (lane == 0) *nsched = cnt;
    }
    __syncthreads();
    const int n = __builtin_amdgcn_readfirstlane(*nsched);
    if (n > 0) {
    uint32_t ent = __builtin_amdgcn_readfirstlane(sched[0]);
    // Row blocks go through three buffers, each copied two blocks ahead of its use. The A waves
    // copy block 0 and then wait for all of their copies at every block barrier. The B waves
    // copy block 1 and, in each iteration k, block k+2 (past the end of the list: block k
    // again, into the free buffer), so that at every block barrier exactly their newest batch,
    // D/32 instructions, stays in flight (the wave that also copies lse/delta issues 2 more,
    // first in its batch, so they are the ones waited for early).
    if (role == 0) dma_block(c0 + (int)(ent & 0xffffffu), 0, 4, kb);
    else if (n > 1) dma_block(c0 + (int)(__builtin_amdgcn_readfirstlane(sched[1]) & 0xffffffu), 1, 4, kb);

    if (role == 0) {
        // ================= X waves (K fragments): S, P, then dV += P^T dO with their own P
        const float sc2 = fabsf(p.scale) * ldexpf(1.0f, -eq) * kLog2e;   // q carries the sign
        int bi = 0;
        for (int k = 0; k < n; ++k) {
            const int rb = c0 + (int)(ent & 0xffffffu);
            const int cls = (int)(ent >> (24 + 4 * (kb >> 1))) & 0xf;
            dma_barrier<0>();   // X: block rb landed in buffer bi; the Y wave has read the last P
            const uint32_t nxt = sched[k + 1 < n ? k + 1 : k];   // next entry, used after the products
            const unsigned char* tq = work + bi * L::kBuf;
            // the walks pass through an opaque move here, so that the per-step offsets are formed
            // in the loop rather than hoisted out of it and held (the registers are short)
            ColWalkX cw;
            cw.base[0] = opaque(cw0.base[0]);
            cw.base[1] = opaque(cw0.base[1]);
            cw.ee[0] = opaque(cw0.ee[0]);
            cw.ee[1] = opaque(cw0.ee[1]);
            RowWalkX rw;
            rw.base = opaque(rw0.base);
            rw.c = opaque(rw0.c);
            const float* lrow = (const float*)(tq + 2 * L::kBlk);
            f16x8 bp[2];
            if (cls != kMaskDead) {
                f32x16 sa;
#pragma unroll
                for (int v = 0; v < 16; ++v) sa[v] = 0.0f;
                // the X waves' products keep the default priority, so the Y wave of the pair
                // (dK, dP and the dS arithmetic: the longer role) issues ahead of them
                rows_chain_x<D, 1>(tq, bkv, sa, rw);
                if (cls == kMaskMixed) {
                    // mask terms staged through the wave's fp32 P slot by a rolled loop, so the
                    // masked case costs the loop below no registers; a fully masked row (and every
                    // padding row past R, lse2 = +inf) reads no mask
#pragma unroll 1
                    for (int v = 0; v < 16; ++v) {
                        const int b = v >> 2, u = v & 3;
                        float mv = neg_inf();
                        if (key_ok && lrow[8 * b + 4 * g + u] != pos_inf()) {
                            const int r = 32 * rb + crow(v, g);
                            const int ii = r / p.G, gh = r - (r / p.G) * p.G;
                            const char* mrow = p.mask + (int64_t)ii * p.m_nb1 +
                                               (int64_t)(p.Hm == 1 ? 0 : hk * p.G + gh) * p.m_nb2;
                            mv = mask_value(p, mrow, ii, myj) * kLog2e;
                        }
                        ((float*)(myF + (b * 64 + lane) * 16))[u] = mv;
                    }
                }
                // the image p * 2^15 (the stored lse carries the 15): rounded to fp16 for the dV
                // products here, in fp32 to the Y wave for dS. 0 for a dead row (lse2 = +inf) or
                // a masked key. Without a mask, a key past M (zero K row) gets an image too: it
                // only reaches that key's own dK and dV columns, which are never written.
                auto image = [&](bool mixed) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const f32x4 l4 = *(const f32x4*)(lrow + 8 * b + 4 * g);
                        f32x4 m4 = {0.0f, 0.0f, 0.0f, 0.0f};
                        if (mixed) m4 = *(const f32x4*)(myF + (b * 64 + lane) * 16);
                        f32x4 p4;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int v = 4 * b + u;
                            p4[u] = fast_exp2(mixed ? fmaf(sa[v], sc2, m4[u] - l4[u]) : fmaf(sa[v], sc2, -l4[u]));
                            bp[v >> 3][v & 7] = (_Float16)p4[u];
                        }
                        *(f32x4*)(myF + (b * 64 + lane) * 16) = p4;
                    }
                };
                if (cls == kMaskMixed) image(true);
                else image(false);
            }
            lds_barrier();     // Y: P published for the Y wave (the copies in flight stay so)
            if (cls != kMaskDead) {
                cols_acc_pf<D>(tq + L::kBlk, bp, acc, cw);
            }
            ent = __builtin_amdgcn_readfirstlane(nxt);
            bi = bi == 2 ? 0 : bi + 1;
        }
    } else {
        // ================= Y waves (V fragments): dK of the previous block, dP, then dS
        // dS = P (dP - delta) 2^-ks = image (dP - delta) 2^(-ks-15); it is kept in registers for
        // the dK products of the next iteration, whose q rows stay in their buffer until then
        const float dsf = ldexpf(1.0f, -ksx - kPScaleLog2);
        int bi = 0, bprev = 0;
        bool live = false;    // the block in bprev needs its dK products (bs holds its dS)
        f16x8 bs[2];
        for (int k = 0; k < n; ++k) {
            const int rb = c0 + (int)(ent & 0xffffffu);
            const int cls = (int)(ent >> (24 + 4 * (kb >> 1))) & 0xf;
            // X: block rb landed; the copy of block k+1 stays in flight (and with DSOUT the two
            // dS stores issued after it)
            dma_barrier<D / 32 + (DSOUT ? 2 : 0)>();
            const uint32_t nxt = sched[k + 1 < n ? k + 1 : k];   // next entry, used after the products
            const unsigned char* tq = work + bi * L::kBuf;
            // the walks pass through an opaque move here, so that the per-step offsets are formed
            // in the loop rather than hoisted out of it and held (the registers are short)
            ColWalkX cw;
            cw.base[0] = opaque(cw0.base[0]);
            cw.base[1] = opaque(cw0.base[1]);
            cw.ee[0] = opaque(cw0.ee[0]);
            cw.ee[1] = opaque(cw0.ee[1]);
            RowWalkX rw;
            rw.base = opaque(rw0.base);
            rw.c = opaque(rw0.c);
            if (live) {
                mfma_prio_hi();
                cols_acc_x<D>(work + bprev * L::kBuf, bs, acc, cw);
                mfma_prio_lo();
            }
            // dP stays in registers across the barrier (0 for a dead block: its dS is formed
            // too, and then not used)
            f32x16 pa;
#pragma unroll
            for (int v = 0; v < 16; ++v) pa[v] = 0.0f;
            if (cls != kMaskDead) {
                mfma_prio_hi();
                rows_chain_x<D, 1>(tq + L::kBlk, bkv, pa, rw);
                mfma_prio_lo();
            }
            lds_barrier();     // Y: P of block rb published; the buffer of block k-1 is read
            // dS is formed for a dead block too (and then not used): assigned on every path, the
            // previous block's dS is dead once its products are issued
            live = cls != kMaskDead;
            {
                const float* drow = (const float*)(tq + 2 * L::kBlk) + 32;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const f32x4 p4 = *(const f32x4*)(myF + (b * 64 + lane) * 16);
                    const f32x4 d4 = *(const f32x4*)(drow + 8 * b + 4 * g);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int v = 4 * b + u;
                        bs[v >> 3][v & 7] = (_Float16)(p4[u] * (pa[v] - d4[u]) * dsf);
                    }
                }
            }
            // the copy of the block two ahead, into the buffer of block k-1 (past the end of the
            // list: block k again)
            dma_block(k + 2 < n ? c0 + (int)(__builtin_amdgcn_readfirstlane(sched[k + 2]) & 0xffffffu) : rb,
                      bi == 0 ? 2 : bi - 1, 4, kb);
            if constexpr (DSOUT) {
                // this block's dS for the dQ pass, as the registers hold it: two streaming stores
                // in every iteration (a dead block's tile is never read), after the copies, so the
                // copy wait above counts them. The lane offsets are formed here from an opaque lane
                // index rather than held across the loop (the registers are short). (Stored after
                // the next block barrier instead, beside the dK products, a walk offset spills
                // into the loop.)
                _Float16* t = p.dsbuf + ((((int64_t)hk * p.RB + rb) * p.ds_kb + 4 * kvt + kb) << 10);
                const int ol = opaque(lane);
                __builtin_nontemporal_store(bs[0], (f16x8*)(t + 8 * ds_pos(0, ol)));
                __builtin_nontemporal_store(bs[1], (f16x8*)(t + 512 + 8 * ds_pos(1, ol)));
            }
            bprev = bi;
            ent = __builtin_amdgcn_readfirstlane(nxt);
            bi = bi == 2 ? 0 : bi + 1;
        }
        if (live) {
            mfma_prio_hi();
            cols_acc_pf<D>(work + bprev * L::kBuf, bs, acc, cw0);
            mfma_prio_lo();
        }
    }
    } }   // rows listed
    wait_all_mem();   // no copy is left in flight when the wave ends
    __syncthreads();  // every wave is done with the row-block buffers: they stage the output
    // Output: a lane holds 16-byte pieces of its key's row, so a direct store instruction would
    // write 32 bytes of each of 32 rows. Each wave instead stages 8 of its 32 key rows at a time
    // (fp32, scaled, padded rows) in an LDS area of its own and writes them back one whole row
    // (D floats) per 64 lanes, so that every store instruction covers whole cache lines.
    const int outk = role == 0 ? 1 : 0;               // X waves hold dV, Y waves dK
    const float fac = outk == 0 ? fabsf(p.scale) * ldexpf(1.0f, ksx - eq - edo) : ldexpf(1.0f, -kPScaleLog2 - edo);
    float* dst0 = split ? p.kv_part + ((((int64_t)(tile - p.kv_full) * p.kv_split + part) * 2 + outk) * kKVKeys +
                                       32 * kb) * D
                        : (outk == 0 ? p.dk : p.dv) + ((int64_t)hk * p.M + key0 + 32 * kb) * D;
    constexpr int kRowB = D * 4 + 16;                 // staged row bytes (padded)
    constexpr int kPass = 8;                          // rows per pass
    static_assert(kKVWaves * kPass * kRowB <= L::kWork, "staging fits the row-block buffers");
    unsigned char* stage = work + wave * kPass * kRowB;
    constexpr int CPR = D / 4;                        // 16-byte chunks per row
#pragma unroll 1
    for (int r0 = 0; r0 < 32; r0 += kPass) {
        if ((l32 & ~(kPass - 1)) == r0) {
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const f32x4 o = {acc[md][4 * b] * fac, acc[md][4 * b + 1] * fac, acc[md][4 * b + 2] * fac,
                                     acc[md][4 * b + 3] * fac};
                    *(f32x4*)(stage + (l32 - r0) * kRowB + 4 * (32 * md + 8 * b + 4 * g)) = o;
                }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the pass's rows are in LDS
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < kPass * CPR / 64; ++t) {
            const int rr = t * (64 / CPR) + lane / CPR, c = lane % CPR;
            const int j = key0 + 32 * kb + r0 + rr;
            if (split || j < p.M) {
                const f32x4 o = *(const f32x4*)(stage + rr * kRowB + 16 * c);
                *(f32x4*)(dst0 + (int64_t)(r0 + rr) * D + 4 * c) = o;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();   // the staged rows are read before the next pass
    }
}

// ----------------------------------------------------------------------------- fills

// Degenerate shapes: N == 0 (dK = dV = 0) or M == 0 (every row fully masked).
// dK and dV of the split key tiles: the kv_split row-range parts summed in part order.
template <int D>
__global__ __launch_bounds__(kThreads) void kvreduce_kernel(Params p, int tail) {
    const int64_t n4 = (int64_t)tail * 2 * kKVKeys * (D / 4);
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x) {
        const int c4 = (int)(e % (D / 4));
        const int64_t kr = e / (D / 4);
        const int key = (int)(kr % kKVKeys);
        const int role = (int)((kr / kKVKeys) % 2);
        const int tt = (int)(kr / (2 * kKVKeys));
        const int tile = p.kv_full + tt;
        const int hk = tile % p.Hkv, kvt = tile / p.Hkv;
        const int j = kvt * kKVKeys + key;
        if (j >= p.M) continue;
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int part = 0; part < p.kv_split; ++part) {
            const f32x4 v = *(const f32x4*)(p.kv_part + ((((int64_t)tt * p.kv_split + part) * 2 + role) * kKVKeys + key) * D + 4 * c4);
            s[0] += v[0];
            s[1] += v[1];
            s[2] += v[2];
            s[3] += v[3];
        }
        *(f32x4*)((role == 0 ? p.dk : p.dv) + ((int64_t)hk * p.M + j) * D + 4 * c4) = s;
    }
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float* a, int64_t n, float val) {
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads)
        a[e] = val;
}

}  // namespace fab
