// Shared device definitions for the flash-attention backward kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_back.h"

#define FAB_DEV __device__ __forceinline__

namespace fab {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kRowBlock = 32;     // rows per MFMA block (the 32 of a 32x32x16 product)
constexpr int kQTileKeys = 64;    // keys per tile in the query-side passes
constexpr int kKVKeys = 128;      // keys owned by one key-side workgroup (32 per wave)
constexpr int kPScaleLog2 = 15;   // P is rounded to fp16 as p * 2^15 (p <= 1)
constexpr int kNegInfBits = 0xff800000;

// Everything the kernels need, passed by value.
struct Params {
    const char* q;
    const char* k;
    const char* v;
    const char* d;
    const char* mask;
    int64_t q_nb0, q_nb1, q_nb2;   // (c, i, h)
    int64_t d_nb0, d_nb1, d_nb2;   // (c, h, i)
    int64_t k_nb1, k_nb2;          // (row j, head hk)
    int64_t v_nb1, v_nb2;
    int64_t m_nb0, m_nb1, m_nb2;   // (j, i, hm)
    int q_type, d_type, k_type, v_type, m_type;
    int D, H, Hkv, G, N, M, Hm;
    int R;            // query rows per KV head: G * N, row r = i*G + g  (h = hk*G + g)
    int RB;           // 32-row blocks per KV head
    int RT;           // query-side row tiles (kWaves row blocks each) per KV head
    int KT;           // 64-key tiles
    int splits;       // key-range splits of the query-side passes
    int tiles_per_split;
    int KVT;          // 128-key tiles of the key-side pass
    int w1_rbs;       // walk 1 by key tiles: row blocks per workgroup
    int w1_tps;       // walk 1 by row tiles: 64-key tiles per key-range split
    int nparts;       // walk-1 records per row that the merge combines (splits or key tiles)
    float scale;
    // outputs (packed)
    float* dq;
    float* dk;
    float* dv;
    float* lse;
    float* delta;
    // workspace
    float* absmax_part;   // [2][npart]
    int npart;
    int* scal;            // [0] = e_q, [1] = e_do (power-of-two exponents)
    _Float16* qr;         // [Hkv][RB*32][D]  q rows scaled by 2^e_q, fp16, row-major
    _Float16* dr;         // [Hkv][RB*32][D]  dO rows scaled by 2^e_do, fp16, row-major
    f32x4* part_rec;      // [nparts][Hkv*RB*32] walk-1 records {max m (log2 units), softmax sum
                          //   at m, sum of e * dp at m (dp in 2^e_do units), max |dp| over visible keys}
    float* row_lse2;      // [Hkv*RB*32]  lse in log2 units minus kPScaleLog2, so that exp2(s - row_lse2)
                          //   is the P image p * 2^15; +inf for dead or padding rows (the image is 0
                          //   for them with no test)
    float* row_dlt;       // [Hkv*RB*32]  delta in 2^e_do units
    int* row_ks;          // [Hkv*RB*32]  the row's dS exponent: dS goes to fp16 as dS * 2^-ks (walk 2)
    float* bound_part;    // [Hkv][nbound] per-block max of max|dp| + |delta| over a head's rows
    int nbound;           // blocks per KV head
    float* dq_part;       // [splits][Hkv*RB*32][D] when splits > 1
    unsigned char* mcls;  // [Hc][RB][KT] mask class of (row block, 64-key tile); Hc = Hm==1 ? 1 : Hkv
    // key side: workgroups 0 .. kv_full-1 own one 128-key tile (tile = workgroup); each of the
    // remaining tiles is split into kv_split row ranges whose dK/dV go to kv_part
    int kv_full, kv_split;
    float* kv_part;       // [tail tile][part][dK, dV][128 keys][D]
    // forward-saved statistics (fa_back_run_saved); null for the full operator
    const float* lse_in;  // [H*N] natural-log LSE, row h*N + i
    const float* o_in;    // [H][N][Dv] forward output O, F32
    float* vmax_part;     // [nvpart] partial max |v| over the cache
    int nvpart;
    float* vcen;          // [Hkv][D] constant taken from V before its fp16 rounding; NULL: none
    float* kcen;          // [Hkv][D] constant taken from K before its fp16 rounding; NULL: none
    unsigned char* kvimg; // [Hkv][img_ns][32-key slot] decoded K and V tiles of the query-side
                          //   walks (kvimage_kernel); NULL: the walks decode for themselves
    int img_ns;           // 32-key sub-tiles per head in kvimg
    _Float16* dsbuf;      // [Hkv][RB][ds_kb][32 x 32] dS tiles the key side stores for the dQ
                          // pass from stored dS (NULL when walk 2 forms dQ)
    int ds_kb;            // 32-key blocks per row block and head in dsbuf (4 per 128-key tile)
};

// Mask classes of a (32-row block, 64-key tile): no masking needed, every entry -inf, other.
constexpr int kMaskZero = 0;
constexpr int kMaskDead = 1;
constexpr int kMaskMixed = 2;

// Row of the 32x32 product held in accumulator register v by a lane of half g (= lane/32);
// the column is lane % 32.
FAB_DEV int crow(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// dS = p (dp - delta) to fp16 as walk 2 forms it: the product rounded to fp32, then to fp16.
// The product passes through an empty asm statement so that the compiler cannot fuse the
// multiply into the conversion (v_fma_mix, one rounding instead of two) in some paths and not in
// others: every path that forms walk 2's dS gives the same bits.
FAB_DEV _Float16 ds_f16(float pv, float dp, float delta) {
    float x = pv * (dp - delta);
    asm volatile("" : "+v"(x));
    return (_Float16)x;
}

FAB_DEV f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

FAB_DEV float neg_inf() { return __int_as_float(kNegInfBits); }
FAB_DEV float pos_inf() { return -neg_inf(); }

FAB_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

FAB_DEV float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

FAB_DEV float load_scalar(const char* p, int type) {
    if (type == FA_BACK_F32) return *(const float*)p;
    if (type == FA_BACK_F16) return (float)*(const _Float16*)p;
    return bf16_to_f32(*(const unsigned short*)p);
}

// A value of lane l combined with that of lane l ^ 32 without going through LDS: two copies of x
// with their halves swapped (v_permlane32_swap) hold, in every lane, the value of lane l & 31
// and that of lane (l & 31) + 32. Both operations are commutative, so every lane gets exactly
// op(x[l], x[l ^ 32]).
FAB_DEV void wave_halves(float x, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
FAB_DEV float max_halves(float x) {
    float lo, hi;
    wave_halves(x, lo, hi);
    return fmaxf(lo, hi);
}
FAB_DEV float sum_halves(float x) {
    float lo, hi;
    wave_halves(x, lo, hi);
    return lo + hi;
}

FAB_DEV float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// Power-of-two exponent s so that amax * 2^s lies in [2^14, 2^15) (0 for an all-zero or
// non-finite input), clamped to [-64, 64].
FAB_DEV int prescale_exponent(float amax) {
    if (!(amax > 0.0f) || !(amax < 3.0e38f)) return 0;
    int e;
    frexpf(amax, &e);   // amax = m * 2^e, m in [0.5, 1)
    int s = 15 - e;
    return s < -64 ? -64 : (s > 64 ? 64 : s);
}

// Exponent ks so that values bounded by b scaled by 2^-ks stay below 2^15.
FAB_DEV int ds_exponent(float b) {
    if (!(b > 0.0f) || !(b < 3.0e38f)) return 0;
    int e;
    frexpf(b, &e);      // b < 2^e
    int ks = e - 15;
    return ks < -100 ? -100 : (ks > 100 ? 100 : ks);
}

}  // namespace fab
