// LDS tiles: K/V tiles decoded once per workgroup from HBM, and the fragment reads of the
// 32x32x16 products. The cache itself is never converted.
#pragma once

#include "fab_common.h"

namespace fab {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// ----------------------------------------------------------------------------- layout

// Row-major fp16 tiles [row][D] are stored without padding, 16-byte chunks of a row permuted
// by an XOR swizzle. It keeps both access patterns free of bank conflicts:
//   - a 16-lane b128 read of one logical chunk from 16 consecutive rows, and
//   - a 32-lane transpose read covering 4 consecutive rows x 4 consecutive chunks.
template <int D>
FAB_DEV int swz_chunk(int row, int chunk) {
    constexpr int CM = (D / 8) - 1;   // chunks per row - 1 (8, 16 or 32 chunks)
    return chunk ^ ((((row & 3) << 2) | ((row >> 2) & 3)) & CM);
}

// halfs offset of (row, chunk) in a swizzled [rows][D] tile
template <int D>
FAB_DEV int tile_off(int row, int chunk) { return row * D + 8 * swz_chunk<D>(row, chunk); }

// Per-lane swizzle terms of the fragment reads below. They depend only on the lane (row
// blocks start at multiples of 16 rows) and are passed through an opaque move where a loop
// starts, so that the compiler computes each step's LDS address in the loop instead of
// keeping one precomputed address per step alive (and spilling them).
struct Swz {
    int rows;    // XOR term of frag_rows: swizzle of row lane%32
    int col0;    // XOR term of frag_cols, first transpose read
    int col1;    // XOR term of frag_cols, second transpose read
};

FAB_DEV int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int D>
FAB_DEV Swz make_swz(int lane) {
    constexpr int CM = (D / 8) - 1;
    const int g = lane >> 5, s = lane & 15;
    auto f = [](int row) { return ((row & 3) << 2) | ((row >> 2) & 3); };
    Swz z;
    z.rows = opaque(f(lane & 31) & CM);
    z.col0 = opaque(f(4 * g + (s >> 2)) & CM);
    z.col1 = opaque(f(8 + 4 * g + (s >> 2)) & CM);
    return z;
}

// A operand of a contraction over d: lane l reads row m0 + l%32, d = 16*ks + 8*(l/32) .. +7.
// m0 must be a multiple of 16.
template <int D>
FAB_DEV f16x8 frag_rows(const _Float16* tile, int m0, int ks, int lane, const Swz& z) {
    const int row = m0 + (lane & 31);
    return *(const f16x8*)(tile + row * D + 8 * ((2 * ks + (lane >> 5)) ^ z.rows));
}

// A operand of a contraction over the rows of a swizzled [row][D] tile (rows are the k index,
// d the m index): lane l gets d = 32*md + l%32 and the 8 rows kbase + crow(t, l/32), t = 0..7
// (that is kbase + 8*(t/4) + 4*(l/32) + t%4), matching the B operand taken from an
// accumulator's registers 8*rh + t. Built from two ds_read_b64_tr_b16: in each 16-lane group
// lane 4a+b receives element b of the 8-byte reads of lanes a, a+4, a+8, a+12.
// kbase must be a multiple of 16.
template <int D>
FAB_DEV f16x8 frag_cols(const _Float16* tile, int md, int kbase, int lane, const Swz& z) {
    const int g = lane >> 5, h16 = (lane >> 4) & 1, s = lane & 15;
    const int dcol = 32 * md + 16 * h16 + 4 * (s & 3);     // first of the 4 columns read
    const int chunk = dcol >> 3, within = dcol & 7;
    f16x8 r;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = kbase + 8 * j + 4 * g + (s >> 2);
        const _Float16* p = tile + row * D + 8 * (chunk ^ (j ? z.col1 : z.col0)) + within;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
        const f16x4 h = __builtin_bit_cast(f16x4, v);
        r[4 * j + 0] = h[0];
        r[4 * j + 1] = h[1];
        r[4 * j + 2] = h[2];
        r[4 * j + 3] = h[3];
    }
    return r;
}

// ----------------------------------------------------------------------------- DMA

// Asynchronous 16-byte-per-lane copy HBM -> LDS; lane l writes lds_wave_base + 16*l.
// lds_wave_base must be the same for every lane of the wave.
FAB_DEV void dma16(const void* gsrc, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// Wait for this wave's outstanding memory operations (DMA included) and make the compiler
// assume LDS may have changed.
FAB_DEV void wait_all_mem() {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}

// ----------------------------------------------------------------------------- q8_0 rows

// q8_0 row geometry: D/32 blocks of 34 bytes; a row's bytes are staged in LDS as the
// 16-byte-aligned chunks that cover it (the row may start at any even address).
template <int D>
struct Q8Row {
    static constexpr int kBytes = D / 32 * 34;
    static constexpr int kChunks = (kBytes + 29) / 16;   // covers a 14-byte misalignment
    static constexpr int kSlot = kChunks * 16;
};

template <int D, int KEYS>
struct RawTile {
    static constexpr int kBytes = KEYS * Q8Row<D>::kSlot + 16;
};

// Issue the DMA of the raw bytes of keys [j0, j0+KEYS) of head hk into `raw` (q8_0 only).
// Chunk idx = key*kChunks + c lands at raw + 16*idx; chunks outside the row are skipped.
// NT threads take part, tid = 0 .. NT-1 being this thread's index among them.
template <int D, int KEYS, int NT>
FAB_DEV void dma_raw_tile(const char* base, int64_t nb1, int64_t nb2, int hk, int j0, int M,
                          unsigned char* raw, int tid) {
    using R = Q8Row<D>;
    constexpr int NCH = KEYS * R::kChunks;
    constexpr int IT = (NCH + NT - 1) / NT;
    const char* hbase = base + (int64_t)hk * nb2;
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int wbase = it * NT + wave * 64;         // first chunk of this wave's instruction
        if (wbase >= NCH) break;                        // wave-uniform
        const int idx = wbase + lane;
        const int key = idx / R::kChunks;
        const int c = idx - key * R::kChunks;
        const int j = j0 + key;
        bool ok = idx < NCH && j < M;
        uintptr_t src = 0;
        if (ok) {
            const uintptr_t a = (uintptr_t)(hbase + (int64_t)j * nb1);
            const uintptr_t a0 = a & ~(uintptr_t)15;
            src = a0 + 16u * (uintptr_t)c;
            ok = src < a + R::kBytes;      // only chunks holding bytes of this row
        }
        if (ok) dma16((const void*)src, raw + 16 * wbase);
    }
}

// 8 consecutive values of an F32, F16 or BF16 row (16-byte aligned), starting at value 8*grp,
// rounded to fp16.
template <int D>
FAB_DEV f16x8 decode8(const char* rowp, int type, int grp, const unsigned char*, int) {
    f16x8 r;
    if (type == FA_BACK_F32) {
        const f32x4 a = *(const f32x4*)(rowp + 32 * grp);
        const f32x4 b = *(const f32x4*)(rowp + 32 * grp + 16);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            r[t] = (_Float16)a[t];
            r[4 + t] = (_Float16)b[t];
        }
    } else if (type == FA_BACK_F16) {
        r = *(const f16x8*)(rowp + 16 * grp);
    } else {   // BF16
        const u32x4 a = *(const u32x4*)(rowp + 16 * grp);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            r[2 * t] = (_Float16)__uint_as_float(a[t] << 16);
            r[2 * t + 1] = (_Float16)__uint_as_float(a[t] & 0xffff0000u);
        }
    }
    return r;
}

// One 32-value q8_0 block of a staged row decoded to fp16: out[c] holds values 8c .. 8c+7.
// All LDS reads are issued before any arithmetic. Each value is formed as
// fma(byte ^ 0x80, d, -128 d) = d * q, exact in fp32, then rounded to fp16 (nearest even),
// the same fp16 an F32 cache holding d * q gives.
FAB_DEV void decode_q8_block(const unsigned char* slot, int off, int blk, f16x8 out[4]) {
    const int base = off + 34 * blk;                  // fp16 scale (even offset)
    const int qb = base + 2;                          // first int8
    const int sh = qb & 3;
    const unsigned int* wp = (const unsigned int*)(slot + (qb & ~3));
    unsigned int w[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k] = wp[k];
    const unsigned short sb = *(const unsigned short*)(slot + base);
    const float d = (float)__builtin_bit_cast(_Float16, sb);
    const float nd = -128.0f * d;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const unsigned int x = __builtin_amdgcn_alignbyte(w[k + 1], w[k], sh) ^ 0x80808080u;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            out[k >> 1][4 * (k & 1) + b] = (_Float16)fmaf((float)((x >> (8 * b)) & 0xffu), d, nd);
    }
}

// Decode keys [j0, j0+KEYS) into the swizzled fp16 tile dst[key][D]. Keys >= M become 0.
// NT threads take part, tid = 0 .. NT-1 being this thread's index among them.
//   q8_0: one item = one 32-value block of a key (from the staged raw bytes)
//   F32/F16/BF16: one item = 8 values of a key, read from global memory; every load of the
//   thread is issued before the first conversion
template <int D, int KEYS, int NT>
FAB_DEV void decode_tile(const char* base, int type, int64_t nb1, int64_t nb2, int hk, int j0,
                         int M, const unsigned char* raw, _Float16* dst, int tid) {
    const char* hbase = base + (int64_t)hk * nb2;
    if (type == FA_BACK_Q8_0) {
        constexpr int BPR = D / 32;                    // blocks per row
        constexpr int ITEMS = KEYS * BPR;
        for (int item = tid; item < ITEMS; item += NT) {
            const int key = item / BPR, blk = item - (item / BPR) * BPR;
            const int j = j0 + key;
            f16x8 out[4];
            if (j < M) {
                const int off = (int)((uintptr_t)(hbase + (int64_t)j * nb1) & 15);
                decode_q8_block(raw + key * Q8Row<D>::kSlot, off, blk, out);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int t = 0; t < 8; ++t) out[c][t] = (_Float16)0.0f;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) *(f16x8*)(dst + tile_off<D>(key, 4 * blk + c)) = out[c];
        }
        return;
    }
    constexpr int GROUPS = D / 8;
    constexpr int ITEMS = KEYS * GROUPS;
    constexpr int IT = (ITEMS + NT - 1) / NT;
    f16x8 vals[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int item = tid + it * NT;
        const int key = item / GROUPS, grp = item - (item / GROUPS) * GROUPS;
        const int j = j0 + key;
#pragma unroll
        for (int t = 0; t < 8; ++t) vals[it][t] = (_Float16)0.0f;
        if (item < ITEMS && j < M) vals[it] = decode8<D>(hbase + (int64_t)j * nb1, type, grp, nullptr, 0);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int item = tid + it * NT;
        const int key = item / GROUPS, grp = item - (item / GROUPS) * GROUPS;
        if (item < ITEMS) *(f16x8*)(dst + tile_off<D>(key, grp)) = vals[it];
    }
}

// K and V q8_0 tiles decoded together (items of both tensors interleaved, so that the LDS
// reads of one overlap the arithmetic of the other). Same result as two decode_tile calls.
template <int D, int KEYS, int NT>
FAB_DEV void decode_q8_pair(const char* kbase, int64_t knb1, int64_t knb2, const char* vbase,
                            int64_t vnb1, int64_t vnb2, int hk, int j0, int M,
                            const unsigned char* rawk, const unsigned char* rawv,
                            _Float16* dstk, _Float16* dstv, int tid) {
    constexpr int BPR = D / 32;
    constexpr int ITEMS = KEYS * BPR;                 // per tensor
    const char* kh = kbase + (int64_t)hk * knb2;
    const char* vh = vbase + (int64_t)hk * vnb2;
    for (int item = tid; item < ITEMS; item += NT) {
        const int key = item / BPR, blk = item - (item / BPR) * BPR;
        const int j = j0 + key;
        f16x8 ok[4], ov[4];
        if (j < M) {
            const int offk = (int)((uintptr_t)(kh + (int64_t)j * knb1) & 15);
            const int offv = (int)((uintptr_t)(vh + (int64_t)j * vnb1) & 15);
            decode_q8_block(rawk + key * Q8Row<D>::kSlot, offk, blk, ok);
            decode_q8_block(rawv + key * Q8Row<D>::kSlot, offv, blk, ov);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int t = 0; t < 8; ++t) ok[c][t] = ov[c][t] = (_Float16)0.0f;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            *(f16x8*)(dstk + tile_off<D>(key, 4 * blk + c)) = ok[c];
            *(f16x8*)(dstv + tile_off<D>(key, 4 * blk + c)) = ov[c];
        }
    }
}

}  // namespace fab
