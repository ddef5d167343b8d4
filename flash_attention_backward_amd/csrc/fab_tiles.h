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

// Issue priority of the calling wave around a chain of matrix products. The other wave on the
// SIMD is then mostly doing vector work; with the chain at the higher priority, each product
// issues as soon as the matrix unit is free instead of waiting behind that work (issue goes to
// the older wave when priorities are equal).
FAB_DEV void mfma_prio_hi() { __builtin_amdgcn_s_setprio(3); }
FAB_DEV void mfma_prio_lo() { __builtin_amdgcn_s_setprio(0); }

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

// The same copy from a uniform base plus a per-lane 32-bit byte offset, written out so that the
// compiler does not see it. The compiler makes every transpose read wait for all LDS DMA it
// knows to be in flight; a copy issued here stays in flight across them. The caller waits for
// it explicitly (wait_all_mem) before any read of its destination, and never reads or writes
// that destination while it is in flight. M0 is saved and restored around the copy.
FAB_DEV void dma16_hidden(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
    // the base and the LDS address are the same in every lane: taken from the first active lane
    // so that they sit in scalar registers whatever the compiler could prove
    // (readfirstlane returns a signed int: each half is taken back to uint32_t before widening)
    const uint64_t a = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    sbase = (const void*)(uintptr_t)((uint64_t)lo | ((uint64_t)hi << 32));
    lds_wave_base = (uint32_t)__builtin_amdgcn_readfirstlane(lds_wave_base);
    int keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(voff), "s"(sbase), "s"(lds_wave_base)
        : "memory");
}

// Wait for this wave's outstanding memory operations (DMA included) and make the compiler
// assume LDS may have changed.
FAB_DEV void wait_all_mem() {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}

// Workgroup barrier that publishes LDS writes only: it waits for this wave's LDS operations
// (lgkmcnt(0); vmcnt and expcnt left at their maxima) but not for global loads or DMA in
// flight, which __syncthreads() would also wait for. No memory access is moved across it.
FAB_DEV void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier once this wave's LDS operations, and all but its V most recent vector memory
// operations, have completed: the V most recent are LDS DMA of a later buffer, left in flight.
template <int V>
FAB_DEV void dma_barrier() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4));   // vmcnt(V) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until all but this wave's V most recent vector memory operations have completed (LDS
// operations are not waited for).
template <int V>
FAB_DEV void wait_vm() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (15 << 8));   // vmcnt(V)
    asm volatile("" ::: "memory");
}

// ----------------------------------------------------------------------------- block rows

// Rows of the ggml block types are staged raw in LDS and decoded from there.
FAB_DEV bool is_block_type(int type) {
    return type == FA_BACK_Q8_0 || type == FA_BACK_Q4_0 || type == FA_BACK_Q4_1 || type == FA_BACK_Q5_0 ||
           type == FA_BACK_Q5_1;
}
// bytes of one 32-value block
FAB_DEV int block_bytes(int type) {
    switch (type) {
        case FA_BACK_Q8_0: return 34;
        case FA_BACK_Q4_0: return 18;
        case FA_BACK_Q4_1: return 20;
        case FA_BACK_Q5_0: return 22;
        default: return 24;   // FA_BACK_Q5_1
    }
}
// bytes of one row of D values (D/32 blocks)
FAB_DEV int block_row_bytes(int type, int D) { return D / 32 * block_bytes(type); }

// Staged row geometry, sized for q8_0 (the longer block row): a row's bytes are staged in LDS
// as the 16-byte-aligned chunks that cover it (the row may start at any even address).
// The slot of a row in LDS has an odd number of 16-byte chunks, so that dword reads of the
// same block of 16 consecutive keys spread over the banks.
template <int D>
struct Q8Row {
    static constexpr int kBytes = D / 32 * 34;
    static constexpr int kChunks = ((kBytes + 29) / 16) | 1;   // covers a 14-byte misalignment
    static constexpr int kSlot = kChunks * 16;
};

template <int D, int KEYS>
struct RawTile {
    static constexpr int kBytes = KEYS * Q8Row<D>::kSlot + 16;
};

// Issue the DMA of the raw bytes of keys [j0, j0+KEYS) of head hk into `raw` (block types
// only; rbytes = bytes of one row, at most Q8Row<D>::kBytes). Chunk idx = key*kChunks + c lands
// at raw + 16*idx; chunks outside the row are skipped.
// NT threads take part, tid = 0 .. NT-1 being this thread's index among them.
template <int D, int KEYS, int NT>
FAB_DEV void dma_raw_tile(const char* base, int64_t nb1, int64_t nb2, int hk, int j0, int M,
                          int rbytes, unsigned char* raw, int tid) {
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
            ok = src < a + (uintptr_t)rbytes;      // only chunks holding bytes of this row
        }
        if (ok) dma16((const void*)src, raw + 16 * wbase);
    }
}

// The 8 values of cen (the row's centre, 32-byte aligned) that go with value group grp.
FAB_DEV void centre8(const float* cen, int grp, float c[8]) {
    const f32x4 x = *(const f32x4*)(cen + 8 * grp);
    const f32x4 y = *(const f32x4*)(cen + 8 * grp + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        c[t] = x[t];
        c[4 + t] = y[t];
    }
}

// 8 consecutive values of an F32, F16 or BF16 row (16-byte aligned), starting at value 8*grp,
// less the centre cen[8*grp + t] when cen is not NULL (F32, F16, BF16 only; the difference is
// formed in fp32), rounded to fp16.
template <int D>
FAB_DEV f16x8 decode8(const char* rowp, int type, int grp, const float* cen) {
    f16x8 r;
    if (type == FA_BACK_F32) {
        const f32x4 a = *(const f32x4*)(rowp + 32 * grp);
        const f32x4 b = *(const f32x4*)(rowp + 32 * grp + 16);
        if (cen) {
            float c[8];
            centre8(cen, grp, c);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                r[t] = (_Float16)(a[t] - c[t]);
                r[4 + t] = (_Float16)(b[t] - c[4 + t]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                r[t] = (_Float16)a[t];
                r[4 + t] = (_Float16)b[t];
            }
        }
    } else if (type == FA_BACK_F16) {
        r = *(const f16x8*)(rowp + 16 * grp);
        if (cen) {
            float c[8];
            centre8(cen, grp, c);
#pragma unroll
            for (int t = 0; t < 8; ++t) r[t] = (_Float16)((float)r[t] - c[t]);
        }
    } else if (type == FA_BACK_Q4_0) {
        // values 8*grp .. +7: block grp/4, elements 8*(grp%4) ..; elements t < 16 are the low
        // nibbles of bytes t, elements t >= 16 the high nibbles of bytes t - 16. The row is
        // 2-byte aligned: the scale and the 8 bytes are read as halfwords. (nibble - 8) * scale
        // is exact in fp32 and rounds once to fp16, as an F32 cache holding it would.
        const char* blk = rowp + 18 * (grp >> 2);
        const float dsc = (float)*(const _Float16*)blk;
        const unsigned short* qs = (const unsigned short*)(blk + 2 + 8 * (grp & 1));
        const int sh = (grp & 2) ? 4 : 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const unsigned int w = qs[t];
            r[2 * t] = (_Float16)((float)((int)((w >> sh) & 15u) - 8) * dsc);
            r[2 * t + 1] = (_Float16)((float)((int)((w >> (8 + sh)) & 15u) - 8) * dsc);
        }
    } else {   // BF16
        const u32x4 a = *(const u32x4*)(rowp + 16 * grp);
        float c[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (cen) centre8(cen, grp, c);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            r[2 * t] = (_Float16)(__uint_as_float(a[t] << 16) - c[2 * t]);
            r[2 * t + 1] = (_Float16)(__uint_as_float(a[t] & 0xffff0000u) - c[2 * t + 1]);
        }
    }
    return r;
}

// One 32-value q8_0 block of a staged row decoded to fp16: out[c] holds values 8c .. 8c+7.
// All LDS reads are issued before any arithmetic. A byte u = q + 128 placed under the fp16
// exponent pattern 0x64 reads as 1024 + u; subtracting 1152 gives q exactly, and one fp16
// product with the scale rounds q * d once (nearest even), which is the fp16 an F32 cache
// holding d * q gives. Both steps run on packed fp16 pairs.
// The scale is read with the int8 as the word before them: it is the high half of that word
// when the int8 start on a word boundary, else the low half of the first word. (The word before
// a slot's first block lies inside the staging buffer or right before it in the same LDS
// allocation; it is used only when it holds the scale.)
FAB_DEV void decode_q8_block(const unsigned char* slot, int off, int blk, f16x8 out[4]) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const int base = off + 34 * blk;                  // fp16 scale (even offset)
    const int qb = base + 2;                          // first int8
    const int sh = qb & 3;
    const unsigned int* wp = (const unsigned int*)(slot + (qb & ~3));
    unsigned int w[9];
    const unsigned int wm = wp[-1];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k] = wp[k];
    const unsigned short sb = (unsigned short)(sh ? (w[0] & 0xffffu) : (wm >> 16));
    const _Float16 dh = __builtin_bit_cast(_Float16, sb);
    const h2 d2 = {dh, dh};
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const unsigned int x = __builtin_amdgcn_alignbyte(w[k + 1], w[k], sh) ^ 0x80808080u;
        const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u));
        const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u));
        const h2 a = (lo + bias) * d2;
        const h2 c = (hi + bias) * d2;
        f16x8& o = out[k >> 1];
        const int b = 4 * (k & 1);
        o[b + 0] = a.x;
        o[b + 1] = a.y;
        o[b + 2] = c.x;
        o[b + 3] = c.y;
    }
}

// One 32-value q4_0 block of a staged row decoded to fp16: out[c] holds values 8c .. 8c+7.
// Value t < 16 is the low nibble of byte t, value t >= 16 the high nibble of byte t - 16. A
// nibble n placed under the fp16 exponent pattern 0x64 reads as 1024 + n; subtracting 1032
// gives n - 8 exactly, and one fp16 product with the scale rounds (n - 8) * d once, which is
// the fp16 an F32 cache holding that value gives. Both steps run on packed fp16 pairs.
FAB_DEV void decode_q4_block(const unsigned char* slot, int off, int blk, f16x8 out[4]) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const int base = off + 18 * blk;                  // fp16 scale (even offset)
    const int qb = base + 2;                          // first byte of nibbles
    const int sh = qb & 3;
    const unsigned int* wp = (const unsigned int*)(slot + (qb & ~3));
    unsigned int w[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) w[k] = wp[k];
    const unsigned short sb = *(const unsigned short*)(slot + base);
    const _Float16 dh = __builtin_bit_cast(_Float16, sb);
    const h2 d2 = {dh, dh};
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {                     // bytes 4k .. 4k+3
        const unsigned int x = __builtin_amdgcn_alignbyte(w[k + 1], w[k], sh);
        const unsigned int lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
        const h2 l01 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u));
        const h2 l23 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u));
        const h2 h01 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u));
        const h2 h23 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u));
        const h2 a = (l01 + bias) * d2, b = (l23 + bias) * d2;
        const h2 c = (h01 + bias) * d2, e = (h23 + bias) * d2;
        f16x8& ol = out[k >> 1];
        f16x8& oh = out[2 + (k >> 1)];
        const int o = 4 * (k & 1);
        ol[o + 0] = a.x;
        ol[o + 1] = a.y;
        ol[o + 2] = b.x;
        ol[o + 3] = b.y;
        oh[o + 0] = c.x;
        oh[o + 1] = c.y;
        oh[o + 2] = e.x;
        oh[o + 3] = e.y;
    }
}

// Values 8c .. 8c+7 of a 32-value q4_1, q5_0 or q5_1 block of a staged row, decoded to fp16.
// Fields are read as halfwords (the row is 2-byte aligned): fp16 d, [fp16 m], [the 32-bit word
// h whose bit t is bit 4 of code t], then 16 bytes, byte b holding the low nibbles of codes b and
// b + 16 (in its low and high half). So values 8c .. 8c+7 take bytes 8(c&1) .. +7, their low
// nibbles when c < 2, else the high ones, and bits 8c .. 8c+7 of h. A value is formed in fp32,
// d * (code - 16) for q5_0 and d * code + m otherwise (d * code is exact, so one fp32 rounding
// at most), and rounded once to fp16, as an F32 cache holding that fp32 value would be.
template <int TYPE>
FAB_DEV f16x8 decode_qx_chunk(const unsigned char* slot, int off, int blk, int c) {
    constexpr bool HAS_M = TYPE != FA_BACK_Q5_0;
    constexpr bool HAS_H = TYPE != FA_BACK_Q4_1;
    constexpr int NB = TYPE == FA_BACK_Q4_1 ? 20 : (TYPE == FA_BACK_Q5_0 ? 22 : 24);
    constexpr int QS = 2 + (HAS_M ? 2 : 0) + (HAS_H ? 4 : 0);   // byte offset of the nibbles
    const unsigned short* hw = (const unsigned short*)(slot + off + NB * blk);
    const float d = (float)__builtin_bit_cast(_Float16, hw[0]);
    const float m = HAS_M ? (float)__builtin_bit_cast(_Float16, hw[1]) : 0.0f;
    unsigned int hb = 0;   // bits 8c .. 8c+7 of h
    if constexpr (HAS_H) hb = ((unsigned int)hw[(HAS_M ? 2 : 1) + (c >> 1)] >> (8 * (c & 1))) & 0xffu;
    unsigned int q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = hw[QS / 2 + 4 * (c & 1) + k];
    const int sh = c < 2 ? 0 : 4;
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int code = (int)((q[i >> 1] >> (8 * (i & 1) + sh)) & 15u);
        if constexpr (HAS_H) code += (int)((hb >> i) & 1u) << 4;
        const float x = TYPE == FA_BACK_Q5_0 ? (float)(code - 16) * d : fmaf((float)code, d, m);
        r[i] = (_Float16)x;
    }
    return r;
}

// Values 8c .. 8c+7 of block blk of a staged row of type q4_1, q5_0 or q5_1.
FAB_DEV f16x8 decode_qx(int type, const unsigned char* slot, int off, int blk, int c) {
    if (type == FA_BACK_Q4_1) return decode_qx_chunk<FA_BACK_Q4_1>(slot, off, blk, c);
    if (type == FA_BACK_Q5_0) return decode_qx_chunk<FA_BACK_Q5_0>(slot, off, blk, c);
    return decode_qx_chunk<FA_BACK_Q5_1>(slot, off, blk, c);
}

// Block blk of a staged q8_0 or q4_0 row.
FAB_DEV void decode_block(int type, const unsigned char* slot, int off, int blk, f16x8 out[4]) {
    if (type == FA_BACK_Q8_0)
        decode_q8_block(slot, off, blk, out);
    else
        decode_q4_block(slot, off, blk, out);
}

// Decode keys [j0, j0+KEYS) into the swizzled fp16 tile dst[key][D]. Keys >= M become 0.
// cen: the head's centre (D floats) taken from every value before its rounding, or NULL
// (F32, F16 and BF16 rows only).
// NT threads take part, tid = 0 .. NT-1 being this thread's index among them.
//   block types: one item = one 32-value block of a key (from the staged raw bytes)
//   F32/F16/BF16: one item = 8 values of a key, read from global memory; every load of the
//   thread is issued before the first conversion
template <int D, int KEYS, int NT>
FAB_DEV void decode_tile(const char* base, int type, int64_t nb1, int64_t nb2, int hk, int j0,
                         int M, const unsigned char* raw, _Float16* dst, int tid,
                         const float* cen = nullptr) {
    const char* hbase = base + (int64_t)hk * nb2;
    if (is_block_type(type)) {
        constexpr int BPR = D / 32;                    // blocks per row
        constexpr int ITEMS = KEYS * BPR;
        for (int item = tid; item < ITEMS; item += NT) {
            const int key = item / BPR, blk = item - (item / BPR) * BPR;
            const int j = j0 + key;
            f16x8 out[4];
            const int off = (int)((uintptr_t)(hbase + (int64_t)j * nb1) & 15);
            const unsigned char* slot = raw + key * Q8Row<D>::kSlot;
            if (j < M && (type == FA_BACK_Q8_0 || type == FA_BACK_Q4_0)) {
                decode_block(type, slot, off, blk, out);
            } else if (j < M) {
                // the other block types a chunk of 8 values at a time, each stored when formed
#pragma unroll 1
                for (int c = 0; c < 4; ++c)
                    *(f16x8*)(dst + tile_off<D>(key, 4 * blk + c)) = decode_qx(type, slot, off, blk, c);
                continue;
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
        if (item < ITEMS && j < M) vals[it] = decode8<D>(hbase + (int64_t)j * nb1, type, grp, cen);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int item = tid + it * NT;
        const int key = item / GROUPS, grp = item - (item / GROUPS) * GROUPS;
        if (item < ITEMS) *(f16x8*)(dst + tile_off<D>(key, grp)) = vals[it];
    }
}

// K and V block-type (q8_0, q4_0) sub-tiles of 32 keys decoded together by 256 threads (4
// waves). One item is
// one 32-value block of one key. A wave-instruction covers 16 keys in the order
// 0,1,4,5,8,9,12,13,2,3,6,7,10,11,14,15 (plus 16 for the second half) times min(4, D/32)
// blocks, so that the 16-byte stores of 16 lanes land on 16 distinct bank groups of the
// swizzled tile and the dword reads of the staged bytes hit each bank at most twice.
//
// At D = 256 the lanes are arranged for the 32 four-byte banks instead (a dword read serves 32
// lanes at a time, a 16-byte store 8 lanes). A staged row takes an odd number of 16-byte
// chunks, so the same dword of keys k and k' falls in the same bank exactly when k = k' mod 8,
// and the int8 of block b start at dword (34b + 2) / 4 of the row, with residues 0 1 1 2 2 3 3 0
// mod 4 for b = 0 .. 7. Lanes 32h + 8j + t take block quad[j] of the blocks {0, 1, 3, 5} or
// {2, 4, 6, 7} (one per residue) and key K(h, t), where the 8 keys of a half have bit 3 equal
// to bit 1 (h = 0) or to its complement (h = 1): distinct in bits 0-2, so each half-wave's
// reads meet 32 distinct banks, and distinct in bits 0, 2 and 3, so each 8-lane group's stores
// meet 8 distinct 16-byte columns of the swizzled tile.
FAB_DEV int perm16(int t) { return (t & 1) | ((t & 6) << 1) | ((t & 8) >> 2); }

// (key within 16, block) of lane `lane` in block-quad bq (0: {0, 1, 3, 5}, 1: {2, 4, 6, 7})
FAB_DEV void item256(int lane, int bq, int& key, int& blk) {
    const int h = lane >> 5, j = (lane >> 3) & 3, t = lane & 7;
    key = (t & 1) | ((t & 2) << 1) | ((t & 4) >> 1) | ((((t >> 2) & 1) ^ h) << 3);
    blk = bq == 0 ? (j == 0 ? 0 : 2 * j - 1) : (j == 3 ? 7 : 2 * j + 2);
}

template <int D>
struct Q8Pair {
    static constexpr int BPR = D / 32;                // blocks per row
    static constexpr int BL = BPR >= 4 ? 4 : BPR;     // blocks per wave-instruction
    static constexpr int KL = 64 / BL;                // keys per wave-instruction
    static constexpr int KG = KL / 16;
    static constexpr int UPT = BPR / 2;               // wave-instructions per tensor
    static constexpr int U = 2 * UPT;                 // wave-instructions per sub-tile pair
};

// Wave-instruction u (0 .. U-1; K first, then V) of the pair decode. Q8 (compile time): both
// tensors are q8_0, with no test of the type in the decode.
template <int D, bool Q8>
FAB_DEV void decode_blk_item(const char* kh, int64_t knb1, int ktype, const char* vh, int64_t vnb1,
                             int vtype, int j0, int M, const unsigned char* rawk,
                             const unsigned char* rawv, _Float16* dstk, _Float16* dstv, int u,
                             int lane) {
    using Q = Q8Pair<D>;
    const bool isv = u >= Q::UPT;
    const int uu = isv ? u - Q::UPT : u;
    int key, blk;
    if constexpr (D == 256) {
        item256(lane, uu / 2, key, blk);
        key += 16 * (uu % 2);
    } else {
        key = perm16(lane & 15) + 16 * ((lane >> 4) % Q::KG) + Q::KL * (uu % (32 / Q::KL));
        blk = (lane >> 4) / Q::KG + Q::BL * (uu / (32 / Q::KL));
    }
    const int j = j0 + key;
    f16x8 o[4];
    if (j < M) {
        const char* h = isv ? vh : kh;
        const int64_t nb1 = isv ? vnb1 : knb1;
        const int off = (int)(((uint32_t)(uintptr_t)h + (uint32_t)j * (uint32_t)nb1) & 15u);
        const unsigned char* slot = (isv ? rawv : rawk) + key * Q8Row<D>::kSlot;
        if (Q8)
            decode_q8_block(slot, off, blk, o);
        else
            decode_block(isv ? vtype : ktype, slot, off, blk, o);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int t = 0; t < 8; ++t) o[c][t] = (_Float16)0.0f;
    }
    _Float16* dst = isv ? dstv : dstk;
#pragma unroll
    for (int c = 0; c < 4; ++c) *(f16x8*)(dst + tile_off<D>(key, 4 * blk + c)) = o[c];
}

// The q8_0 pair decode with fixed row strides (both multiples of 16 bytes, so a row's
// misalignment is that of the head's base): this lane's read and store offsets are the same
// for every sub-tile, so they are formed once (Q8Fixed::init) and each sub-tile adds only its
// buffers' addresses. A sub-tile wholly inside [0, M) takes no per-key test. The conversion is
// decode_q8_block's, instruction for instruction.
template <int D>
struct Q8Fixed {
    static constexpr int NIT = (Q8Pair<D>::U + 3) / 4;     // items of a wave (K first, then V)
    uint32_t rd[NIT];       // byte offset in the staged tile of the word before the item's int8
    uint32_t wr[NIT][4];    // byte offsets in the fp16 tile of its 4 sixteen-byte pieces
    int sh[NIT];            // byte offset of the int8 in their first word (0 or 2)
    int key[NIT];

    // first = this wave's index among the 4; offk / offv: the K / V heads' bases mod 16
    FAB_DEV void init(int first, int offk, int offv, int lane) {
        using Q = Q8Pair<D>;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int u = first + 4 * it;
            const bool isv = u >= Q::UPT;
            const int uu = isv ? u - Q::UPT : u;
            int k, blk;
            if constexpr (D == 256) {
                item256(lane, uu / 2, k, blk);
                k += 16 * (uu % 2);
            } else {
                k = perm16(lane & 15) + 16 * ((lane >> 4) % Q::KG) + Q::KL * (uu % (32 / Q::KL));
                blk = (lane >> 4) / Q::KG + Q::BL * (uu / (32 / Q::KL));
            }
            const int qb = (isv ? offv : offk) + 34 * blk + 2;
            key[it] = k;
            sh[it] = qb & 3;
            rd[it] = (uint32_t)(k * Q8Row<D>::kSlot + (qb & ~3) - 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) wr[it][c] = (uint32_t)(2 * tile_off<D>(k, 4 * blk + c));
        }
    }

    template <bool TAIL>
    FAB_DEV void decode_items(int j0, int M, const unsigned char* rawk, const unsigned char* rawv,
                              unsigned char* dstk, unsigned char* dstv, int first, int last) const {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int u = first + 4 * it;
            if (u >= Q8Pair<D>::U || u >= last) break;     // wave-uniform
            const bool isv = u >= Q8Pair<D>::UPT;          // wave-uniform
            const unsigned int* wp = (const unsigned int*)((isv ? rawv : rawk) + rd[it]);
            unsigned int w[10];
#pragma unroll
            for (int k = 0; k < 10; ++k) w[k] = wp[k];
            const unsigned short sb = (unsigned short)(sh[it] ? (w[1] & 0xffffu) : (w[0] >> 16));
            const _Float16 dh = __builtin_bit_cast(_Float16, sb);
            const h2 d2 = {dh, dh};
            f16x8 o[4];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const unsigned int x = __builtin_amdgcn_alignbyte(w[k + 2], w[k + 1], sh[it]) ^ 0x80808080u;
                const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u));
                const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u));
                const h2 a = (lo + bias) * d2;
                const h2 c = (hi + bias) * d2;
                const int b = 4 * (k & 1);
                o[k >> 1][b + 0] = a.x;
                o[k >> 1][b + 1] = a.y;
                o[k >> 1][b + 2] = c.x;
                o[k >> 1][b + 3] = c.y;
            }
            if constexpr (TAIL) {
                if (j0 + key[it] >= M) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[c][e] = (_Float16)0.0f;
                }
            }
            unsigned char* dst = isv ? dstv : dstk;
#pragma unroll
            for (int c = 0; c < 4; ++c) *(f16x8*)(dst + wr[it][c]) = o[c];
        }
    }

    FAB_DEV void decode(int j0, int M, const unsigned char* rawk, const unsigned char* rawv,
                        unsigned char* dstk, unsigned char* dstv, int first, int last) const {
        if (j0 + 32 <= M)                                   // uniform: no key past M
            decode_items<false>(j0, M, rawk, rawv, dstk, dstv, first, last);
        else
            decode_items<true>(j0, M, rawk, rawv, dstk, dstv, first, last);
    }
};

// The wave-instructions u = first, first + 4, ... below `last` for one of 4 waves.
template <int D, bool Q8>
FAB_DEV void decode_blk_pair32(const char* kh, int64_t knb1, int ktype, const char* vh, int64_t vnb1,
                               int vtype, int j0, int M, const unsigned char* rawk,
                               const unsigned char* rawv, _Float16* dstk, _Float16* dstv, int first,
                               int last, int lane) {
#pragma unroll
    for (int u = first; u < Q8Pair<D>::U; u += 4) {
        if (u >= last) break;                          // wave-uniform
        decode_blk_item<D, Q8>(kh, knb1, ktype, vh, vnb1, vtype, j0, M, rawk, rawv, dstk, dstv, u, lane);
    }
}

// DMA of consecutive q8_0 or q4_0 sub-tiles (KEYS keys each, sub-tile after sub-tile) into a staging
// buffer by NT threads; the row stride must be below 2^32. When the stride is a multiple of 16
// every row has the same alignment, so a chunk's source address only advances by KEYS rows from
// one sub-tile to the next and whether it holds bytes of its row never changes: a lane keeps the
// address of each chunk it moves and a sub-tile that lies inside [0, M) costs one 64-bit add per
// chunk. Otherwise (and for the last sub-tile) the address is formed from the key and the
// chunk's offset inside the aligned-down row.
template <int D, int KEYS, int NT>
struct RawDma {
    using R = Q8Row<D>;
    static constexpr int NCH = KEYS * R::kChunks;
    static constexpr int IT = (NCH + NT - 1) / NT;
    const char* base;      // the head's key 0 (wave-uniform)
    uint32_t nb1;          // row stride in bytes
    uint32_t rbytes;       // bytes of one row (at most R::kBytes)
    int j0;                // first key of the next sub-tile (wave-uniform)
    bool fixed;            // nb1 % 16 == 0 (wave-uniform)
    int kc[IT];            // key | (chunk byte offset << 8); -1 past the last chunk
    uint64_t src[IT];      // source of chunk `it` of the next sub-tile (fixed strides)
    bool on[IT];           // chunk `it` holds bytes of its row (fixed strides)

    FAB_DEV void init(const char* hbase, int64_t row_stride, int row_bytes, int first_key, int tid) {
        base = hbase;
        nb1 = (uint32_t)row_stride;
        rbytes = (uint32_t)row_bytes;
        j0 = first_key;
        fixed = (nb1 & 15u) == 0;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = it * NT + tid;
            const int key = idx / R::kChunks;
            kc[it] = idx < NCH ? key | ((16 * (idx - key * R::kChunks)) << 8) : -1;
            const int c16 = kc[it] >> 8;
            const uint64_t a = (uint64_t)(uintptr_t)base + (uint64_t)(uint32_t)(j0 + key) * nb1;
            src[it] = (a & ~(uint64_t)15) + (uint32_t)c16;
            on[it] = kc[it] >= 0 && (uint32_t)c16 < (uint32_t)(a & 15) + rbytes;
        }
    }
    // wave: this thread's wave among the NT threads (uniform); raw: staging buffer
    FAB_DEV void issue(unsigned char* raw, int M, int wave) {
        const uint64_t step = (uint64_t)KEYS * nb1;
        if (fixed && j0 + KEYS <= M) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int wbase = it * NT + wave * 64;
                if (wbase >= NCH) break;               // wave-uniform
                if (on[it]) dma16((const void*)(uintptr_t)src[it], raw + 16 * wbase);
                src[it] += step;
            }
        } else {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int wbase = it * NT + wave * 64;
                if (wbase >= NCH) break;               // wave-uniform
                const int key = kc[it] & 255, c16 = kc[it] >> 8;
                const int j = j0 + key;
                const uint64_t a = (uint64_t)(uintptr_t)base + (uint64_t)(uint32_t)j * nb1;
                const uint64_t sa = (a & ~(uint64_t)15) + (uint32_t)c16;
                // only chunks holding bytes of this row
                if (kc[it] >= 0 && j < M && (uint32_t)c16 < (uint32_t)(a & 15) + rbytes)
                    dma16((const void*)(uintptr_t)sa, raw + 16 * wbase);
                src[it] += step;
            }
        }
        j0 += KEYS;
    }
};

// ----------------------------------------------------------------------------- Gray walks

// Fragment reads stepped in Gray-code order: step t uses index gray(t) = t ^ (t >> 1), so
// consecutive steps differ in one bit b = ctz(t + 1) and, under the XOR swizzle, the lane's
// LDS address changes by a per-lane +-delta: one add per step.
FAB_DEV constexpr int gray(int t) { return t ^ (t >> 1); }
FAB_DEV constexpr int gray_bit(int t) { return __builtin_ctz(t + 1); }

FAB_DEV int swz_term(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// frag_rows reads (rows m0 + lane%32, d = 16*ks + 8*(lane/32) ..) of a swizzled [row][D] tile:
// byte offset of step ks = 0 for m0 = 0 and the per-bit steps of ks.
template <int D>
struct RowWalk {
    static constexpr int KS = D / 16;
    static constexpr int NB = KS == 16 ? 4 : (KS == 8 ? 3 : 2);
    int a0;
    int e[NB];   // step when bit b of ks goes 0 -> 1; minus it for 1 -> 0
};

template <int D>
FAB_DEV RowWalk<D> make_row_walk(int lane) {
    constexpr int CM = (D / 8) - 1;
    const int zr = swz_term(lane & 31) & CM, c = zr >> 1, g = lane >> 5;
    RowWalk<D> w;
    w.a0 = opaque((lane & 31) * D * 2 + 16 * (g ^ (zr & 1)) + 32 * c);
#pragma unroll
    for (int b = 0; b < RowWalk<D>::NB; ++b) w.e[b] = opaque(((c >> b) & 1) ? -(32 << b) : (32 << b));
    return w;
}

// byte offset change from step t to t+1 of a Gray walk with per-bit steps e
template <int NB>
FAB_DEV int gray_step(int t, const int (&e)[NB]) {
    const int b = gray_bit(t);
    return ((gray(t) >> b) & 1) ? -e[b] : e[b];
}

// frag_cols reads of a swizzled [row][D] tile, md stepped in Gray order: byte offsets of the
// two transpose reads for md = 0, kbase = 0 and their per-bit steps of md.
template <int D>
struct ColWalk {
    static constexpr int MD = D / 32;
    static constexpr int NB = MD == 8 ? 3 : (MD == 4 ? 2 : 1);
    int a0[2];
    int e[2][NB];
};

template <int D>
FAB_DEV ColWalk<D> make_col_walk(int lane) {
    constexpr int CM = (D / 8) - 1;
    const int g = lane >> 5, h16 = (lane >> 4) & 1, s = lane & 15;
    ColWalk<D> w;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * j + 4 * g + (s >> 2);
        const int zc = swz_term(row) & CM;
        const int cc = (2 * h16 + ((s & 3) >> 1)) ^ (zc & 3);
        const int ee = zc >> 2;
        w.a0[j] = opaque(row * D * 2 + 16 * (4 * ee + cc) + 8 * (s & 1));
#pragma unroll
        for (int b = 0; b < ColWalk<D>::NB; ++b) w.e[j][b] = opaque(((ee >> b) & 1) ? -(64 << b) : (64 << b));
    }
    return w;
}

FAB_DEV f16x4 tr_read(const unsigned char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(f16x4, v);
}

FAB_DEV f16x8 join(f16x4 a, f16x4 b) {
    f16x8 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        r[t] = a[t];
        r[4 + t] = b[t];
    }
    return r;
}

// sa += K Q^T and pa += V dO^T over d for one 32-key sub-tile: A operands from the K tile at
// `tile` and the V tile right after it (same rows), B operands bq/bd in registers; reads
// issued PF steps ahead, the two accumulator chains interleaved.
template <int D, int PF>
FAB_DEV void pair_rows(const unsigned char* tile, const f16x8* bq, const f16x8* bd, f32x16& sa,
                       f32x16& pa, const RowWalk<D>& w) {
    constexpr int KS = D / 16, NB = PF + 1;
    constexpr int VOFF = 32 * D * 2;                  // V tile follows the 32-row K tile
    int a = w.a0;                                     // offset of the next step to read
    f16x8 rk[NB], rv[NB];
#pragma unroll
    for (int t = 0; t < PF; ++t) {
        rk[t] = *(const f16x8*)(tile + a);
        rv[t] = *(const f16x8*)(tile + a + VOFF);
        if (t + 1 < KS) a += gray_step(t, w.e);
    }
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        if (t + PF < KS) {
            rk[(t + PF) % NB] = *(const f16x8*)(tile + a);
            rv[(t + PF) % NB] = *(const f16x8*)(tile + a + VOFF);
            if (t + PF + 1 < KS) a += gray_step(t + PF, w.e);
        }
        const int ks = gray(t);
        sa = mfma32(rk[t % NB], bq[ks], sa);
        pa = mfma32(rv[t % NB], bd[ks], pa);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// acc += A B over d for a 32x32 block: A operands frag_rows of the tile at `t` (its rows
// 0..31), B operands b[ks] in registers; steps in Gray order, reads PF steps ahead.
template <int D, int PF>
FAB_DEV void rows_chain(const unsigned char* t, const f16x8* b, f32x16& acc, const RowWalk<D>& w) {
    constexpr int KS = D / 16, NB = PF + 1;
    int a = w.a0;
    f16x8 r[NB];
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        r[s] = *(const f16x8*)(t + a);
        if (s + 1 < KS) a += gray_step(s, w.e);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (s + PF < KS) {
            r[(s + PF) % NB] = *(const f16x8*)(t + a);
            if (s + PF + 1 < KS) a += gray_step(s + PF, w.e);
        }
        acc = mfma32(r[s % NB], b[gray(s)], acc);
    }
}

// Compact forms of the two walks for waves short of registers: the address of step s is
// rebuilt from the lane's base and XOR term (an XOR and a shift-add) instead of stepping.
struct RowWalkX {
    int base;   // byte offset of the lane's row and half (g ^ zr0) part
    int c;      // ks is XORed with c
};
template <int D>
FAB_DEV RowWalkX make_row_walk_x(int lane) {
    constexpr int CM = (D / 8) - 1;
    const int zr = swz_term(lane & 31) & CM, g = lane >> 5;
    return {opaque((lane & 31) * D * 2 + 16 * (g ^ (zr & 1))), opaque(zr >> 1)};
}
FAB_DEV int row_addr(const RowWalkX& w, int ks) { return w.base + 32 * (ks ^ w.c); }

struct ColWalkX {
    int base[2];   // byte offsets of the two transpose reads without the md part
    int ee[2];     // md is XORed with ee
};
template <int D>
FAB_DEV ColWalkX make_col_walk_x(int lane) {
    constexpr int CM = (D / 8) - 1;
    const int g = lane >> 5, h16 = (lane >> 4) & 1, s = lane & 15;
    ColWalkX w;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * j + 4 * g + (s >> 2);
        const int zc = swz_term(row) & CM;
        const int cc = (2 * h16 + ((s & 3) >> 1)) ^ (zc & 3);
        w.base[j] = opaque(row * D * 2 + 16 * cc + 8 * (s & 1));
        w.ee[j] = opaque(zc >> 2);
    }
    return w;
}

// rows_chain with the compact walk
template <int D, int PF>
FAB_DEV void rows_chain_x(const unsigned char* t, const f16x8* b, f32x16& acc, const RowWalkX& w) {
    constexpr int KS = D / 16, NB = PF + 1;
    f16x8 r[NB];
#pragma unroll
    for (int s = 0; s < PF; ++s) r[s] = *(const f16x8*)(t + row_addr(w, gray(s)));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (s + PF < KS) r[(s + PF) % NB] = *(const f16x8*)(t + row_addr(w, gray(s + PF)));
        acc = mfma32(r[s % NB], b[gray(s)], acc);
    }
}

FAB_DEV uint32_t lds_addr(const unsigned char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// cols_acc with the compact walk, reads right before use (8 registers of fragments)
template <int D>
FAB_DEV void cols_acc_x(const unsigned char* t, const f16x8 b[2], f32x16* acc, const ColWalkX& w) {
    constexpr int MD = D / 32;
    constexpr int RH = 16 * D * 2;
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        const int md = gray(s);
        const int a0 = w.base[0] + 64 * (md ^ w.ee[0]);
        const int a1 = w.base[1] + 64 * (md ^ w.ee[1]);
        const f16x8 r0 = join(tr_read(t + a0), tr_read(t + a1));
        const f16x8 r1 = join(tr_read(t + a0 + RH), tr_read(t + a1 + RH));
        acc[md] = mfma32(r0, b[0], acc[md]);
        acc[md] = mfma32(r1, b[1], acc[md]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// cols_acc with the compact walk, each step's transpose reads issued one step ahead (two
// fragment sets in flight). The wave must have no LDS DMA in flight that the compiler knows of.
template <int D>
FAB_DEV void cols_acc_pf(const unsigned char* t, const f16x8 b[2], f32x16* acc, const ColWalkX& w) {
    constexpr int MD = D / 32;
    constexpr int RH = 16 * D * 2;
    f16x8 r0[2], r1[2];
    auto rd = [&](int s) {
        const int md = gray(s);
        const int a0 = w.base[0] + 64 * (md ^ w.ee[0]);
        const int a1 = w.base[1] + 64 * (md ^ w.ee[1]);
        r0[s & 1] = join(tr_read(t + a0), tr_read(t + a1));
        r1[s & 1] = join(tr_read(t + a0 + RH), tr_read(t + a1 + RH));
    };
    rd(0);
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        if (s + 1 < MD) rd(s + 1);
        const int md = gray(s);
        acc[md] = mfma32(r0[s & 1], b[0], acc[md]);
        acc[md] = mfma32(r1[s & 1], b[1], acc[md]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Transposed pair for key-owned waves: sa += K Q^T (A: bk in registers, B: q rows of the tile
// at t) and pa += V dO^T (A: bv, B: dO rows of the tile at t + DOFF), over d in the Gray order
// of pair_rows, reads PF steps ahead. One query row per lane column, 16 keys per lane. ZERO:
// the sums start from zero instead of from sa and pa.
template <int D, int PF, int DOFF, bool ZERO = false>
FAB_DEV void pair_rows_t(const unsigned char* t, const f16x8* bk, const f16x8* bv, f32x16& sa, f32x16& pa,
                         const RowWalk<D>& w) {
    constexpr int KS = D / 16, NB = PF + 1;
    int a = w.a0;
    f16x8 rq[NB], rd[NB];
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        rq[s] = *(const f16x8*)(t + a);
        rd[s] = *(const f16x8*)(t + a + DOFF);
        if (s + 1 < KS) a += gray_step(s, w.e);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (s + PF < KS) {
            rq[(s + PF) % NB] = *(const f16x8*)(t + a);
            rd[(s + PF) % NB] = *(const f16x8*)(t + a + DOFF);
            if (s + PF + 1 < KS) a += gray_step(s + PF, w.e);
        }
        const int ks = gray(s);
        sa = mfma32(bk[ks], rq[s % NB], (ZERO && s == 0) ? f32x16{} : sa);
        pa = mfma32(bv[ks], rd[s % NB], (ZERO && s == 0) ? f32x16{} : pa);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Key-side pair: sa += Q K^T (A: q rows of the tile at tq, B: bk in registers) and
// pa += dO V^T (A: dO rows of the tile at tq + DOFF, B: V rows of the tile at tv), over d in
// the same Gray order as pair_rows, so both sides sum every score in the same order.
template <int D, int PF, int DOFF>
FAB_DEV void pair_rows_kv(const unsigned char* tq, const unsigned char* tv, const f16x8* bk, f32x16& sa,
                          f32x16& pa, const RowWalk<D>& w) {
    constexpr int KS = D / 16, NB = PF + 1;
    int a = w.a0;
    f16x8 rq[NB], rd[NB], rv[NB];
#pragma unroll
    for (int t = 0; t < PF; ++t) {
        rq[t] = *(const f16x8*)(tq + a);
        rd[t] = *(const f16x8*)(tq + a + DOFF);
        rv[t] = *(const f16x8*)(tv + a);
        if (t + 1 < KS) a += gray_step(t, w.e);
    }
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        if (t + PF < KS) {
            rq[(t + PF) % NB] = *(const f16x8*)(tq + a);
            rd[(t + PF) % NB] = *(const f16x8*)(tq + a + DOFF);
            rv[(t + PF) % NB] = *(const f16x8*)(tv + a);
            if (t + PF + 1 < KS) a += gray_step(t + PF, w.e);
        }
        sa = mfma32(rq[t % NB], bk[gray(t)], sa);
        pa = mfma32(rd[t % NB], rv[t % NB], pa);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// acc[md] += A(md, 0) b[0] + A(md, 1) b[1] for md = 0 .. D/32-1, A(md, rh) the frag_cols read
// of rows 16*rh .. 16*rh+15 of the tile at `t` (a contraction over its 32 rows); md in Gray
// order. The reads run PF steps ahead of their products (8 registers per step); PF = 0 reads
// right before use.
template <int D, int PF = 1>
FAB_DEV void cols_acc(const unsigned char* t, const f16x8 b[2], f32x16* acc, const ColWalk<D>& w) {
    constexpr int MD = D / 32;
    constexpr int RH = 16 * D * 2;                    // bytes of 16 rows
    constexpr int NB = PF + 1;
    int a0 = w.a0[0], a1 = w.a0[1];
    f16x8 r0[NB], r1[NB];
    // the reads of step s + PF (md = gray(s + PF)); the walk is stepped as they are issued
    auto rd = [&](int q) {
        r0[q % NB] = join(tr_read(t + a0), tr_read(t + a1));
        r1[q % NB] = join(tr_read(t + a0 + RH), tr_read(t + a1 + RH));
        if (q + 1 < MD) {
            a0 += gray_step(q, w.e[0]);
            a1 += gray_step(q, w.e[1]);
        }
    };
#pragma unroll
    for (int q = 0; q < PF; ++q) rd(q);
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        if (s + PF < MD) rd(s + PF);
        const int md = gray(s);
        acc[md] = mfma32(r0[s % NB], b[0], acc[md]);
        acc[md] = mfma32(r1[s % NB], b[1], acc[md]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace fab
