// K/V tile decoding into LDS: each tile is read from HBM with 16-byte loads and decoded to
// fp16 exactly once per workgroup. The cache itself is never converted.
#pragma once

#include "fab_common.h"

namespace fab {

// q8_0 row geometry: D/32 blocks of 34 bytes; a row's bytes are staged in LDS as the
// 16-byte-aligned chunks that cover it (the row may start at any even address).
template <int D>
struct Q8Row {
    static constexpr int kBytes = D / 32 * 34;
    static constexpr int kChunks = (kBytes + 29) / 16;   // covers a 14-byte misalignment
    static constexpr int kSlot = kChunks * 16;
};

template <int D, int KEYS>
struct TileLds {
    static constexpr int kLd = D + 8;            // fp16 row stride of a [key][d] tile
    static constexpr int kLdT = KEYS + 8;        // fp16 row stride of a [d][key] tile
    static constexpr int kRaw = KEYS * Q8Row<D>::kSlot + 16;
};

// Position of key `key` (within a tile) in a transposed [d][key] tile. Inside each group of
// 16 keys, position 8*g + t holds key 8*(t/4) + 4*g + t%4, so the 8 keys that a lane of half
// g supplies to a contraction over keys (rows crow(8*rh + t, g) of a 32x32 product) are
// contiguous.
FAB_DEV int tpos(int key) {
    const int k16 = key & 15;
    return (key & ~15) + 8 * ((k16 >> 2) & 1) + 4 * (k16 >> 3) + (k16 & 3);
}

// Phase 1: stage the raw bytes of keys [j0, j0+KEYS) of head hk into `raw` (q8_0 only).
template <int D, int KEYS>
FAB_DEV void stage_tile(const char* base, int type, int64_t nb1, int64_t nb2, int hk, int j0,
                        int M, unsigned char* raw) {
    if (type != FA_BACK_Q8_0) return;
    using R = Q8Row<D>;
    constexpr int NCH = KEYS * R::kChunks;
    constexpr int IT = (NCH + kThreads - 1) / kThreads;
    const char* hbase = base + (int64_t)hk * nb2;
    u32x4 buf[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = threadIdx.x + it * kThreads;
        buf[it] = u32x4{0u, 0u, 0u, 0u};
        if (idx < NCH) {
            const int key = idx / R::kChunks;
            const int c = idx - key * R::kChunks;
            const int j = j0 + key;
            if (j < M) {
                const uintptr_t a = (uintptr_t)(hbase + (int64_t)j * nb1);
                const uintptr_t a0 = a & ~(uintptr_t)15;
                // only chunks that hold bytes of this row are read
                if (a0 + 16u * (uintptr_t)c < a + R::kBytes)
                    buf[it] = *(const u32x4*)(a0 + 16u * (uintptr_t)c);
            }
        }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = threadIdx.x + it * kThreads;
        if (idx < NCH) *(u32x4*)(raw + 16 * idx) = buf[it];
    }
}

// 8 consecutive values of row `key` starting at value 8*grp, decoded to fp16.
template <int D>
FAB_DEV f16x8 decode8(const char* rowp, int type, int grp, const unsigned char* rawslot, int off) {
    f16x8 r;
    if (type == FA_BACK_Q8_0) {
        const int blk = grp >> 2;
        const int so = off + 34 * blk;                  // scale offset within the slot (even)
        const unsigned short sb = *(const unsigned short*)(rawslot + so);
        const float sc = (float)__builtin_bit_cast(_Float16, sb);
        const int qo = so + 2 + 8 * (grp & 3);          // first int8 (even)
        const unsigned int* wp = (const unsigned int*)(rawslot + (qo & ~3));
        const unsigned int w0 = wp[0], w1 = wp[1], w2 = wp[2];
        const unsigned int lo = __builtin_amdgcn_alignbyte(w1, w0, qo & 3);
        const unsigned int hi = __builtin_amdgcn_alignbyte(w2, w1, qo & 3);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            r[t] = (_Float16)(sc * (float)(signed char)(lo >> (8 * t)));
            r[4 + t] = (_Float16)(sc * (float)(signed char)(hi >> (8 * t)));
        }
    } else if (type == FA_BACK_F32) {
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

// Phase 2: decode keys [j0, j0+KEYS) into dst ([key][d], stride kLd) and, if TRANS, into
// dstT ([d][tpos(key)], stride kLdT). Keys >= M become 0. Work item = 4 keys x 8 values.
template <int D, int KEYS, bool TRANS>
FAB_DEV void decode_tile(const char* base, int type, int64_t nb1, int64_t nb2, int hk, int j0,
                         int M, const unsigned char* raw, _Float16* dst, _Float16* dstT) {
    using L = TileLds<D, KEYS>;
    constexpr int GROUPS = D / 8;
    constexpr int ITEMS = (KEYS / 4) * GROUPS;
    const char* hbase = base + (int64_t)hk * nb2;
    for (int item = threadIdx.x; item < ITEMS; item += kThreads) {
        const int kq = item / GROUPS;
        const int grp = item - kq * GROUPS;
        f16x8 vals[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int key = 4 * kq + kk;
            const int j = j0 + key;
            if (j < M) {
                const char* rowp = hbase + (int64_t)j * nb1;
                const int off = (int)((uintptr_t)rowp & 15);
                vals[kk] = decode8<D>(rowp, type, grp, raw + key * Q8Row<D>::kSlot, off);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) vals[kk][t] = (_Float16)0.0f;
            }
            *(f16x8*)(dst + key * L::kLd + 8 * grp) = vals[kk];
        }
        if (TRANS) {
            const int pos = tpos(4 * kq);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f16x4 col = {vals[0][t], vals[1][t], vals[2][t], vals[3][t]};
                *(f16x4*)(dstT + (8 * grp + t) * L::kLdT + pos) = col;
            }
        }
    }
}

}  // namespace fab
