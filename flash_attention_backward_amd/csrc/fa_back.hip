// Host side of the flash-attention backward library: descriptor validation, output layout,
// workspace sizing, the plan, and the launch sequence. Device code is in fab_kernels.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "fa_back.h"
#include "fab_kernels.h"

using namespace fab;

namespace {

constexpr int kVmaxBlocks = 256;   // partial max |v| blocks of fa_back_run_saved

constexpr uint64_t kAlign = 256;

// The layout's CU count: fa_back_layout_query plans for a whole MI355X (256 compute units).
// The workspace holds the key side's split tail tiles for each CU count a gfx950 device (or
// partition of one) has, so it is a function of the descriptor only; a device with another
// count gets no tail split if its split would not fit.
constexpr int kRefCUs = 256;
constexpr int kLayoutCUs[] = {32, 64, 128, 256};
constexpr int kMaxW1Splits = 32;   // key-range splits of walk 1 by row tiles, at most

// Key-side tail tiles: one workgroup per CU at a time (LDS), so the tiles past the last full
// round of workgroups would run nearly alone; each of them is split into up to 4 row ranges.
// Returns the number of split tiles and sets *split to the ranges per tile (1 if none).
int tail_split(int T, int cus, int* split) {
    const int tail = T > cus ? T % cus : 0;
    const int sp = tail > 0 ? std::min(4, cus / tail) : 1;
    if (tail > 0 && tail <= cus / 2 && sp >= 2) {
        *split = sp;
        return tail;
    }
    *split = 1;
    return 0;
}

constexpr uint32_t kKnownFlags = FA_BACK_FLAG_CENTER_V | FA_BACK_FLAG_WALK1_KEYS | FA_BACK_FLAG_WALK1_ROWS |
                                  FA_BACK_FLAG_CENTER_K | FA_BACK_FLAG_KV_IMAGE | FA_BACK_FLAG_KV_INLINE |
                                  FA_BACK_FLAG_DS_STORE | FA_BACK_FLAG_DS_RECOMPUTE;
constexpr int kMaxDqSplits = 8;     // key-range splits of the dQ pass from stored dS, at most
constexpr uint64_t kMaxDsBytes = 16ull << 30;   // stored dS the plan takes without a flag, at most

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int64_t elem_size(int type) {
    switch (type) {
        case FA_BACK_F32: return 4;
        case FA_BACK_F16: return 2;
        case FA_BACK_BF16: return 2;
        case FA_BACK_Q8_0: return 34;   // one 32-value block
        case FA_BACK_Q4_0: return 18;   // one 32-value block
        case FA_BACK_Q4_1: return 20;
        case FA_BACK_Q5_0: return 22;
        case FA_BACK_Q5_1: return 24;
        default: return 0;
    }
}

bool is_block_kv(int type) {
    return type == FA_BACK_Q8_0 || type == FA_BACK_Q4_0 || type == FA_BACK_Q4_1 || type == FA_BACK_Q5_0 ||
           type == FA_BACK_Q5_1;
}

// Everything derived from a valid descriptor: shapes, plan choices, offsets.
struct Geometry {
    int cus;               // compute units the work split is planned for
    int D, Dv, H, Hkv, G, N, M, Hm;
    int R, RB, RT, KT, splits, tiles_per_split, KVT;
    int kv_full, kv_tail, kv_split;   // key side: unsplit tiles, split tiles, parts per split tile
    int64_t kv_parts_ws;              // split-tile parts the workspace holds (any planned CU count)
    bool w1keys;           // walk 1 by key tiles (else by row tiles)
    int KT1, RS1, w1_rbs;  // its 256-key tiles, row splits and row blocks per workgroup
    int w1_splits, w1_tps; // walk 1 by row tiles: key-range splits, 64-key tiles per split
    int nparts;            // walk-1 records per row
    int nparts_ws;         // walk-1 records per row the workspace holds (any planned CU count)
    bool img;              // the query-side walks copy K/V tiles from the decoded image
    int img_ns;            // its 32-key sub-tiles per KV head
    bool dss;              // dQ from the dS the key side stores (else walk 2 recomputes it)
    int ds_kb;             // 32-key blocks per row block and head in the stored dS
    int dq_splits_ws;      // dQ split partials the workspace holds
    int npart, nbound;
    fa_back_layout layout;
    // workspace offsets (bytes)
    uint64_t ws_absmax, ws_scal, ws_qr, ws_dr;
    uint64_t ws_rec, ws_lse2, ws_dlt, ws_rks, ws_bound, ws_dqp, ws_mcls, ws_kvp, ws_vmax;
    uint64_t ws_vcen;      // [Hkv][D] V centre (FA_BACK_FLAG_CENTER_V only)
    uint64_t ws_kcen;      // [Hkv][D] K centre (FA_BACK_FLAG_CENTER_K only)
    uint64_t ws_img;       // [Hkv][img_ns][32-key slot] decoded K/V tiles (img only)
    uint64_t ws_ds;        // [Hkv][RB][ds_kb][2048 bytes] stored dS tiles (dss only)
};

bool tensor_nonneg(const fa_back_tensor& t) {
    return t.ne[0] >= 0 && t.ne[1] >= 0 && t.ne[2] >= 0;
}

int check_strides(const fa_back_tensor& t, bool rows16) {
    const int64_t es = elem_size(t.type);
    if (t.nb[0] != es) return FA_BACK_ESTRIDE;
    if (t.nb[1] <= 0 || t.nb[2] <= 0) return FA_BACK_ESTRIDE;
    const int64_t a = rows16 ? 16 : (is_block_kv(t.type) ? 2 : es);
    if (t.nb[1] % a || t.nb[2] % a) return FA_BACK_ESTRIDE;
    return FA_BACK_OK;
}

// Validates `d` and plans the work for a device with `cus` compute units.
int validate(const fa_back_desc* d, int cus, Geometry* g) {
    if (!d) return FA_BACK_EINVAL;
    const fa_back_tensor &q = d->q, &k = d->k, &v = d->v, &dd = d->d, &m = d->mask;
    // types
    auto is_act = [](int t) { return t == FA_BACK_F32 || t == FA_BACK_F16 || t == FA_BACK_BF16; };
    auto is_kv = [&](int t) { return is_act(t) || is_block_kv(t); };
    auto is_blk = [](int t) { return is_block_kv(t); };
    if (!is_act(q.type) || !is_act(dd.type) || !is_kv(k.type) || !is_kv(v.type)) return FA_BACK_EUNSUPPORTED;
    const bool has_mask = m.type != FA_BACK_NONE;
    const bool causal = m.type == FA_BACK_CAUSAL_TAIL;   // implicit: no storage, no strides
    if (has_mask && !causal && m.type != FA_BACK_F32 && m.type != FA_BACK_F16) return FA_BACK_EUNSUPPORTED;
    if (!std::isfinite(d->scale)) return FA_BACK_EINVAL;
    if (d->flags & ~kKnownFlags) return FA_BACK_EINVAL;
    if ((d->flags & FA_BACK_FLAG_WALK1_KEYS) && (d->flags & FA_BACK_FLAG_WALK1_ROWS)) return FA_BACK_EINVAL;
    if ((d->flags & FA_BACK_FLAG_KV_IMAGE) && (d->flags & FA_BACK_FLAG_KV_INLINE)) return FA_BACK_EINVAL;
    if ((d->flags & FA_BACK_FLAG_DS_STORE) && (d->flags & FA_BACK_FLAG_DS_RECOMPUTE)) return FA_BACK_EINVAL;
    if ((d->flags & FA_BACK_FLAG_DS_STORE) && (d->flags & FA_BACK_FLAG_KV_INLINE)) return FA_BACK_EINVAL;
    if ((d->flags & FA_BACK_FLAG_CENTER_V) && is_blk(v.type)) return FA_BACK_EUNSUPPORTED;
    if ((d->flags & FA_BACK_FLAG_CENTER_K) && is_blk(k.type)) return FA_BACK_EUNSUPPORTED;
    if (!tensor_nonneg(q) || !tensor_nonneg(k) || !tensor_nonneg(v) || !tensor_nonneg(dd) ||
        (has_mask && !tensor_nonneg(m)))
        return FA_BACK_EINVAL;
    const int64_t D = q.ne[0], N = q.ne[1], H = q.ne[2];
    const int64_t M = k.ne[1], Hkv = k.ne[2], Dv = v.ne[0];
    if (D == 0 || H == 0 || Hkv == 0 || Dv == 0) return FA_BACK_EINVAL;
    // shapes
    if (k.ne[0] != D) return FA_BACK_ESHAPE;
    if (v.ne[1] != M || v.ne[2] != Hkv) return FA_BACK_ESHAPE;
    if (dd.ne[0] != Dv || dd.ne[1] != H || dd.ne[2] != N) return FA_BACK_ESHAPE;
    if (H % Hkv) return FA_BACK_ESHAPE;
    if (is_blk(k.type) && D % 32) return FA_BACK_ESHAPE;
    if (is_blk(v.type) && Dv % 32) return FA_BACK_ESHAPE;
    int64_t Hm = 0;
    if (has_mask) {
        if (m.ne[0] != M || m.ne[1] != N) return FA_BACK_ESHAPE;
        Hm = m.ne[2];
        if (Hm != 1 && Hm != H) return FA_BACK_ESHAPE;
        if (causal && Hm != 1) return FA_BACK_ESHAPE;
    }
    // strides: rows contiguous; F32/F16/BF16 cache rows are read with 16-byte loads
    int rc;
    if ((rc = check_strides(q, false)) || (rc = check_strides(dd, false))) return rc;
    if ((rc = check_strides(k, !is_blk(k.type))) || (rc = check_strides(v, !is_blk(v.type))))
        return rc;
    if (has_mask && !causal && (rc = check_strides(m, false))) return rc;
    if (k.nb[1] >= ((int64_t)1 << 32) || v.nb[1] >= ((int64_t)1 << 32)) return FA_BACK_EUNSUPPORTED;
    // supported sizes
    if (D != Dv || (D != 64 && D != 128 && D != 256)) return FA_BACK_EUNSUPPORTED;
    const int64_t G = H / Hkv;
    if (N * H >= (int64_t)1 << 30 || M * Hkv >= (int64_t)1 << 30 || G * N >= (int64_t)1 << 30 || H > 65535)
        return FA_BACK_EUNSUPPORTED;

    g->cus = cus;
    g->D = (int)D; g->Dv = (int)Dv; g->H = (int)H; g->Hkv = (int)Hkv; g->G = (int)G;
    g->N = (int)N; g->M = (int)M; g->Hm = (int)Hm;
    g->R = (int)(G * N);
    g->RB = (g->R + 31) / 32;
    g->RT = (g->RB + kWaves - 1) / kWaves;
    g->KT = (g->M + kQTileKeys - 1) / kQTileKeys;
    g->KVT = (g->M + kKVKeys - 1) / kKVKeys;
    // key side: the tail tiles are split (tail_split); a workgroup lists at most KVLds::kMaxRB
    // row blocks, so with more rows every tile is split into ranges of at most that many
    {
        const int T = g->KVT * (int)Hkv;
        const int pmin = (g->RB + KVLds<64>::kMaxRB - 1) / KVLds<64>::kMaxRB;
        if (pmin > 1) {
            g->kv_tail = T;
            g->kv_split = pmin;
            g->kv_parts_ws = (int64_t)T * pmin;
        } else {
            int64_t most = 0;
            for (int c : kLayoutCUs) {
                int sp;
                const int t = tail_split(T, c, &sp);
                most = std::max<int64_t>(most, (int64_t)t * sp);
            }
            g->kv_parts_ws = most;
            g->kv_tail = tail_split(T, cus, &g->kv_split);
            if ((int64_t)g->kv_tail * g->kv_split > most) {   // a CU count the layout does not plan for
                g->kv_tail = 0;
                g->kv_split = 1;
            }
        }
        g->kv_full = T - g->kv_tail;
    }
    // key-range splits of the query-side passes: aim for >= 512 workgroups (two per CU on
    // 256 CUs) but keep >= 4 key tiles per split so the dQ partials stay small
    {
        const int base = g->RT * g->Hkv;
        int splits = base > 0 ? (512 + base - 1) / base : 1;
        const int max_splits = g->KT >= 4 ? g->KT / 4 : 1;
        if (splits > max_splits) splits = max_splits;
        if (splits < 1) splits = 1;
        const int tps = g->KT > 0 ? (g->KT + splits - 1) / splits : 1;
        g->tiles_per_split = tps;
        g->splits = g->KT > 0 ? (g->KT + tps - 1) / tps : 1;
    }
    // the decoded image of the cache: when each sub-tile would be decoded by at least 4 row
    // tiles of the query-side walks (a flag forces either way)
    {
        bool img = g->RT >= 4;
        if (d->flags & FA_BACK_FLAG_KV_IMAGE) img = true;
        if (d->flags & FA_BACK_FLAG_KV_INLINE) img = false;
        // dQ from stored dS (it reads K from the image): by default whenever the image is used
        // and the tiles fit kMaxDsBytes; a flag forces either way
        const uint64_t ds_bytes = (uint64_t)Hkv * g->RB * (4ull * g->KVT) * 2048ull;
        bool dss = img && ds_bytes <= kMaxDsBytes;
        if (d->flags & FA_BACK_FLAG_DS_STORE) dss = true;
        if (d->flags & FA_BACK_FLAG_DS_RECOMPUTE) dss = false;
        g->dss = dss && g->M > 0 && g->R > 0;
        if (g->dss) img = true;
        g->img = img && g->M > 0 && g->R > 0;
        g->img_ns = (g->M + kSubKeys - 1) / kSubKeys;
        g->ds_kb = 4 * g->KVT;
        g->dq_splits_ws = g->splits;
        if (g->dss) {
            // the dQ pass's own key-range splits, for its workgroups of 256 rows: minimise rounds
            // of `cus` workgroups x (64-key tiles per split + 1), at most kMaxDqSplits
            const int kt = std::max(g->KT, 1);
            const int wgs = (g->RB + kQsWaves - 1) / kQsWaves * g->Hkv;
            const int sp_max = std::min(kMaxDqSplits, kt);
            double best_cost = 1e300;
            for (int sp = 1; sp <= sp_max; ++sp) {
                const int tps = (kt + sp - 1) / sp;
                const int n = (kt + tps - 1) / tps;
                const double cost = std::ceil((double)wgs * n / (double)cus) * (tps + 1.0);
                if (cost < best_cost - 1e-9) { best_cost = cost; g->splits = n; g->tiles_per_split = tps; }
            }
            g->dq_splits_ws = sp_max;   // the workspace does not depend on the CU count
        }
    }
    // walk 1 by key tiles when the cache is long next to the rows and not in the image (each
    // K/V tile is then decoded once per 256 keys instead of once per 128 rows); over the image
    // by row tiles of 256 rows, where all 8 waves form products; a flag picks the walk
    {
        g->KT1 = (g->M + kW1Keys - 1) / kW1Keys;
        bool keys = g->M >= 2 * (int64_t)g->R && !g->img;
        if (d->flags & FA_BACK_FLAG_WALK1_KEYS) keys = true;
        if (d->flags & FA_BACK_FLAG_WALK1_ROWS) keys = false;
        g->w1keys = keys && g->M > 0 && g->R > 0;
        g->RS1 = 1;
        g->w1_rbs = g->RB;
        if (g->w1keys) {
            // row splits: minimise rounds of `cus` workgroups x (setup + row blocks per
            // workgroup), the setup (decoding 256 keys) counted as 8 row blocks
            const int rs_min = (g->RB + W1Lds<64>::kMaxRB - 1) / W1Lds<64>::kMaxRB;
            int best = rs_min;
            double best_cost = 1e300;
            for (int rs = rs_min; rs <= 16; ++rs) {
                const int rbs = (g->RB + rs - 1) / rs;
                const double rounds = std::ceil((double)g->KT1 * g->Hkv * rs / (double)cus);
                const double cost = rounds * (8.0 + rbs);
                if (cost < best_cost - 1e-9) { best_cost = cost; best = rs; }
            }
            g->w1_rbs = (g->RB + best - 1) / best;
            g->RS1 = (g->RB + g->w1_rbs - 1) / g->w1_rbs;
        }
        // walk 1 by row tiles: its own key-range splits, chosen for its workgroups (256 rows
        // each over the image, else 128): minimise rounds of `cus` workgroups x (64-key tiles
        // per split + 1)
        const int rows_wg = g->img ? 8 : kWaves;
        const int wgs = ((g->RB + rows_wg - 1) / rows_wg) * g->Hkv;
        const int kt = std::max(g->KT, 1);
        const int sp_max = std::min(kMaxW1Splits, kt);
        double best_cost = 1e300;
        g->w1_splits = 1;
        g->w1_tps = kt;
        for (int sp = 1; sp <= sp_max; ++sp) {
            const int tps = (kt + sp - 1) / sp;
            const int n = (kt + tps - 1) / tps;
            const double cost = std::ceil((double)wgs * n / (double)cus) * (tps + 1.0);
            if (cost < best_cost - 1e-9) { best_cost = cost; g->w1_splits = n; g->w1_tps = tps; }
        }
        g->nparts = g->w1keys ? g->KT1 : g->w1_splits;
        // the records the workspace holds do not depend on the CU count (the most splits allowed)
        g->nparts_ws = g->w1keys ? g->KT1 : sp_max;
    }
    g->npart = (int)std::min<int64_t>(512, std::max<int64_t>(1, N * H / 8));
    const int64_t total_rows = (int64_t)g->Hkv * g->RB * 32;
    g->nbound = (int)std::min<int64_t>(kMergeMaxBlocks, std::max<int64_t>(1, (g->RB * 32 + kMergeRows - 1) / kMergeRows));

    // packed output
    fa_back_layout& L = g->layout;
    L.off_dq = 0;
    L.off_dk = align_up(L.off_dq + 4ull * D * N * H, kAlign);
    L.off_dv = align_up(L.off_dk + 4ull * D * M * Hkv, kAlign);
    L.off_lse = align_up(L.off_dv + 4ull * Dv * M * Hkv, kAlign);
    L.off_delta = L.off_lse + 4ull * N * H;
    L.out_bytes = std::max<uint64_t>(align_up(L.off_delta + 4ull * N * H, kAlign), kAlign);
    // workspace
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) { const uint64_t at = o; o = align_up(o + bytes, kAlign); return at; };
    const uint64_t frag = 2ull * total_rows * D;
    const uint64_t prow = (uint64_t)std::max(g->nparts, g->nparts_ws) * total_rows;
    g->ws_absmax = take(8ull * g->npart);
    g->ws_scal = take(64);
    g->ws_qr = take(frag);
    g->ws_dr = take(frag);
    g->ws_rec = take(16 * prow);
    g->ws_lse2 = take(4ull * total_rows);
    g->ws_dlt = take(4ull * total_rows);
    g->ws_rks = take(4ull * total_rows);
    g->ws_bound = take(4ull * g->nbound * g->Hkv);
    g->ws_dqp = take(g->dq_splits_ws > 1 ? 4ull * g->dq_splits_ws * total_rows * D : 0);
    // mask classes: stored masks only (the causal-tail classes are computed where needed)
    const bool stored_mask = has_mask && d->mask.type != FA_BACK_CAUSAL_TAIL;
    g->ws_mcls = take(stored_mask ? (uint64_t)(Hm == 1 ? 1 : g->Hkv) * g->RB * g->KT : 0);
    g->ws_kvp = take(4ull * g->kv_parts_ws * 2 * kKVKeys * D);
    g->ws_vmax = take(4ull * kVmaxBlocks);   // fa_back_run_saved only
    g->ws_vcen = take((d->flags & FA_BACK_FLAG_CENTER_V) ? 4ull * g->Hkv * D : 0);
    g->ws_kcen = take((d->flags & FA_BACK_FLAG_CENTER_K) ? 4ull * g->Hkv * D : 0);
    g->ws_img = take(g->img ? (uint64_t)g->Hkv * g->img_ns * (uint64_t)(4 * kSubKeys * D) : 0);
    g->ws_ds = take(g->dss ? (uint64_t)g->Hkv * g->RB * g->ds_kb * 2048ull : 0);
    L.workspace_bytes = std::max<uint64_t>(o, kAlign);
    L.plan_flags = d->flags & (FA_BACK_FLAG_CENTER_V | FA_BACK_FLAG_CENTER_K);
    if (g->M > 0 && g->R > 0) {
        L.plan_flags |= g->w1keys ? FA_BACK_FLAG_WALK1_KEYS : FA_BACK_FLAG_WALK1_ROWS;
        L.plan_flags |= g->img ? FA_BACK_FLAG_KV_IMAGE : FA_BACK_FLAG_KV_INLINE;
        L.plan_flags |= g->dss ? FA_BACK_FLAG_DS_STORE : FA_BACK_FLAG_DS_RECOMPUTE;
    }
    return FA_BACK_OK;
}

// Static LDS of the largest tile kernel for head size D (the tile kernels use 1 workgroup
// per CU; the small kernels use a few KB).
template <int D>
int max_lds_bytes_d() {
    return std::max(std::max(std::max(QLds<D>::kBytes, QLds<D, true>::kBytes), W1Lds<D>::kBytes),
                    std::max(std::max(KVLds<D>::kBytes, R1Lds<D>::kBytes), QsLds<D>::kBytes));
}
int max_lds_bytes(int D) {
    return D == 64 ? max_lds_bytes_d<64>() : D == 128 ? max_lds_bytes_d<128>() : max_lds_bytes_d<256>();
}

// Records an event after each phase when `ev` is non-NULL (ev[0] is recorded by the caller
// before the first phase). Phases: absmax, prep, walk 1, merge, walk 2, dQ reduce, key side.
struct PhaseMarks {
    hipEvent_t* ev;        // 2 per phase: its start and its end
    hipStream_t st;
    void begin(int phase) const {
        if (ev) (void)hipEventRecord(ev[2 * phase], st);
    }
    void end(int phase) const {
        if (ev) (void)hipEventRecord(ev[2 * phase + 1], st);
    }
};

// The query-side walk, in the instantiation of the K/V decode the types need.
template <int D, bool GRAD>
void launch_qpass(const Geometry& g, const Params& P, hipStream_t st) {
    if (!GRAD && P.kvimg) {
        // walk 1 over the image: every wave owns rows
        const dim3 grid1((g.RB + kR1Waves - 1) / kR1Waves * g.Hkv, g.w1_splits);
        hipLaunchKernelGGL(walk1_rows_kernel<D>, grid1, dim3(kR1Threads), 0, st, P);
        return;
    }
    const dim3 grid(g.RT * g.Hkv, GRAD ? g.splits : g.w1_splits), block(kQThreads);
    // the pair decode covers q8_0 and q4_0; the other block types take the general decode
    const bool blk_k = P.k_type == FA_BACK_Q8_0 || P.k_type == FA_BACK_Q4_0;
    const bool blk_v = P.v_type == FA_BACK_Q8_0 || P.v_type == FA_BACK_Q4_0;
    if (GRAD && P.kvimg)
        hipLaunchKernelGGL((qpass_kernel<D, true, kDecImg>), grid, block, 0, st, P);
    else if (P.k_type == FA_BACK_Q8_0 && P.v_type == FA_BACK_Q8_0)
        hipLaunchKernelGGL((qpass_kernel<D, GRAD, kDecQ8>), grid, block, 0, st, P);
    else if (blk_k && blk_v)
        hipLaunchKernelGGL((qpass_kernel<D, GRAD, kDecBlk>), grid, block, 0, st, P);
    else
        hipLaunchKernelGGL((qpass_kernel<D, GRAD, kDecGen>), grid, block, 0, st, P);
}

// The decoded image of the cache, in the decode the types need.
template <int D>
void launch_kvimage(const Geometry& g, const Params& P, hipStream_t st) {
    const dim3 grid(g.img_ns, g.Hkv), block(kImgThreads);
    // the pair decode covers q8_0 and q4_0; the other block types take the general decode
    const bool blk_k = P.k_type == FA_BACK_Q8_0 || P.k_type == FA_BACK_Q4_0;
    const bool blk_v = P.v_type == FA_BACK_Q8_0 || P.v_type == FA_BACK_Q4_0;
    if (P.k_type == FA_BACK_Q8_0 && P.v_type == FA_BACK_Q8_0)
        hipLaunchKernelGGL((kvimage_kernel<D, kDecQ8>), grid, block, 0, st, P);
    else if (blk_k && blk_v)
        hipLaunchKernelGGL((kvimage_kernel<D, kDecBlk>), grid, block, 0, st, P);
    else
        hipLaunchKernelGGL((kvimage_kernel<D, kDecGen>), grid, block, 0, st, P);
}

template <int D>
int launch_all(const Geometry& g, Params& P, hipStream_t st, const PhaseMarks& pm) {
    if (g.N == 0 || g.M == 0) {
        // degenerate: zero dK, dV (N == 0) or every row fully masked (M == 0)
        pm.begin(0);
        const int64_t nk = (int64_t)g.D * g.M * g.Hkv;
        if (nk) hipLaunchKernelGGL(fill_kernel, dim3(256), dim3(kThreads), 0, st, P.dk, nk, 0.0f);
        if (nk) hipLaunchKernelGGL(fill_kernel, dim3(256), dim3(kThreads), 0, st, P.dv, nk, 0.0f);
        const int64_t nq = (int64_t)g.D * g.N * g.H;
        if (nq) hipLaunchKernelGGL(fill_kernel, dim3(256), dim3(kThreads), 0, st, P.dq, nq, 0.0f);
        const int64_t nr = (int64_t)g.N * g.H;
        if (nr) hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(kThreads), 0, st, P.lse, nr, -INFINITY);
        if (nr) hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(kThreads), 0, st, P.delta, nr, 0.0f);
        pm.end(0);
        for (int ph = 1; ph < FA_BACK_NUM_PHASES; ++ph) {
            pm.begin(ph);
            pm.end(ph);
        }
        return hipGetLastError() == hipSuccess ? FA_BACK_OK : FA_BACK_EHIP;
    }
    pm.begin(0);
    hipLaunchKernelGGL(absmax_kernel, dim3(g.npart), dim3(kThreads), 0, st, P);
    if (P.vcen) hipLaunchKernelGGL(centre_kernel<false>, dim3(g.Hkv), dim3(kThreads), 0, st, P);
    if (P.kcen) hipLaunchKernelGGL(centre_kernel<true>, dim3(g.Hkv), dim3(kThreads), 0, st, P);
    pm.end(0);
    pm.begin(1);
    hipLaunchKernelGGL(prep_kernel<D>, dim3(g.Hkv * g.RB), dim3(kThreads), 0, st, P);
    if (g.Hm > 0 && P.m_type != FA_BACK_CAUSAL_TAIL) {
        const dim3 grid((g.Hm == 1 ? 1 : g.Hkv) * g.RB, (g.KT + kClassTilesPerBlock - 1) / kClassTilesPerBlock);
        if (g.Hm == 1) {
            // one mask head: each distinct query row of a row block is read once
            if (P.m_type == FA_BACK_F16)
                hipLaunchKernelGGL(maskclass_rows_kernel<2>, grid, dim3(kThreads), 0, st, P);
            else
                hipLaunchKernelGGL(maskclass_rows_kernel<4>, grid, dim3(kThreads), 0, st, P);
        } else if (P.m_type == FA_BACK_F16) {
            hipLaunchKernelGGL(maskclass_kernel<2>, grid, dim3(kThreads), 0, st, P);
        } else {
            hipLaunchKernelGGL(maskclass_kernel<4>, grid, dim3(kThreads), 0, st, P);
        }
    }
    if (P.kvimg) launch_kvimage<D>(g, P, st);
    pm.end(1);
    if (P.lse_in) {
        // forward-saved LSE and O: the row statistics without walk 1 and the merge
        pm.begin(2);
        hipLaunchKernelGGL(vmax_kernel, dim3(kVmaxBlocks), dim3(kThreads), 0, st, P);
        pm.end(2);
        pm.begin(3);
        hipLaunchKernelGGL(saved_rows_kernel, dim3(g.nbound, g.Hkv), dim3(kThreads), 0, st, P);
        pm.end(3);
    } else {
        pm.begin(2);
        if (g.w1keys)
            hipLaunchKernelGGL(walk1_keys_kernel<D>, dim3(g.KT1 * g.Hkv, g.RS1), dim3(kW1Threads), 0, st, P);
        else
            launch_qpass<D, false>(g, P, st);
        pm.end(2);
        pm.begin(3);
        hipLaunchKernelGGL(merge_kernel, dim3(g.nbound, g.Hkv), dim3(kThreads), 0, st, P);
        if (P.vcen || P.kcen) {
            // the merge wrote delta - dO . c (V centred) and lse - scale q . c (K centred)
            const int64_t rows = (int64_t)g.H * g.N;
            const int blocks = (int)std::min<int64_t>(4096, (rows + kWaves - 1) / kWaves);
            hipLaunchKernelGGL(centre_out_kernel, dim3(blocks), dim3(kThreads), 0, st, P);
        }
        pm.end(3);
    }
    auto dq_reduce = [&]() {
        pm.begin(5);
        if (g.splits > 1) {
            const int64_t n4 = (int64_t)g.Hkv * g.RB * 32 * (D / 4);
            const int blocks = (int)std::min<int64_t>(65536, (n4 + kDqThreads - 1) / kDqThreads);
            hipLaunchKernelGGL(dqreduce_kernel<D>, dim3(blocks), dim3(kDqThreads), 0, st, P);
        }
        pm.end(5);
    };
    if (!g.dss) {
        pm.begin(4);
        launch_qpass<D, true>(g, P, st);
        pm.end(4);
        dq_reduce();
    }
    pm.begin(6);
    const dim3 kvgrid(g.kv_full + g.kv_tail * g.kv_split);
    if (g.dss)
        hipLaunchKernelGGL((kvpass_kernel<D, true>), kvgrid, dim3(kKVThreads), 0, st, P);
    else
        hipLaunchKernelGGL((kvpass_kernel<D, false>), kvgrid, dim3(kKVThreads), 0, st, P);
    if (g.kv_tail) {
        const int64_t n4 = (int64_t)g.kv_tail * 2 * kKVKeys * (D / 4);
        const int blocks = (int)std::min<int64_t>(2048, (n4 + kThreads - 1) / kThreads);
        hipLaunchKernelGGL(kvreduce_kernel<D>, dim3(blocks), dim3(kThreads), 0, st, P, g.kv_tail);
    }
    pm.end(6);
    if (g.dss) {
        // dQ from the dS tiles the key side stored
        pm.begin(4);
        const dim3 grid((g.RB + kQsWaves - 1) / kQsWaves * g.Hkv, g.splits);
        hipLaunchKernelGGL(dq_stored_kernel<D>, grid, dim3(kQsThreads), 0, st, P);
        pm.end(4);
        dq_reduce();
    }
    return hipGetLastError() == hipSuccess ? FA_BACK_OK : FA_BACK_EHIP;
}

// Workspace for fa_back_run_noalloc: a static device array, one copy per GPU the library runs
// on, held until the process ends. In host code `scratch` only names the symbol; the device
// address of each GPU's copy comes from hipGetSymbolAddress with that GPU current, and only
// that address is handed to kernels.
constexpr uint64_t kScratchBytes = 64ull << 20;
static_assert(kScratchBytes == FA_BACK_NOALLOC_MAX_WORKSPACE, "header and library disagree");
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The address of this device's `scratch` (the device must be current). nullptr on failure.
void* scratch_address(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[device] = ptr;
    }
    return g_scratch_ptr[device];
}

}  // namespace

struct fa_back_plan {
    fa_back_desc desc;
    Geometry geo;
    int device;
    void* scratch;   // this device's static scratch (fa_back_run_noalloc), or nullptr
};

extern "C" {

const char* fa_back_status_string(int s) {
    switch (s) {
        case FA_BACK_OK: return "ok";
        case FA_BACK_EINVAL: return "invalid argument";
        case FA_BACK_ESHAPE: return "inconsistent shapes";
        case FA_BACK_ESTRIDE: return "unsupported strides";
        case FA_BACK_EUNSUPPORTED: return "unsupported type, size or device";
        case FA_BACK_EHIP: return "HIP runtime error";
        case FA_BACK_EALIGN: return "misaligned device pointer";
        case FA_BACK_ESCRATCH: return "workspace larger than the static scratch of fa_back_run_noalloc";
        default: return "unknown status";
    }
}

int fa_back_layout_query(const fa_back_desc* desc, fa_back_layout* layout) {
    if (!layout) return FA_BACK_EINVAL;
    Geometry g;
    const int rc = validate(desc, kRefCUs, &g);
    if (rc == FA_BACK_OK) *layout = g.layout;
    return rc;
}

int fa_back_create(const fa_back_desc* desc, int device, fa_back_plan** plan, fa_back_layout* layout) {
    if (!plan) return FA_BACK_EINVAL;
    *plan = nullptr;
    Geometry g;
    int rc = validate(desc, kRefCUs, &g);   // descriptor errors before any device call
    if (rc != FA_BACK_OK) return rc;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return FA_BACK_EUNSUPPORTED;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return FA_BACK_EHIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return FA_BACK_EUNSUPPORTED;
    if ((size_t)max_lds_bytes(g.D) > prop.sharedMemPerBlock) return FA_BACK_EUNSUPPORTED;
    if (prop.multiProcessorCount < 1) return FA_BACK_EUNSUPPORTED;
    rc = validate(desc, prop.multiProcessorCount, &g);
    if (rc != FA_BACK_OK) return rc;
    // the device's copy of the static scratch (fa_back_run_noalloc), looked up with it current
    void* scr = nullptr;
    {
        int old = -1;
        if (hipGetDevice(&old) != hipSuccess) return FA_BACK_EHIP;
        if (old != device && hipSetDevice(device) != hipSuccess) return FA_BACK_EHIP;
        scr = scratch_address(device);
        if (old != device) (void)hipSetDevice(old);
        if (!scr) return FA_BACK_EHIP;
    }
    fa_back_plan* p = new (std::nothrow) fa_back_plan;
    if (!p) return FA_BACK_EINVAL;
    p->desc = *desc;
    p->geo = g;
    p->device = device;
    p->scratch = scr;
    *plan = p;
    if (layout) *layout = g.layout;
    return FA_BACK_OK;
}

void fa_back_destroy(fa_back_plan* plan) { delete plan; }

static int run_impl(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                    const void* d, const void* mask, const float* lse_in, const float* o_in, bool saved,
                    void* out, void* workspace, void* stream, float* phase_ms) {
    if (!plan || !out || !workspace) return FA_BACK_EINVAL;
    const fa_back_desc& ds = plan->desc;
    const Geometry& g = plan->geo;
    // a tensor without elements may be passed as NULL
    const bool q_empty = (int64_t)g.N * g.H == 0, kv_empty = (int64_t)g.M == 0;
    if ((!q && !q_empty) || (!d && !q_empty) || (!k && !kv_empty) || (!v && !kv_empty)) return FA_BACK_EINVAL;
    if (saved && (!lse_in || !o_in) && !q_empty) return FA_BACK_EINVAL;
    const bool causal = ds.mask.type == FA_BACK_CAUSAL_TAIL;
    const bool has_mask = ds.mask.type != FA_BACK_NONE && !causal;   // a stored mask
    if (!has_mask && mask) return FA_BACK_EINVAL;
    if (has_mask && !mask && (int64_t)g.M * g.N != 0) return FA_BACK_EINVAL;
    auto misaligned = [](const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) != 0; };
    auto kv_align = [](int t) -> uintptr_t { return is_block_kv(t) ? 2 : 16; };
    if (misaligned(q, elem_size(ds.q.type)) || misaligned(d, elem_size(ds.d.type)) ||
        misaligned(k, kv_align(ds.k.type)) || misaligned(v, kv_align(ds.v.type)) ||
        (has_mask && misaligned(mask, elem_size(ds.mask.type))) || misaligned(out, kAlign) ||
        (saved && (misaligned(lse_in, 4) || misaligned(o_in, 4))) ||
        misaligned(workspace, kAlign))
        return FA_BACK_EALIGN;

    int old = -1;
    if (hipGetDevice(&old) != hipSuccess) return FA_BACK_EHIP;
    if (old != plan->device && hipSetDevice(plan->device) != hipSuccess) return FA_BACK_EHIP;
    (void)hipGetLastError();   // clear a stale error so the check below sees only ours

    Params P;
    std::memset(&P, 0, sizeof(P));
    P.q = (const char*)q; P.k = (const char*)k; P.v = (const char*)v; P.d = (const char*)d;
    P.mask = (const char*)mask;
    P.q_nb0 = ds.q.nb[0]; P.q_nb1 = ds.q.nb[1]; P.q_nb2 = ds.q.nb[2];
    P.d_nb0 = ds.d.nb[0]; P.d_nb1 = ds.d.nb[1]; P.d_nb2 = ds.d.nb[2];
    P.k_nb1 = ds.k.nb[1]; P.k_nb2 = ds.k.nb[2];
    P.v_nb1 = ds.v.nb[1]; P.v_nb2 = ds.v.nb[2];
    if (!causal) { P.m_nb0 = ds.mask.nb[0]; P.m_nb1 = ds.mask.nb[1]; P.m_nb2 = ds.mask.nb[2]; }
    P.q_type = ds.q.type; P.d_type = ds.d.type; P.k_type = ds.k.type; P.v_type = ds.v.type;
    P.m_type = ds.mask.type;
    P.D = g.D; P.H = g.H; P.Hkv = g.Hkv; P.G = g.G; P.N = g.N; P.M = g.M; P.Hm = g.Hm;
    P.R = g.R; P.RB = g.RB; P.RT = g.RT; P.KT = g.KT; P.splits = g.splits;
    P.tiles_per_split = g.tiles_per_split; P.KVT = g.KVT;
    P.w1_rbs = g.w1_rbs; P.w1_tps = g.w1_tps; P.nparts = g.nparts;
    P.scale = ds.scale;
    char* o = (char*)out;
    P.dq = (float*)(o + g.layout.off_dq);
    P.dk = (float*)(o + g.layout.off_dk);
    P.dv = (float*)(o + g.layout.off_dv);
    P.lse = (float*)(o + g.layout.off_lse);
    P.delta = (float*)(o + g.layout.off_delta);
    char* w = (char*)workspace;
    P.absmax_part = (float*)(w + g.ws_absmax);
    P.npart = g.npart;
    P.scal = (int*)(w + g.ws_scal);
    P.qr = (_Float16*)(w + g.ws_qr);
    P.dr = (_Float16*)(w + g.ws_dr);
    P.part_rec = (f32x4*)(w + g.ws_rec);
    P.row_ks = (int*)(w + g.ws_rks);
    P.row_lse2 = (float*)(w + g.ws_lse2);
    P.row_dlt = (float*)(w + g.ws_dlt);
    P.bound_part = (float*)(w + g.ws_bound);
    P.nbound = g.nbound;
    P.dq_part = (float*)(w + g.ws_dqp);
    P.mcls = (unsigned char*)(w + g.ws_mcls);
    P.kv_full = g.kv_full;
    P.kv_split = g.kv_split;
    P.kv_part = (float*)(w + g.ws_kvp);
    if (ds.flags & FA_BACK_FLAG_CENTER_V) P.vcen = (float*)(w + g.ws_vcen);
    if (ds.flags & FA_BACK_FLAG_CENTER_K) P.kcen = (float*)(w + g.ws_kcen);
    if (g.img) {
        P.kvimg = (unsigned char*)(w + g.ws_img);
        P.img_ns = g.img_ns;
    }
    if (g.dss) {
        P.dsbuf = (_Float16*)(w + g.ws_ds);
        P.ds_kb = g.ds_kb;
    }
    if (saved && !q_empty) {
        P.lse_in = lse_in;
        P.o_in = o_in;
        P.vmax_part = (float*)(w + g.ws_vmax);
        P.nvpart = kVmaxBlocks;
    }

    hipStream_t st = (hipStream_t)stream;
    hipEvent_t ev[2 * FA_BACK_NUM_PHASES];
    int nev = 0;
    PhaseMarks pm{nullptr, st};
    int rc = FA_BACK_OK;
    if (phase_ms) {
        for (; nev < 2 * FA_BACK_NUM_PHASES; ++nev)
            if (hipEventCreate(&ev[nev]) != hipSuccess) { rc = FA_BACK_EHIP; break; }
        pm.ev = ev;
    }
    if (rc == FA_BACK_OK) {
        switch (g.D) {
            case 64: rc = launch_all<64>(g, P, st, pm); break;
            case 128: rc = launch_all<128>(g, P, st, pm); break;
            case 256: rc = launch_all<256>(g, P, st, pm); break;
            default: rc = FA_BACK_EUNSUPPORTED;
        }
    }
    if (phase_ms && rc == FA_BACK_OK) {
        // every phase recorded its start and end events on the stream
        for (int e = 0; rc == FA_BACK_OK && e < 2 * FA_BACK_NUM_PHASES; ++e)
            if (hipEventSynchronize(ev[e]) != hipSuccess) rc = FA_BACK_EHIP;
        for (int ph = 0; rc == FA_BACK_OK && ph < FA_BACK_NUM_PHASES; ++ph)
            if (hipEventElapsedTime(&phase_ms[ph], ev[2 * ph], ev[2 * ph + 1]) != hipSuccess) rc = FA_BACK_EHIP;
    }
    for (int e = 0; e < nev; ++e) (void)hipEventDestroy(ev[e]);
    if (old != plan->device) (void)hipSetDevice(old);
    return rc;
}

int fa_back_run(const fa_back_plan* plan, const void* q, const void* k, const void* v, const void* d,
                const void* mask, void* out, void* workspace, void* stream) {
    return run_impl(plan, q, k, v, d, mask, nullptr, nullptr, false, out, workspace, stream, nullptr);
}

int fa_back_run_timed(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                      const void* d, const void* mask, void* out, void* workspace, void* stream,
                      float* phase_ms) {
    if (!phase_ms) return FA_BACK_EINVAL;
    return run_impl(plan, q, k, v, d, mask, nullptr, nullptr, false, out, workspace, stream, phase_ms);
}

int fa_back_run_saved(const fa_back_plan* plan, const void* q, const void* k, const void* v, const void* d,
                      const void* mask, const float* lse, const float* o, void* out, void* workspace,
                      void* stream) {
    return run_impl(plan, q, k, v, d, mask, lse, o, true, out, workspace, stream, nullptr);
}

int fa_back_run_noalloc(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                        const void* d, const void* mask, void* out, void* stream) {
    if (!plan) return FA_BACK_EINVAL;
    if (plan->geo.layout.workspace_bytes > kScratchBytes) return FA_BACK_ESCRATCH;
    if (!plan->scratch) return FA_BACK_EHIP;
    return run_impl(plan, q, k, v, d, mask, nullptr, nullptr, false, out, plan->scratch, stream, nullptr);
}

int fa_back_run_saved_timed(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                            const void* d, const void* mask, const float* lse, const float* o, void* out,
                            void* workspace, void* stream, float* phase_ms) {
    if (!phase_ms) return FA_BACK_EINVAL;
    return run_impl(plan, q, k, v, d, mask, lse, o, true, out, workspace, stream, phase_ms);
}

}  // extern "C"
