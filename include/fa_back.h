/*
 * fa_back.h -- flash-attention backward (FLASH_ATTN_BACK) on AMD Instinct MI355X (gfx950).
 *
 * The operation (page "CambrianTech/llama.cpp PR #63", first review, "The math in
 * fattn_back_q" and "The math in fattn_back_kv"): for query heads h with KV head
 * hk = h / (H / Hkv), query rows i and keys j,
 *     s_ij    = scale * q_i . k_j + mask[j, i, h % Hm]          (mask optional)
 *     lse_i   = log sum_j exp(s_ij)                              (-inf if every s_ij = -inf)
 *     p_ij    = exp(s_ij - lse_i)                                (0 on a fully masked row)
 *     dp_ij   = dO_i . v_j
 *     delta_i = sum_j p_ij dp_ij          ( = rowsum(dO o O), O is never formed )
 *     dS_ij   = p_ij (dp_ij - delta_i)
 *     dQ_i    = scale * sum_j dS_ij k_j
 *     dK_j    = scale * sum_{h in group(hk), i} dS_ij q_i
 *     dV_j    =         sum_{h in group(hk), i} p_ij dO_i
 * The N x M score matrix is never stored and the K/V cache is never converted as a whole:
 * each K/V tile is decoded once per workgroup into on-chip memory.
 *
 * Tensors are described ggml-style: ne[] are extents innermost first, nb[] byte strides.
 *     q    ne = {D,  N, H  }   F32 | F16 | BF16
 *     k    ne = {D,  M, Hkv}   F32 | F16 | BF16 | Q8_0 | Q4_0 | Q4_1 | Q5_0 | Q5_1
 *     v    ne = {Dv, M, Hkv}   the same types (K and V types independent)
 *     d    ne = {Dv, H, N  }   F32 | F16 | BF16          (dO; note the H, N order, as the
 *                                                         operator's "Layout and shape" states)
 *     mask ne = {M,  N, Hm }   F32 | F16, Hm in {1, H}; type FA_BACK_NONE for no mask;
 *                              type FA_BACK_CAUSAL_TAIL for the causal-tail mask without
 *                              storage: ne = {M, N, 1}, nb ignored, and fa_back_run takes
 *                              mask = NULL. Query row i then sees keys j <= M - N + i (mask
 *                              entry 0) and no others (-inf), for every head: the results are
 *                              bitwise those of the same mask stored as F16 or F32.
 * nb[0] must equal the element size (34 bytes per 32-value block for Q8_0), i.e. each row
 * is contiguous; rows and heads may have any positive stride (e.g. a cache view whose heads
 * are interleaved per cell). A Q8_0 block is a little-endian fp16 scale followed by 32 int8;
 * its value is scale * int8. A Q4_0 block (18 bytes, nb[0] = 18) is a little-endian fp16
 * scale followed by 16 bytes; byte t holds element t in its low nibble and element t + 16 in
 * its high nibble, and an element's value is scale * (nibble - 8) (the ggml q4_0 block, the
 * format of the served cache on the "torad-labs/llama.cpp PR #71" page). The other ggml block
 * types (the pages name none of them; every field little-endian, 16 bytes of nibbles laid
 * out as in Q4_0, code t = nibble t plus 16 times bit t of the word h where there is one):
 *     Q4_1 (20 bytes): fp16 d, fp16 m, nibbles;           value = d * nibble + m
 *     Q5_0 (22 bytes): fp16 d, 32-bit h, nibbles;         value = d * (code - 16)
 *     Q5_1 (24 bytes): fp16 d, fp16 m, 32-bit h, nibbles; value = d * code + m
 * A block value is formed in fp32 and rounded once to fp16, as an F32 cache holding that fp32
 * value would be.
 *
 * Output: one packed F32 buffer, laid out as the operator's packed result (first review,
 * "Layout and shape"; second review, output index):
 *     dQ    at off_dq    [D,  N, H  ]  element (c, i, h)  at ((h*N + i)*D + c)
 *     dK    at off_dk    [D,  M, Hkv]  element (c, j, hk) at ((hk*M + j)*D + c)
 *     dV    at off_dv    [Dv, M, Hkv]  element (c, j, hk) at ((hk*M + j)*Dv + c)
 *     LSE   at off_lse   N*H floats, row h*N + i (natural log; -inf for a fully masked row)
 *     delta at off_delta = off_lse + 4*N*H bytes, N*H floats, row h*N + i
 * Regions start 256-byte aligned (except delta, which directly follows LSE); bytes between
 * regions are unspecified. Every defined byte is written by every run.
 *
 * Numerics: every product runs on fp16 MFMA with fp32 accumulation; Q and dO are scaled by
 * exact powers of two before rounding to fp16, P by 2^15 and dS by a power of two derived
 * from the data, and all scaling is undone exactly in fp32. The per-row softmax sums and
 * delta are carried across key tiles in fp64. K and V values must lie within fp16 range
 * (|x| < 65504). Inputs holding NaN or +-inf (other than -inf mask entries) give undefined
 * results. Results are bitwise reproducible for the same inputs and device type: every
 * output element has exactly one writer and every reduction runs in a fixed order; no
 * atomics are used.
 *
 * Supported: D == Dv in {64, 128, 256}; H % Hkv == 0; N, M >= 0 (N == 0: dK = dV = 0;
 * M == 0: every row is fully masked); F32/F16/BF16 K or V rows 16-byte aligned (base and
 * strides); block-type rows 2-byte aligned; K and V row strides (nb[1]) below 2^32 bytes.
 */
#ifndef FA_BACK_H
#define FA_BACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define FA_BACK_NONE (-1)
#define FA_BACK_F32 0
#define FA_BACK_F16 1
#define FA_BACK_BF16 2
#define FA_BACK_Q8_0 8
#define FA_BACK_Q4_0 9
#define FA_BACK_Q4_1 10
#define FA_BACK_Q5_0 11
#define FA_BACK_Q5_1 12
#define FA_BACK_CAUSAL_TAIL 16 /* mask only: query i sees keys j <= M - N + i; no storage */

/* Flags (fa_back_desc.flags; 0 = the plain operator).
 *
 * FA_BACK_FLAG_CENTER_V: for caches whose V rows differ in their low bits only (near-constant
 * V: the case the second review of "CambrianTech/llama.cpp PR #63" added to its oracle cases,
 * "compensated products", and that its fused revision keeps under the 1e-5 bar). The products
 * round V to fp16, which keeps about 11 significant bits; dS = P o (dP - delta) then cancels
 * the part that all keys share, and what is left is mostly rounding. With the flag, a
 * constant c[hk][c'] (the mean of the first 256 keys of each KV head and column) is taken from
 * V before the rounding. For every row P sums to 1, so dP - delta, and with it dS, dQ, dK and
 * dV, are unchanged in exact arithmetic; only the rounding now falls on V - c. The delta
 * output is delta' + dO . c, with dO . c formed in fp64. V must be F32, F16 or BF16
 * (FA_BACK_EUNSUPPORTED for the block types). Costs: one pass over 256 keys of V and one over dO,
 * and one subtraction per decoded V value. Bits other than the FA_BACK_FLAG_* below are
 * FA_BACK_EINVAL. */
#define FA_BACK_FLAG_CENTER_V 1u

/* FA_BACK_FLAG_WALK1_KEYS, FA_BACK_FLAG_WALK1_ROWS: which way the pass that forms each row's
 * LSE and delta walks the problem. Both give results that meet the same bar; they differ in
 * speed only. With neither bit the plan takes the row-owned walk when the cache is decoded into
 * the image (FA_BACK_FLAG_KV_IMAGE below), else the key-owned walk when the cache is long next
 * to the rows (M >= 2 * G * N, G = H / Hkv), else the row-owned walk. WALK1_KEYS forces the
 * key-owned walk (each K/V tile decoded once per 256 keys, one statistics record per row and
 * 256-key tile), WALK1_ROWS the row-owned one (row tiles walk the keys, one record per row and
 * key-range split, at most 32 splits; over the image, tiles of 256 rows copy each 32-key tile
 * once). Setting both is FA_BACK_EINVAL. The choice changes the workspace size: pass the same
 * flags to fa_back_layout_query and fa_back_create. */
#define FA_BACK_FLAG_WALK1_KEYS 2u
#define FA_BACK_FLAG_WALK1_ROWS 4u

/* FA_BACK_FLAG_CENTER_K: for caches whose K rows differ in their low bits only (near-constant
 * K). A per-(KV head, column) constant c (the mean of the first 256 keys) is taken from K
 * before its fp16 rounding. For query row i, every score then moves by the same amount
 * scale * q_i . c, which the softmax does not see: P, dP, dS and dK are unchanged in exact
 * arithmetic, and so is dQ = scale * sum_j dS_ij (k_j - c), because sum_j dS_ij = 0 on every
 * row. The LSE output is the centred row's LSE plus scale * q_i . c, formed in fp64 (a fully
 * masked row keeps -inf). K must be F32, F16 or BF16 (FA_BACK_EUNSUPPORTED for the block types).
 * Costs: one pass over 256 keys of K and one over q, and one subtraction per decoded K value.
 * The fa_back_run_saved entry takes the uncentred LSE and removes the shift itself. */
#define FA_BACK_FLAG_CENTER_K 8u

/* FA_BACK_FLAG_KV_IMAGE, FA_BACK_FLAG_KV_INLINE: where the query-side walks get the fp16 K and
 * V tiles their products read. With KV_IMAGE a first kernel decodes every 32-key sub-tile of
 * the cache once into the workspace (128 * D bytes per sub-tile and KV head: the K and V tiles
 * as the walks lay them out in LDS), and the walks copy those tiles instead of decoding them;
 * with KV_INLINE every workgroup of the walks decodes the sub-tiles it reads. The results are
 * bitwise the same. With neither bit the plan takes the image when at least 4 row tiles (of
 * 128 query rows of one KV head) read each sub-tile. Setting both is FA_BACK_EINVAL. The choice
 * changes the workspace size: pass the same flags to fa_back_layout_query and fa_back_create;
 * KV_INLINE keeps the image out of a workspace that must stay within
 * FA_BACK_NOALLOC_MAX_WORKSPACE. */
#define FA_BACK_FLAG_KV_IMAGE 16u
#define FA_BACK_FLAG_KV_INLINE 32u

/* FA_BACK_FLAG_DS_STORE, FA_BACK_FLAG_DS_RECOMPUTE: how dQ = scale * dS K is formed. The pages'
 * structure ("CambrianTech/llama.cpp PR #63", third review) forms it in the query-side kernel,
 * which walks the keys a second time and recomputes S and dP for it (DS_RECOMPUTE). With
 * DS_STORE the key-side pass, which forms dS anyway, stores it in the workspace as fp16 tiles
 * (2 bytes per visible-or-not (row, key) pair of every listed 32-row block: Hkv * ceil(G*N/32)
 * * 4 * ceil(M/128) * 2048 bytes), and a dQ pass forms dS K from them; the query-side walk over
 * the keys for dQ is not run. It takes the decoded image of the cache (FA_BACK_FLAG_KV_INLINE
 * with DS_STORE is FA_BACK_EINVAL). The results meet the same bar, not bitwise the same: dS is
 * rounded with one exponent per KV head instead of one per row. With neither bit the plan
 * stores dS whenever it takes the image and the tiles need at most 16 GiB, and recomputes
 * otherwise. Setting both is FA_BACK_EINVAL. The choice changes the workspace size;
 * DS_RECOMPUTE keeps the tiles out of a workspace that must stay within
 * FA_BACK_NOALLOC_MAX_WORKSPACE. */
#define FA_BACK_FLAG_DS_STORE 64u
#define FA_BACK_FLAG_DS_RECOMPUTE 128u

/* status codes (no entry point aborts or exits) */
#define FA_BACK_OK 0
#define FA_BACK_EINVAL (-1)       /* null pointer, negative extent, non-finite scale, unknown flag bit */
#define FA_BACK_ESHAPE (-2)       /* extents disagree (D, Dv, N, M, H % Hkv, Hm, q8_0 width) */
#define FA_BACK_ESTRIDE (-3)      /* nb[0] != element size, zero stride, misaligned stride  */
#define FA_BACK_EUNSUPPORTED (-4) /* type combination, D/Dv, size limit, device not gfx950  */
#define FA_BACK_EHIP (-5)         /* a HIP runtime call or kernel launch failed             */
#define FA_BACK_EALIGN (-6)       /* a device pointer passed to fa_back_run is misaligned   */
#define FA_BACK_ESCRATCH (-7)     /* fa_back_run_noalloc: the plan's workspace exceeds
                                     FA_BACK_NOALLOC_MAX_WORKSPACE                        */

typedef struct {
    int32_t type;    /* FA_BACK_* element type */
    int64_t ne[3];   /* extents, innermost first */
    int64_t nb[3];   /* byte strides */
} fa_back_tensor;

typedef struct {
    fa_back_tensor q, k, v, d, mask;   /* mask.type == FA_BACK_NONE: no mask */
    float scale;                        /* softmax scale, e.g. 1/sqrt(D) */
    uint32_t flags;                     /* FA_BACK_FLAG_* bits, 0 for the plain operator */
} fa_back_desc;

typedef struct {
    uint64_t off_dq, off_dk, off_dv, off_lse, off_delta;  /* byte offsets in `out` */
    uint64_t out_bytes;        /* size the caller allocates for `out` */
    uint64_t workspace_bytes;  /* device scratch the caller allocates for `workspace` */
    uint32_t plan_flags;       /* the plan's choices as FA_BACK_FLAG_* bits: one of WALK1_KEYS /
                                  WALK1_ROWS, one of KV_IMAGE / KV_INLINE, one of DS_STORE /
                                  DS_RECOMPUTE (and the CENTER bits of the descriptor); a
                                  degenerate shape (N or M zero) reports none of the six */
} fa_back_layout;

typedef struct fa_back_plan fa_back_plan;

/* Validate a descriptor and compute the output layout and workspace size. Touches no
 * device, so it runs on a host without a GPU. The layout is a function of the descriptor
 * only (flags included), never of the device: fa_back_create returns the same one. Returns
 * FA_BACK_OK or an error code; `layout` is written only on success. */
int fa_back_layout_query(const fa_back_desc* desc, fa_back_layout* layout);

/* Validate `desc` (before touching the device), read the device's limits once, and build an
 * immutable plan. `device` must be a gfx950 GPU whose per-workgroup LDS (sharedMemPerBlock)
 * holds the largest tile buffer of the kernels for this head size (up to about 152 KiB at
 * D = 256), else FA_BACK_EUNSUPPORTED. The device's compute-unit count sets how work is split
 * over workgroups (the key-side tail split, the key-owned walk's row ranges); it never changes
 * the layout or the results' bits beyond what the split orders fix (same device type, same
 * bits). The plan is a pure function of the descriptor and these device limits; nothing in the
 * library reads the environment. On success *plan owns host memory only and `layout` (if
 * non-NULL) receives the same layout as fa_back_layout_query. On failure *plan is set to NULL. */
int fa_back_create(const fa_back_desc* desc, int device, fa_back_plan** plan,
                   fa_back_layout* layout);

/* Enqueue the backward on `stream` (a hipStream_t; NULL = the default stream) of the
 * plan's device. q, k, v, d, mask are device pointers to the first element of each view
 * (mask must be NULL iff the plan has no mask); out (layout.out_bytes) and workspace
 * (layout.workspace_bytes) are device buffers owned by the caller, 256-byte aligned, kept
 * alive until the stream has finished the work. The call allocates nothing, does not
 * synchronise, and the plan may be shared by concurrent runs that use distinct out and
 * workspace buffers. Workspace contents need not be initialised and are clobbered. */
int fa_back_run(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                const void* d, const void* mask, void* out, void* workspace, void* stream);

/* Number of kernel phases reported by fa_back_run_timed:
 * 0 absmax of q and dO, 1 q/dO to fp16 fragments, 2 query-side walk 1 (LSE and delta
 * statistics), 3 merge of key-range splits (writes LSE and delta), 4 query-side walk 2 (dQ),
 * or with FA_BACK_FLAG_DS_STORE the dQ pass from the stored dS, 5 dQ split reduction (empty
 * when the keys were not split), 6 key-side pass (dK, dV). They run in this order, except
 * that with FA_BACK_FLAG_DS_STORE phases 4 and 5 run after phase 6. */
#define FA_BACK_NUM_PHASES 7

/* fa_back_run plus timing, for profiling: records a HIP event on `stream` before and after
 * each phase, waits for the last one, and writes each phase's elapsed milliseconds to
 * phase_ms[0 .. FA_BACK_NUM_PHASES-1]. Unlike fa_back_run it blocks the
 * host until the run has finished; it creates and destroys its own events. */
int fa_back_run_timed(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                      const void* d, const void* mask, void* out, void* workspace, void* stream,
                      float* phase_ms);

/* fa_back_run with the forward's saved statistics: the natural-log LSE of every row (F32,
 * N*H floats at row h*N + i, -inf for a fully masked row) and the forward output
 * O = softmax(S) V (F32, contiguous [Dv, N, H], element (c, i, h) at (h*N + i)*Dv + c), both
 * device buffers owned by the caller. delta is then rowsum(dO o O), the definition the
 * operator's pages give for it (first review, "The math in fattn_back_q"), formed per row,
 * and the walk over the keys that forms LSE and delta (phases 2 and 3) is not run: phase 2
 * is a bound of |v| over the cache and phase 3 forms the row statistics from lse and o.
 * The packed LSE output is the given LSE, the delta output the computed delta. The results
 * equal fa_back_run's when lse and o are the forward's (same inputs, same mask) up to their
 * own rounding; nothing checks that they are. Same conventions, buffers and errors as
 * fa_back_run; lse and o may be NULL only when N*H == 0. This entry is not one the pages'
 * operator has: it is the form an SDPA backward takes when the forward saved LSE and O (as
 * the "AMD-AGI/TraceLens PR #757" page models it). */
int fa_back_run_saved(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                      const void* d, const void* mask, const float* lse, const float* o, void* out,
                      void* workspace, void* stream);

/* fa_back_run_saved plus the timing of fa_back_run_timed. */
int fa_back_run_saved_timed(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                            const void* d, const void* mask, const float* lse, const float* o,
                            void* out, void* workspace, void* stream, float* phase_ms);

/* Largest workspace (layout.workspace_bytes) fa_back_run_noalloc accepts: 64 MiB. */
#define FA_BACK_NOALLOC_MAX_WORKSPACE (64ull << 20)

/* fa_back_run for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, conventions and results
 * as fa_back_run (the same kernels run), except that there is no workspace argument: the
 * library's own static device array of FA_BACK_NOALLOC_MAX_WORKSPACE bytes serves as the
 * workspace. Each GPU the library runs on holds one copy of it from the plan's creation until
 * the process ends; fa_back_create looks up its address. The caller still passes the inputs
 * and `out`. The call allocates and frees nothing (no hipMalloc, no allocating library call).
 * Returns FA_BACK_ESCRATCH, enqueuing nothing, when the plan's workspace is larger than the
 * array. Every call on one GPU uses that GPU's single array: calls whose work overlaps on one
 * GPU (other streams, other threads, other plans) race, and the caller must order them, e.g.
 * on one stream. The array keeps the last call's contents; no kernel relies on them. */
int fa_back_run_noalloc(const fa_back_plan* plan, const void* q, const void* k, const void* v,
                        const void* d, const void* mask, void* out, void* stream);

/* Free a plan (NULL is allowed). */
void fa_back_destroy(fa_back_plan* plan);

/* Static text for a status code. */
const char* fa_back_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_BACK_H */
