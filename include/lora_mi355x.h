/*
 * lora_mi355x.h -- C ABI of the multi-LoRA batched layer for MI355X (gfx950).
 *
 * The layer, for a heterogeneous batch in which every row i carries an
 * adapter id a_i (or -1 for a base-only row):
 *
 *     y_i = x_i W + s_{a_i} * (x_i A[a_i]) B[a_i]
 *
 * Row-vector convention with W [d_in, d_out], A [d_in, r], B [r, d_out]:
 * "Serving multiple LoRAs: segmented matrix multiplies and adapter
 * scheduling", section "Not merging the weights, computing in batches".
 * The base product x W is computed once for the whole batch ("Multi-LoRA
 * batching and adapter paging", section "Walking through a batch"); the
 * low-rank term is a shrink (x -> xA, rank r) followed by an expand
 * ((xA) -> (xA)B) that is added to the base output (same page 3 section).
 * BGMV gathers each row's adapter by index (decode); SGMV groups rows by
 * adapter and runs one small product per segment (prefill) (same section;
 * also "Serving Many LoRA Adapters" (praveentn.live), section "Punica: The
 * Segmented Gather-Scatter Kernel").
 *
 * Conventions shared by every entry point
 *  - All tensors are caller-owned DEVICE memory unless marked "host".
 *    The library never frees them.  Row-major; ld* are leading dimensions
 *    in elements.
 *  - Element types: x, W, A and B share one dtype (LORA_F32 or LORA_BF16);
 *    the rank-r intermediate t is always fp32; y may be fp32 or bf16.
 *    Products accumulate in fp32 and y is rounded once (nearest even).
 *  - Pointers handed to the library must be 16-byte aligned, and so must
 *    ld* times the element size; otherwise LORA_E_UNSUPPORTED.
 *  - Every call that takes a stream only enqueues work on it and returns;
 *    argument errors are reported synchronously, before any launch, and
 *    nothing is enqueued then.  Nothing throws or aborts.  n_rows = 0 is a
 *    valid no-op.
 *  - Hot calls never allocate.  Scratch memory is a caller-provided
 *    workspace sized by the matching *_workspace query.  A workspace must
 *    be zero-filled once before its first use (lora_workspace_clear does
 *    it); every call leaves it in that state again.  Calls that overlap in
 *    time must not share a workspace.
 *  - Ids outside [-1, n_adapters) are treated as base-only rows and set
 *    bit 0 of the pool's device error word (see lora_pool_last_error).
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LORA_OK = 0,
    LORA_E_INVALID = 1,     /* bad argument: null pointer, size, rank, id table */
    LORA_E_UNSUPPORTED = 2, /* valid but not handled: alignment, rank > 64, ... */
    LORA_E_WORKSPACE = 3,   /* workspace missing or too small */
    LORA_E_ID_RANGE = 4,    /* reported by lora_pool_last_error only */
    LORA_E_DEVICE = 5,      /* a HIP runtime call failed */
    LORA_E_NOT_RESIDENT = 6, /* lora_cache_map: an adapter is not resident yet */
    LORA_E_SCRATCH = 7      /* lora_layer_apply_noalloc: the call needs more than
                               LORA_NOALLOC_SCRATCH_BYTES of scratch */
} lora_status_t;

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype_t;

/* Pool layouts ("Serving many LoRA adapters" (blog.ecitis.org), section
 * "Batching across different adapters": a uniform-rank pool is a dense 3-D
 * tensor; mixed ranks need ragged indexing or padding to the maximum). */
typedef enum { LORA_LAYOUT_UNIFORM = 0, LORA_LAYOUT_RAGGED = 1 } lora_layout_t;

/* How lora_layer_apply computes the low-rank term. */
typedef enum { LORA_MODE_AUTO = 0, LORA_MODE_BGMV = 1, LORA_MODE_SGMV = 2 } lora_mode_t;

/* Storage of the base weight.  LORA_W_IN_OUT: W as [d_in, d_out] (the
 * page-3 convention y = xW).  LORA_W_OUT_IN: W stored transposed, [d_out,
 * d_in] (the x W^T convention of "Serving Many LoRA Adapters"
 * (praveentn.live), section "Why Naive Batching Breaks").  Both give the
 * same bits.  LORA_W_OUT_IN is the fast one: the decode path needs it, and
 * on batches of thousands of rows the GEMM over LORA_W_IN_OUT, whose tiles
 * are transposed on their way into LDS, takes about twice as long. */
typedef enum { LORA_W_IN_OUT = 0, LORA_W_OUT_IN = 1 } lora_w_layout_t;

typedef struct lora_pool_s* lora_pool_t;

/* Segment descriptor written by lora_segments_build (all device, caller-owned):
 *   perm[n_rows]      rows in ascending adapter-id order, original order
 *                     inside a run (a stable argsort of the ids);
 *   seg_ids[cap]      id of each run; the run of base-only rows (id -1, and
 *                     invalid ids) comes first when present;
 *   seg_off[cap + 1]  run boundaries into perm; seg_off[n_seg] = n_rows;
 *   n_seg[1]          number of runs.
 *   cap               capacity of seg_ids, >= min(n_rows, n_adapters + 1).
 * The group-by is the stable argsort + run detection of "Serving multiple
 * LoRAs...", section "Not merging the weights, computing in batches". */
typedef struct {
    int32_t* perm;
    int32_t* seg_ids;
    int32_t* seg_off;
    int32_t* n_seg;
    int32_t cap;
} lora_segments_t;

/* Human-readable name of a status code (static storage). */
const char* lora_status_string(lora_status_t status);

/* Parameters of one adapter of rank r on a d_in -> d_out projection:
 * r * (d_in + d_out) ("Serving many LoRA adapters" (blog.ecitis.org),
 * section "Low-rank structure and additivity": 131,072 at 4096/4096/16).
 * Returns -1 for non-positive arguments.  Host only. */
int64_t lora_adapter_param_count(int32_t rank, int32_t d_in, int32_t d_out);

/* Element offsets for a ragged pool (host only, no device work).
 * ranks[n_adapters] (host) in [1, 64].  Writes a_off/b_off[n_adapters] (host)
 * and the total element counts of the A and B buffers.  Adapter u occupies
 * A[a_off[u] .. a_off[u] + d_in*ranks[u]) as row-major [d_in, r_u] and
 * B[b_off[u] .. + r_u*d_out) as row-major [r_u, d_out]; every block starts
 * on a 256-byte boundary for either dtype. */
lora_status_t lora_pool_ragged_offsets(int32_t n_adapters, const int32_t* ranks,
                                       int32_t d_in, int32_t d_out,
                                       int64_t* a_off, int64_t* b_off,
                                       int64_t* a_total, int64_t* b_total);

/* Describe a packed adapter pool over caller-owned device buffers A and B
 * (which must outlive the pool).
 *   UNIFORM: A is [n_adapters, d_in, r_max], B is [n_adapters, r_max, d_out];
 *            ranks/a_off/b_off must be NULL.  Padding lower ranks to r_max
 *            with zeros is this layout too.
 *   RAGGED:  ranks/a_off/b_off (host, n_adapters each) give every adapter's
 *            rank (1..r_max) and element offsets; blocks must not overlap and
 *            must start 16-byte aligned.
 * scales (host, n_adapters) is each adapter's s = alpha/r, which travels
 * with the adapter ("Serving many LoRA adapters" (blog.ecitis.org), section
 * "Correctness across tenants").  1 <= r_max <= 64.
 * Allocates small device tables (ranks, offsets, scales, error word) and
 * copies them synchronously on the null stream; the pool is immutable
 * afterwards and may be used from several streams at once. */
lora_status_t lora_pool_create(lora_pool_t* out, lora_layout_t layout, lora_dtype_t dtype,
                               int32_t n_adapters, int32_t d_in, int32_t d_out, int32_t r_max,
                               const int32_t* ranks, const int64_t* a_off, const int64_t* b_off,
                               const void* A, const void* B, const float* scales);

/* Free the pool's device tables (waits for the device first). NULL is a no-op. */
lora_status_t lora_pool_destroy(lora_pool_t pool);

/* r_u * (d_in + d_out) for adapter u of the pool, or -1 if u is out of range. */
int64_t lora_pool_param_count(lora_pool_t pool, int32_t adapter);

/* Synchronize `stream`, then read and clear the pool's device error word
 * into *out (bit 0: some call saw an id outside [-1, n_adapters)).
 * Returns LORA_E_ID_RANGE when bit 0 was set, LORA_OK otherwise. */
lora_status_t lora_pool_last_error(lora_pool_t pool, hipStream_t stream, int32_t* out);

/* Zero-fill a workspace on `stream` with a fill kernel (safe under graph
 * capture, unlike a memset node). */
lora_status_t lora_workspace_clear(void* ws, size_t bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Segments                                                                */
/* ---------------------------------------------------------------------- */

/* Workspace bytes for lora_segments_build: always 0 with the present
 * one-workgroup counting sort (the argument is kept so that a build for
 * larger pools can take scratch without an interface change); ws may be NULL. */
lora_status_t lora_segments_workspace(int32_t n_rows, int32_t n_adapters, size_t* bytes);

/* Stable group-by of ids[n_rows] (device) into *seg (one launch, integer
 * only, bit-exact).  n_adapters <= 16383.  `status` (device, may be NULL)
 * gets bit 0 set when an id is outside [-1, n_adapters). */
lora_status_t lora_segments_build(const int32_t* ids, int32_t n_rows, int32_t n_adapters,
                                  const lora_segments_t* seg, int32_t* status,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* BGMV: per-row gather of the row's adapter (decode)                     */
/* ---------------------------------------------------------------------- */

/* Shrink: t[i, 0:r_max] = x_i A[a_i] (fp32, unscaled), one launch for the
 * whole batch: every row gathers its own adapter's A by id ("Serving
 * multiple LoRAs: segmented matrix multiplies and adapter scheduling",
 * section "Not merging the weights, computing in batches"; "Serving Many
 * LoRA Adapters" (praveentn.live), section "Punica: The Segmented
 * Gather-Scatter Kernel": one launch over a heterogeneous batch).  Columns
 * [r_{a_i}, r_max) and base-only rows are written 0.
 *   x [n_rows, ldx] (pool dtype), ids [n_rows], t [n_rows, ldt] fp32,
 *   ldt >= r_max.  No workspace. */
lora_status_t lora_bgmv_shrink(lora_pool_t pool, const void* x, int64_t ldx,
                               const int32_t* ids, int32_t n_rows,
                               float* t, int64_t ldt, hipStream_t stream);

/* Expand: y_i (+)= s_{a_i} * t_i B[a_i], one launch for the whole batch,
 * each row gathering its own adapter's B (same passages as the shrink; the
 * scale travels with the adapter: "Serving many LoRA adapters"
 * (blog.ecitis.org), section "Correctness across tenants").
 * accumulate = 0: y_i is overwritten with the LoRA term (0 on base-only
 * rows).  accumulate = 1: the term is added to y_i; base-only rows are not
 * touched.  y [n_rows, ldy] of y_dtype. */
lora_status_t lora_bgmv_expand(lora_pool_t pool, const float* t, int64_t ldt,
                               const int32_t* ids, int32_t n_rows,
                               void* y, lora_dtype_t y_dtype, int64_t ldy, int accumulate,
                               hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* SGMV: rows grouped by adapter, one small product per segment (prefill) */
/* ---------------------------------------------------------------------- */

/* Workspace bytes with which lora_sgmv_shrink splits K for this batch size
 * (0: it does not split).  No zero-filling is needed. */
lora_status_t lora_sgmv_shrink_workspace(lora_pool_t pool, int32_t n_rows, size_t* bytes);

/* Shrink over segments from lora_segments_build, one small product per
 * segment ("Serving multiple LoRAs...", section "Not merging the weights,
 * computing in batches": sort rows by adapter, then one contraction per run)
 * (same t layout and values as lora_bgmv_shrink: original row order).  Rows of the base-only run get
 * t = 0.  Id-range errors are reported by lora_segments_build's `status`.
 * The grid is sized from n_rows and the pool size, so the segment count
 * never has to come back to the host.  With a workspace of
 * lora_sgmv_shrink_workspace bytes, K is cut into slices whose fp32 partial
 * sums a second launch adds in slice order (results do not depend on
 * timing, but differ from the unsplit form in rounding); with ws = NULL
 * every workgroup walks all of K.  A non-NULL ws that is too small or not
 * 16-byte aligned is LORA_E_WORKSPACE. */
lora_status_t lora_sgmv_shrink(lora_pool_t pool, const void* x, int64_t ldx,
                               const lora_segments_t* seg, int32_t n_rows,
                               float* t, int64_t ldt, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Expand over segments (same semantics as lora_bgmv_expand; the results go
 * back to each row's original position: "Serving many LoRA adapters"
 * (blog.ecitis.org), section "Replay": grouped product, then scatter-add). */
lora_status_t lora_sgmv_expand(lora_pool_t pool, const float* t, int64_t ldt,
                               const lora_segments_t* seg, int32_t n_rows,
                               void* y, lora_dtype_t y_dtype, int64_t ldy, int accumulate,
                               hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* The fused layer                                                         */
/* ---------------------------------------------------------------------- */

/* Workspace bytes for lora_layer_apply.  The W layout is not an argument,
 * so for BGMV batches of 65..1024 rows of a bf16 pool the size covers the
 * few-hundred-row form (W stored [d_out, d_in]): segments, fp32 base
 * partials (S * n_rows * d_out * 4 bytes, S <= 8 K slices) and t partials.
 * For a bf16 pool it also covers the fp32 K-slice partials of a tiled GEMM
 * launch that splits K (a 128x128 launch of few tiles over a long K, W
 * stored [d_out, d_in]), whatever the W layout and y dtype of the call. */
lora_status_t lora_layer_workspace(lora_pool_t pool, int32_t n_rows, lora_mode_t mode,
                                   size_t* bytes);

/* y = x W + s * (x A[ids]) B[ids] for the whole batch: the shrink runs in
 * one launch (BGMV or SGMV), then one MFMA GEMM launch computes x W for all
 * rows and adds the scaled expand before the single rounding of y
 * ("Serving many LoRA adapters" (blog.ecitis.org), section "Replay":
 * segmented gather, grouped GEMM, scatter-add, fused output).  Each GEMM
 * tile adds the expand either as extra K-blocks per distinct adapter (tiles
 * of long runs of one id) or row by row after its K loop (tiles whose rows
 * mostly carry different adapters).  Two forms differ:
 *  - decode (BGMV, 1..64 rows, bf16 pool, W stored [d_out, d_in]): the two
 *    launches of lora_decode_stream / lora_decode_finish;
 *  - few hundred rows (BGMV, 65..1024 rows, bf16 pool, W stored [d_out,
 *    d_in]): the shrink per segment tile (rows grouped by adapter, so each
 *    distinct adapter's A is read once per tile), the base product in fp32
 *    K-slice partials, and a finish per segment tile that adds the partials
 *    and the scaled expand (each adapter's B read once per tile) and rounds
 *    y once ("Serving many LoRA adapters", section "Batching across
 *    different adapters": the cost is reading each distinct adapter).
 *    Segments are built in the workspace unless `seg` is given.
 *   x [n_rows, ldx]; W per w_layout with leading dimension ldw; y [n_rows,
 *   ldy] of y_dtype.  `seg` may be NULL (SGMV builds segments in the
 *   workspace) or a descriptor already built for these ids by
 *   lora_segments_build; any other content is undefined behaviour (the
 *   kernels gather x and scatter t and y through perm, and not every kernel
 *   checks its entries).
 *   mode AUTO picks BGMV when n_rows <= 64 or n_rows <= 2 * n_adapters
 *   (segments would mostly hold one or two rows) and SGMV otherwise. */
lora_status_t lora_layer_apply(lora_pool_t pool, const void* x, int64_t ldx,
                               const void* W, int64_t ldw, lora_w_layout_t w_layout,
                               const int32_t* ids, const lora_segments_t* seg, int32_t n_rows,
                               void* y, lora_dtype_t y_dtype, int64_t ldy,
                               lora_mode_t mode, void* ws, size_t ws_bytes, hipStream_t stream);

/* lora_layer_apply for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation and kernels as lora_layer_apply (same arguments, same bits),
 * but with no workspace argument: the scratch it needs lives in one
 * file-scope device array of LORA_NOALLOC_SCRATCH_BYTES per GPU, which the
 * library holds from the first call on that GPU until the process ends.
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  The scratch needed is what lora_layer_workspace
 * reports for (pool, n_rows, mode); beyond the maximum the call returns
 * LORA_E_SCRATCH before any launch (use lora_layer_apply with a workspace
 * then).  Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (two streams, or two threads) race and give
 * wrong results: serialize them.  The device is the stream's. */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lora_status_t lora_layer_apply_noalloc(lora_pool_t pool, const void* x, int64_t ldx,
                                       const void* W, int64_t ldw, lora_w_layout_t w_layout,
                                       const int32_t* ids, const lora_segments_t* seg,
                                       int32_t n_rows, void* y, lora_dtype_t y_dtype, int64_t ldy,
                                       lora_mode_t mode, hipStream_t stream);

/* The second half of lora_layer_apply on its own:
 *   y = x W + s * t B[ids]   (t from lora_bgmv_shrink or lora_sgmv_shrink),
 *   y = x W                  when t is NULL (the base-only product).
 * Same argument rules as lora_layer_apply; t [n_rows, ldt] fp32 with
 * ldt >= r_max.  The workspace (lora_base_gemm_expand_workspace) holds the
 * scaled, split copy of t that the GEMM reads as extra K-blocks (tiles that
 * add the expand row by row read t itself); with t NULL no workspace is
 * needed.  The base-only form measures what the adapters add
 * to a step ("Serving many LoRA adapters" (blog.ecitis.org), section "What
 * to measure": adapter overhead fraction). */
lora_status_t lora_base_gemm_expand_workspace(lora_pool_t pool, int32_t n_rows, size_t* bytes);
lora_status_t lora_base_gemm_expand(lora_pool_t pool, const void* x, int64_t ldx,
                                    const void* W, int64_t ldw, lora_w_layout_t w_layout,
                                    const int32_t* ids, const float* t, int64_t ldt,
                                    int32_t n_rows, void* y, lora_dtype_t y_dtype, int64_t ldy,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Merged weights                                                          */
/* ---------------------------------------------------------------------- */

/* Fold adapter `adapter` into a base weight, in place:
 *   W += sign * s_a * A_a B_a
 * ("Serving many LoRA adapters" (blog.ecitis.org), section "Merge or keep
 * separate": a replica with the adapter merged serves its requests as plain
 * base-model GEMMs; sign = -1 takes the adapter back out, other values scale
 * the term.)
 *   W: device, the pool's dtype, caller-owned; layout per w_layout
 *      ([d_in, d_out] or [d_out, d_in]) with leading dimension ldw.
 *   Each element is read once, updated in fp32 and rounded once, so for a
 *   bf16 W a merge followed by an unmerge restores W only to within bf16
 *   rounding of each step.
 *   Errors: LORA_E_ID_RANGE for an adapter outside [0, n_adapters);
 *   LORA_E_INVALID for a null W, a non-finite sign or ldw below the row
 *   length; LORA_E_UNSUPPORTED for a W or ldw that is not 16-byte aligned. */
lora_status_t lora_merge_adapter(lora_pool_t pool, int32_t adapter, void* W, int64_t ldw,
                                 lora_w_layout_t w_layout, float sign, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Decode layer in two launches                                            */
/* ---------------------------------------------------------------------- */

/* For decode batches (bf16 pool, 1 <= n_rows <= 64, W stored LORA_W_OUT_IN)
 * lora_layer_apply in BGMV mode runs as these two launches; they are
 * exported so callers can place other work between them or time them.
 *   lora_decode_stream: partial base products x W over K slices, and, when
 *     with_lora != 0, the BGMV shrink of every row (each row gathers its own
 *     adapter's A) over K slices, all into the workspace;
 *   lora_decode_finish: y = sum of the base partials + s * (sum of the
 *     shrink partials) B[ids], rounded once into y (with_lora = 0: y = x W).
 * Both calls must see the same pool, ids, n_rows, with_lora and workspace;
 * the workspace holds fp32 partial sums only (no zeroing needed).
 * Sums run in a fixed order, so results are identical from run to run.
 * ("Multi-LoRA batching and adapter paging", section "Walking through a
 * batch": W is read once for all rows; the adapter term per row.) */
lora_status_t lora_decode_workspace(lora_pool_t pool, int32_t n_rows, int with_lora, size_t* bytes);
lora_status_t lora_decode_stream(lora_pool_t pool, const void* x, int64_t ldx, const void* W,
                                 int64_t ldw, const int32_t* ids, int32_t n_rows, int with_lora,
                                 void* ws, size_t ws_bytes, hipStream_t stream);
/* The stream launch over a 4-bit base weight, with bf16 x and bf16 adapters
 * ("Serving Many LoRA Adapters" (praveentn.live), section "When It Falls
 * Down": a 4-bit base with FP16/BF16 adapters needs a mixed-precision path).
 * The pages leave the format open; the one taken:
 *   Wq [d_out, ldq] bytes (device): the weight of output n and input k is a
 *     signed 4-bit two's-complement value in byte Wq[n * ldq + k / 2], k
 *     even in the low nibble;
 *   w_scale [d_out, lds] fp32 (device): the scale of inputs k = 128 g ..
 *     128 g + 127 of output n is w_scale[n * lds + g];
 *   the weight is q * scale (the layer's W[k][n]).
 * Products of x with the 4-bit values accumulate in fp32 per group of 128
 * inputs, and each group's sum is scaled once.  Follow with
 * lora_decode_finish (same pool, ids, n_rows, with_lora, workspace), which
 * adds the adapter term and rounds y once; lora_decode_workspace sizes the
 * workspace.  Requires d_in % 128 == 0, ldq >= d_in / 2 with ldq % 16 == 0, a
 * 16-byte aligned Wq, a 4-byte aligned w_scale and lds >= d_in / 128
 * (otherwise LORA_E_UNSUPPORTED / LORA_E_INVALID); the other rules are
 * lora_decode_stream's. */
lora_status_t lora_decode_stream_q4(lora_pool_t pool, const void* x, int64_t ldx, const uint8_t* Wq,
                                    int64_t ldq, const float* w_scale, int64_t lds, const int32_t* ids,
                                    int32_t n_rows, int with_lora, void* ws, size_t ws_bytes,
                                    hipStream_t stream);
lora_status_t lora_decode_finish(lora_pool_t pool, const int32_t* ids, int32_t n_rows, int with_lora,
                                 void* y, lora_dtype_t y_dtype, int64_t ldy, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* The layer over a 4-bit base weight, any batch size, with bf16 x and bf16
 * adapters ("Serving Many LoRA Adapters" (praveentn.live), section "When It
 * Falls Down": a 4-bit quantized base with BF16 adapters needs the batched
 * adapter kernels to run on a mixed-precision path).  The weight format is
 * lora_decode_stream_q4's (signed nibbles, one fp32 scale per output and 128
 * inputs); the adapter term is the bf16 one, unchanged.
 *   1..64 rows: lora_decode_stream_q4 + lora_decode_finish;
 *   65..1024 rows: segments (built in the workspace unless `seg` is given),
 *     the shrink per segment tile, the base product over 128 x 64 tiles whose
 *     4-bit W blocks are widened exactly to bf16 in LDS (each 128-deep block
 *     is one scale group: its sums are scaled once and added), and the
 *     finish per segment tile (base partials + s * t B_a, y rounded once);
 *     the workspace holds fp32 base partials of n_rows * d_out * 4 bytes;
 *   more rows: lora_layer_apply's SGMV form (segments, the SGMV shrink, one
 *     fused GEMM over 256 x 256 tiles with the adapter term in its K loop)
 *     whose W tiles are widened to bf16(q * scale), each weight rounded once
 *     (at most 2^-9 of its value, the precision of a bf16 base weight).
 * lora_layer_q4_workspace sizes the workspace.  Requires a bf16 pool, d_in % 128 == 0,
 * ldq >= d_in / 2 with ldq % 16 == 0, a 16-byte aligned Wq, a 4-byte aligned
 * w_scale and lds >= d_in / 128; otherwise LORA_E_UNSUPPORTED /
 * LORA_E_INVALID.  The other rules are lora_layer_apply's. */
lora_status_t lora_layer_q4_workspace(lora_pool_t pool, int32_t n_rows, size_t* bytes);
lora_status_t lora_layer_apply_q4(lora_pool_t pool, const void* x, int64_t ldx, const uint8_t* Wq,
                                  int64_t ldq, const float* w_scale, int64_t lds, const int32_t* ids,
                                  const lora_segments_t* seg, int32_t n_rows, void* y,
                                  lora_dtype_t y_dtype, int64_t ldy, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Adapter slot cache (paging)                                             */
/* ---------------------------------------------------------------------- */

/* GPU adapter slots treated as a cache over adapters kept in host memory
 * ("Multi-LoRA batching and adapter paging", section "Adapter paging": a
 * resident adapter is scheduled at once; a missing one evicts a cold
 * adapter and is copied in; concurrent loads are capped; pinned adapters
 * are never evicted.  "Serving many LoRA adapters" (blog.ecitis.org),
 * section "Paging adapters": a fetch never blocks the step, a miss delays
 * only that request's admission while the load runs, eviction is LRU over
 * adapter ids, and an adapter with queued requests is not evicted.
 * "Serving Many LoRA Adapters" (praveentn.live), section "S-LoRA": adapters
 * outside the batch live in host DRAM and are prefetched over PCIe while
 * the GPU computes.)
 *
 * An adapter is a set of n_parts projections (e.g. every projection of
 * every layer), part p being A_p [d_in[p], r] and B_p [r, d_out[p]] with
 * one rank r and one scale s for the whole adapter.  A slot holds a whole
 * adapter; each part is exposed as a RAGGED lora_pool_t over the slot
 * arena (lora_cache_pool) whose "adapter ids" are slot numbers, so the hot
 * calls run unchanged on ids translated by lora_cache_map.  A slot has room
 * for rank r_max; an adapter of rank r is computed at rank r.
 *
 * Host blob.  Each registered adapter is one contiguous host buffer in the
 * compact layout of lora_cache_blob_layout (part p's A at a_off[p], its B
 * at b_off[p], row-major, element offsets).  A load is one host-to-device
 * copy of that blob plus one small table-update kernel, both on the cache's
 * own copy stream (default priority).  The blob should be pinned
 * (hipHostMalloc); it must stay valid and unchanged while registered.
 *
 * Not thread-safe: one thread drives a cache.  Destroying the cache waits
 * for the device and frees the arena, the pools and the copy stream. */
typedef struct lora_cache_s* lora_cache_t;

typedef enum {
    LORA_CACHE_RESIDENT = 0, /* loaded: lora_cache_map accepts it */
    LORA_CACHE_LOADING = 1,  /* a copy is in flight (started now or earlier) */
    LORA_CACHE_DEFERRED = 2  /* not resident and no load started: the load cap
                                is reached or every slot is pinned, held or in use */
} lora_cache_state_t;

/* flags for lora_cache_create */
#define LORA_CACHE_HOST_ONLY 1 /* policy only: no device memory and no HIP call;
                                  loads complete only at lora_cache_poll or
                                  lora_cache_wait (so a run of the policy depends
                                  on the call sequence alone); no pools; blobs
                                  may be NULL */
#define LORA_CACHE_ANY_RANK 2  /* accept every rank 1..r_max (otherwise ranks must
                                  be multiples of 16 bytes of elements that divide
                                  512*16/elem, the ranks the streaming shrink takes) */
#define LORA_CACHE_EXPLICIT_POLL 4 /* a device cache whose loads complete only at
                                  lora_cache_poll or lora_cache_wait, never inside
                                  lora_cache_request or lora_cache_map: admission
                                  then depends on the call sequence and the points
                                  where the caller polls, not on copy timing */

typedef struct {
    int64_t requests;          /* lora_cache_request calls */
    int64_t hits;              /* ... that found the adapter resident */
    int64_t pending;           /* ... that found its load still in flight */
    int64_t loads_started;     /* ... that started a load (the misses served) */
    int64_t deferred_load_cap; /* ... deferred: loads_in_flight == max */
    int64_t deferred_no_slot;  /* ... deferred: no evictable slot */
    int64_t loads_completed;
    int64_t evictions;         /* loads that replaced a resident adapter */
    int64_t bytes_loaded;      /* host-to-device bytes of started loads */
    int64_t bytes_resident;    /* blob bytes of the adapters in slots */
    int32_t n_slots;
    int32_t slots_resident;    /* loaded */
    int32_t slots_loading;     /* = loads in flight */
    int32_t slots_bound;       /* mapped by a batch not yet released */
} lora_cache_stats_t;

/* Element offsets of each part inside an adapter's compact blob for rank r
 * (host only).  a_off/b_off are [n_parts] (host out); every block starts on
 * a 256-byte boundary.  *blob_elems is the blob length in elements. */
lora_status_t lora_cache_blob_layout(lora_cache_t cache, int32_t rank, int64_t* a_off,
                                     int64_t* b_off, int64_t* blob_elems);

/* Create a cache of n_slots slots over adapters 0..n_adapters-1.
 *   d_in/d_out (host, n_parts each) are the part shapes; 1 <= r_max <= 64;
 *   1 <= max_loads_in_flight.  Allocates the slot arena (n_slots blobs of
 *   rank r_max), the per-part pool tables and the copy stream (all freed by
 *   lora_cache_destroy) unless flags has LORA_CACHE_HOST_ONLY. */
lora_status_t lora_cache_create(lora_cache_t* out, lora_dtype_t dtype, int32_t n_parts,
                                const int32_t* d_in, const int32_t* d_out, int32_t r_max,
                                int32_t n_adapters, int32_t n_slots,
                                int32_t max_loads_in_flight, int32_t flags);
lora_status_t lora_cache_destroy(lora_cache_t cache);

/* Register adapter `adapter` (host tier): rank, scale s = alpha/r, and the
 * host blob.  Re-registering a resident, loading or bound adapter is
 * LORA_E_INVALID.  Ranks outside [1, r_max] (or not taken, see
 * LORA_CACHE_ANY_RANK) are LORA_E_UNSUPPORTED. */
lora_status_t lora_cache_register(lora_cache_t cache, int32_t adapter, int32_t rank, float scale,
                                  const void* blob);

/* Pin (pinned != 0) or unpin an adapter: a pinned adapter is never evicted
 * while resident.  Pinning does not load it. */
lora_status_t lora_cache_pin(lora_cache_t cache, int32_t adapter, int32_t pinned);

/* Add delta to the adapter's count of queued requests; an adapter with a
 * positive count is not evicted.  A count below zero is LORA_E_INVALID. */
lora_status_t lora_cache_hold(lora_cache_t cache, int32_t adapter, int32_t delta);

/* Ask for an adapter (never blocks).  Resident: marks it recently used and
 * returns RESIDENT.  Loading: LOADING.  Otherwise a load starts when fewer
 * than max_loads_in_flight are in flight and a slot is free or evictable
 * (the least recently used slot whose adapter is not pinned, held or bound;
 * empty slots first, ties to the lowest slot): LOADING; else DEFERRED.
 * Completed loads are noticed first (see lora_cache_poll). */
lora_status_t lora_cache_request(lora_cache_t cache, int32_t adapter, lora_cache_state_t* state);

/* Notice completed loads without waiting (HOST_ONLY: complete them all).
 * lora_cache_request and lora_cache_map notice completed loads too, except
 * in a HOST_ONLY cache.
 * *n_completed (may be NULL) gets the number noticed by this call. */
lora_status_t lora_cache_poll(lora_cache_t cache, int32_t* n_completed);

/* Block until every load in flight has completed (a warm-up job's
 * prefetch), then poll. */
lora_status_t lora_cache_wait(lora_cache_t cache);

/* Bind a batch: adapters[n] (host, -1 = base-only row) -> slots[n] (host out,
 * -1 stays -1).  Every id >= 0 must be registered (else LORA_E_INVALID) and
 * resident (else LORA_E_NOT_RESIDENT); on error nothing is bound.  Bound
 * adapters are marked recently used and are not evicted until
 * lora_cache_release; `stream` is made to wait for their loads.  Several
 * maps may precede one release (e.g. one per part). */
lora_status_t lora_cache_map(lora_cache_t cache, const int32_t* adapters, int32_t n,
                             int32_t* slots, hipStream_t stream);

/* End of the batch's use of its bound slots: records on `stream` (after the
 * batch's launches) the point a later eviction of those slots waits for. */
lora_status_t lora_cache_release(lora_cache_t cache, hipStream_t stream);

/* The pool of part p (owned by the cache; lora_pool_destroy refuses it).
 * NULL for a HOST_ONLY cache or p out of range. */
lora_pool_t lora_cache_pool(lora_cache_t cache, int32_t part);

/* Slot of an adapter, or -1 when it is neither resident nor loading. */
int32_t lora_cache_slot_of(lora_cache_t cache, int32_t adapter);

lora_status_t lora_cache_stats(lora_cache_t cache, lora_cache_stats_t* out);

/* ---------------------------------------------------------------------- */
/* Adapter-aware admission                                                 */
/* ---------------------------------------------------------------------- */

/* Forms each step's batch from a queue of requests (host only, no device
 * work).  Every queued request scores
 *     w_fair * (now - arrival) + w_local * locality * rows,
 * locality being 1 when the request's adapter is active (used by the
 * previous step's batch or already admitted to this one) and 0 otherwise
 * ("Serving many LoRA adapters" (blog.ecitis.org), section "Adapter-aware
 * scheduling": cost grows with distinct adapters per step; the wait term
 * grows without bound, so no tenant starves).  The batch fills in score
 * order (ties: earlier arrival, then earlier submission) under:
 *   - max_rows rows (tokens) per batch;
 *   - max_adapters distinct adapters per batch ("Serving multiple LoRAs...",
 *     section "Scheduling the adapters": requests beyond the cap wait for a
 *     later batch); base-only requests (adapter -1) never count;
 *   - rank_groups != 0: one rank class per batch, classes being ranks
 *     1, 2, 3-4, 5-8, 9-16, 17-32, 33-64 (same section, exercise 2: batch
 *     by rank group);
 *   - with a cache: the adapter must be resident.  A request whose adapter
 *     is not is skipped for this step, and asking the cache for it starts
 *     its load ("Serving many LoRA adapters", section "Paging adapters":
 *     defer that request, prefetch while it queues).  Queued requests hold
 *     their adapter in the cache (lora_cache_hold) so it is not evicted.
 * A request that does not fit stays queued.  Not thread-safe. */
typedef struct lora_sched_s* lora_sched_t;

typedef struct {
    double w_fair;        /* weight of the wait, per unit of the caller's clock (>= 0) */
    double w_local;       /* weight of locality x rows (>= 0) */
    int32_t max_adapters; /* distinct adapters per batch, >= 1 */
    int32_t max_rows;     /* rows per batch, >= 1 */
    int32_t rank_groups;  /* != 0: one rank class per batch */
} lora_sched_config_t;

typedef struct {
    int32_t admitted;            /* requests in the batch */
    int32_t rows;                /* their rows */
    int32_t distinct_adapters;   /* distinct ids >= 0 in the batch */
    int32_t skipped_rows;        /* skipped: would exceed max_rows (or capacity) */
    int32_t skipped_cap;         /* skipped: new adapter with the batch at max_adapters */
    int32_t skipped_rank_group;  /* skipped: other rank class */
    int32_t deferred_not_resident; /* skipped: adapter not resident in the cache */
    int32_t queued;              /* requests left in the queue */
    double max_wait_admitted;    /* longest wait among admitted requests */
    double max_wait_queued;      /* longest wait among those left */
} lora_sched_step_t;

/* ranks (host, n_adapters) may be NULL unless cfg->rank_groups != 0;
 * cache may be NULL (every adapter counts as resident).  The cache must
 * outlive the scheduler and cover the same adapter ids. */
lora_status_t lora_sched_create(lora_sched_t* out, const lora_sched_config_t* cfg,
                                int32_t n_adapters, const int32_t* ranks, lora_cache_t cache);
/* Drops the queue (and the cache holds of its requests). */
lora_status_t lora_sched_destroy(lora_sched_t sched);

/* Queue a request of `rows` rows (>= 1) for adapter `adapter` (-1: base
 * only) that arrived at time `arrival` (finite). */
lora_status_t lora_sched_submit(lora_sched_t sched, int64_t request, int32_t adapter, int32_t rows,
                                double arrival);

/* Form one batch at time `now` of at most `capacity` requests.  Writes,
 * in admission order, requests/adapters/rows/waits[0 .. info->admitted)
 * (host out arrays of `capacity` entries each; waits may be NULL) and the
 * step's counts into *info.  If asking the cache fails, the fill stops
 * there: the requests admitted so far form the batch (and leave the queue)
 * and the cache's error is returned. */
lora_status_t lora_sched_step(lora_sched_t sched, double now, int32_t capacity, int64_t* requests,
                              int32_t* adapters, int32_t* rows, double* waits,
                              lora_sched_step_t* info);

/* Requests waiting in the queue. */
int32_t lora_sched_queued(lora_sched_t sched);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
