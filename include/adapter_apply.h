/*
 * adapter_apply -- multi-LoRA delta kernels for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument documented "device" is a HIP device pointer;
 * "host" pointers are read during the call only.  `stream` is a hipStream_t
 * (NULL = the null stream).  The library allocates nothing and keeps no
 * pointer after a call returns; every call enqueues work on `stream` and
 * returns without synchronising.  All argument checks run on the host before
 * anything is enqueued: a call that returns an error has launched nothing.
 * No C++ exception crosses this interface.
 *
 * Sources of the operations (cited by page title and section):
 *   [vLLM] "vllm.lora.layers" API page.
 *   [SGL]  SGLang "lora_manager.py" source page.
 *   [PR]   "PR #48884 report" page (vLLM Inkling LoRA support).
 *
 * Common argument conventions
 * ---------------------------
 *   T        tokens (rows of x and y), T >= 0 (T == 0 is a no-op).
 *   K        input features (hidden size), K >= 1, K % 8 == 0.
 *   S        slices (packed sub-layers: 3 for QKV, 2 for gate_up), 1..8.
 *   N[S]     host array: output width of each slice, each >= 1 and % 4 == 0.
 *   L        adapter slots (max_loras), 1..1024.
 *   R        padded rank of the stacked tensors, 1..512.
 *   A[S]     host array of S device pointers; A[s] is the stacked lora_a of
 *            slice s, row-major [L][R][K] ([vLLM] MergedColumnParallelLinear-
 *            WithLoRA.create_lora_weights; the page's singleton dim dropped).
 *   B[S]     host array of S device pointers; B[s] is the stacked lora_b of
 *            slice s, row-major [L][N[s]][R].
 *   idx      device int32 [T]: adapter slot of each token.  idx < 0 means
 *            "no adapter" ([vLLM] the -1 entry of adapter_enabled); idx >= L
 *            is treated the same way and counted as invalid by
 *            lora_build_segments.
 *   slot_rank device int32 [L] or NULL: true rank r_s <= R of each slot
 *            ([SGL] prepare_lora_batch lora_ranks).  0 marks an empty slot,
 *            whose tokens pass through.  NULL means every slot has rank R.
 *            Only rank rows/columns j < r_s are read; the stored slot must be
 *            zero (or at least finite) beyond r_s, as reset_lora/set_lora
 *            leave it ([vLLM] MergedColumnParallelLinearWithLoRA).
 *   scale    device float [L]: per-slot scaling applied once to each output
 *            element of the expand ([SGL] prepare_lora_batch scalings).
 *   dtype    LORA_DT_BF16 (x, A, B, y all bf16) or LORA_DT_F32 (all fp32;
 *            decode path only).  The intermediate buffer is always fp32.
 *   path     The kernels a call runs.  LORA_PATH_AUTO chooses; any other
 *            value forces that path and returns LORA_E_PATH when its shapes
 *            do not allow the arguments.  lora_plan_packed reports the path
 *            lora_apply_packed takes, without running it.
 *
 *            Paths and the shapes each takes ("rows of 8": every N[s], ldy
 *            and y_col_offset % 8 == 0):
 *              RELAY    lora_apply_packed only.  One launch; the shrink is
 *                       split over K chunks of 256 columns and handed to the
 *                       expand work-groups of the same launch through a
 *                       region at the END of ws.  bf16, R in {16, 32},
 *                       T <= 1024, L <= 64, K % 256 == 0, K <= 8192, rows
 *                       of 8; needs ws (see ws below).
 *              FUSED    lora_apply_packed only.  One launch, no workspace;
 *                       each work-group recomputes its group's shrink.
 *                       bf16, R % 16 == 0, R <= 32, T <= 1024,
 *                       K % 1024 == 0, rows of 8.
 *              GROUPED  slot-grouped split-K MFMA shrink, MFMA expand (two
 *                       launches; groups found from idx inside the kernels
 *                       while L <= 64 and T <= 1024, else from the segment
 *                       table).  bf16, R % 16 == 0, R <= 128, T <= 4096;
 *                       shrink: K % 64 == 0, K <= 8192; expand: rows of 8;
 *                       LORA_FLAG_PARTIAL only for R <= 64.
 *              PREFILL  segments, MFMA tile shrink (split over K when its
 *                       tiles are few), MFMA tile expand.  bf16, R % 16 == 0
 *                       (the persistent expand: R in {16, 32, 64, 128} and
 *                       rows of 8).
 *              TOKEN    lora_apply_packed only.  One launch, no workspace;
 *                       work-group = (token, 256 output columns of a slice),
 *                       each recomputing its token's shrink (VALU).  Every
 *                       shape and dtype the call accepts whose grid
 *                       (T x the slices' 256-column chunks) is at most
 *                       2^31 - 1 work-groups.
 *              DECODE   segments, VALU split-K shrink, VALU expand.  Every
 *                       shape and dtype the call accepts.
 *
 *            LORA_PATH_AUTO in lora_apply_packed ("narrow": the slices sum
 *            to at most 16384 columns; "a relay batch": with
 *            U = L (1 - exp(-T / L)) the slots expected to draw tokens,
 *            U + T / 32 <= 12 or T >= 24 U; W = T * sum ceil(N[s] / 256),
 *            TOKEN's work-groups; e = 2 (bf16) or 4 (fp32) bytes; the first
 *            row that holds wins):
 *              | condition                                        | path    |
 *              | ceil(W / 1024) * ceil(R / 16) <= 4,              | TOKEN   |
 *              |   K*R*e <= 1 MB, W*K*R*e <= 44 MB (bf16, narrow, |         |
 *              |   RELAY's shapes and ws), 72 MB (other bf16) or  |         |
 *              |   512 MB (fp32)                                  |         |
 *              | RELAY's shapes, ws of lora_workspace_size(), and | RELAY   |
 *              |   not narrow, or narrow and a relay batch        |         |
 *              | GROUPED's shapes, R == 16, T <= 4096, L <= 128,  | GROUPED |
 *              |   narrow                                         |         |
 *              | T >= 512, T / min(T, L) >= 64, bf16, R % 16 == 0 | PREFILL |
 *              | FUSED's shapes, narrow, L <= 64                  | FUSED   |
 *              | GROUPED's shapes, L <= 64, R <= 64, narrow       | GROUPED |
 *              | bf16, R in {16, 32, 64, 128}, rows of 8          | PREFILL |
 *              | otherwise                                        | DECODE  |
 *            LORA_PATH_AUTO in lora_shrink / lora_expand (RELAY and FUSED
 *            are not theirs):
 *              | condition                                        | path    |
 *              | T >= 512, T / min(T, L) >= 64, bf16, R % 16 == 0 | PREFILL |
 *              | no LORA_FLAG_PARTIAL, bf16, L > 64 or R > 64,    | PREFILL |
 *              |   R in {16, 32, 64, 128} (expand: rows of 8)     |         |
 *              | otherwise                                        | DECODE  |
 *            A shrink and an expand called apart exchange the token-ordered
 *            buffer, which every path writes and reads alike, so the two
 *            calls need not take the same path (with LORA_FLAG_PARTIAL they
 *            must).
 *   ws       device workspace of at least lora_workspace_size() bytes,
 *            256-byte aligned, owned by the caller.  Calls sharing a
 *            workspace must be ordered on one stream.  The workspace must be
 *            zero-filled before its first use (lora_workspace_init); the
 *            library leaves its counters at zero after every call.  RELAY
 *            keeps its partial sums and counters in a region at the END of ws
 *            (ws_bytes decides where) that must be zero on entry and is left
 *            zero; every other region starts at offset 0.  So a workspace
 *            shared by calls of several shapes must hold
 *            lora_workspace_size() at the largest value of each size
 *            argument, and it must not be shared with the fused-MoE calls.
 *   flags    LORA_FLAG_SEGMENTS_READY: the workspace already holds the
 *            segments of this (idx, slot_rank, T, L) from lora_build_segments
 *            (built once per batch and shared by every LoRA layer, as [SGL]
 *            prepare_lora_batch does); otherwise the call rebuilds them.
 *            LORA_FLAG_ACTIVE_ONLY (lora_shrink): write only the buffer entries
 *            of tokens that carry an adapter and ranks j < r; the other
 *            entries keep their contents (saves a fill when the buffer only
 *            feeds lora_expand, which never reads them).
 *            LORA_FLAG_PARTIAL (lora_shrink then lora_expand, same ws, buf
 *            and path): on the DECODE and GROUPED paths the shrink leaves its
 *            per-K-chunk partial sums in the workspace and the expand adds
 *            them (one launch fewer); buf is then neither written nor read.
 *            The prefill path ignores the flag and goes through buf.
 *
 * Alignment: x, y, A[s], B[s] 16-byte aligned; K and ldx % 8 == 0; every
 * N[s], ldy and y_col_offset % 4 == 0; R % 8 == 0 for bf16 and R % 4 == 0
 * for fp32 (whole 16-byte units per lora_b row); buf 16-byte aligned.
 * Violations -> LORA_E_ALIGN.
 * Aliasing of y with x, A, B, buf or ws is not allowed.
 */
#ifndef ADAPTER_APPLY_H
#define ADAPTER_APPLY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lora_status_t;

#define LORA_OK           0
#define LORA_E_NULL       1  /* a required pointer is NULL                        */
#define LORA_E_SHAPE      2  /* size out of range or ld smaller than the row      */
#define LORA_E_DTYPE      3  /* unknown dtype                                     */
#define LORA_E_RANK       4  /* R outside [1, 512]                                */
#define LORA_E_SLICES     5  /* S outside [1, 8]                                  */
#define LORA_E_WORKSPACE  6  /* ws_bytes smaller than the required size           */
#define LORA_E_ALIGN      7  /* pointer or stride alignment not met               */
#define LORA_E_PATH       8  /* forced path cannot run these arguments            */
#define LORA_E_LAUNCH     9  /* the HIP runtime rejected a launch                 */
#define LORA_E_TIMEOUT   10  /* lora_workspace_check: a RELAY hand-over wait gave up */
#define LORA_E_RUNTIME   11  /* a HIP runtime call (not a launch) failed          */
#define LORA_E_SCRATCH   12  /* lora_apply_packed_noalloc: the call needs more
                                scratch than LORA_STATIC_SCRATCH_BYTES holds      */

#define LORA_DT_F32   0
#define LORA_DT_BF16  1

#define LORA_PATH_AUTO     0
#define LORA_PATH_DECODE   1
#define LORA_PATH_PREFILL  2
#define LORA_PATH_FUSED    3
#define LORA_PATH_GROUPED  4
#define LORA_PATH_RELAY    5
#define LORA_PATH_TOKEN    6

#define LORA_FLAG_SEGMENTS_READY 1u
#define LORA_FLAG_ACTIVE_ONLY    2u
#define LORA_FLAG_PARTIAL        4u
#define LORA_FLAG_RELAY_GIVE_UP  8u   /* test hook, see lora_workspace_check */

#define LORA_MAX_SLICES 8
#define LORA_MAX_RANK   512
#define LORA_MAX_SLOTS  1024

/* Human-readable text of a status code (static storage). */
const char *lora_status_string(lora_status_t status);

/* Bytes of workspace needed by the linear calls for these sizes
 * (covers lora_build_segments, lora_shrink, lora_expand, lora_apply_packed). */
lora_status_t lora_workspace_size(int32_t T, int32_t K, int32_t S, int32_t R, int32_t L,
                                  size_t *bytes);

/* Zero-fill a workspace (a fill kernel on `stream`, no memset node). */
lora_status_t lora_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * Status of the calls made on a workspace since its last check, for the one
 * path whose kernels wait on each other: RELAY hands partial sums from shrink
 * to expand work-groups of one launch, and each wait is bounded (it ends
 * because work-groups start in block order; the bound only guards against a
 * dispatcher that does not).  A wait that gives up sets an error word in the
 * first int32 of the workspace's last 256-byte line and lets the kernel
 * finish; that call's y is then not valid, and late partial sums may be left
 * in the workspace where the next RELAY call would take them for its own.
 * This call synchronises `stream`, reads the word and returns LORA_OK when it
 * is zero; otherwise it zero-fills the whole workspace (so the next call
 * starts clean; segments built with lora_build_segments must be built again),
 * synchronises again and returns LORA_E_TIMEOUT.  ([SGL] reports failures of
 * its control-plane calls explicitly, LoRAUpdateOutput(success,
 * error_message); this is the data path's counterpart.)  Blocking: not for
 * graph capture.  LORA_FLAG_RELAY_GIVE_UP (a test hook) makes every wait of a
 * RELAY call give up after its first poll, so the error path can be forced
 * from the host while every kernel still ends normally.
 * The fused-MoE workspace keeps the same line free, so the check returns
 * LORA_OK on it.
 */
lora_status_t lora_workspace_check(void *ws, size_t ws_bytes, void *stream);
/* ws == NULL with ws_bytes == 0 checks (and repairs) the current device's
 * static scratch of lora_apply_packed_noalloc instead. */

/* Byte offsets, inside the workspace, of the segment arrays written by
 * lora_build_segments, so callers and tests can read them back:
 *   header  int32[4] = {active tokens, invalid tokens (idx >= L), decode tiles, prefill tiles}
 *   slot_start int32[L+1], perm int32[T] (-1 past the active tokens). */
typedef struct {
    int64_t header;
    int64_t slot_start;
    int64_t perm;
    int64_t tiles_decode;
    int64_t tiles_prefill;
    int32_t tile_decode_tokens;
    int32_t tile_prefill_tokens;
} lora_segment_layout_t;

lora_status_t lora_segment_layout(int32_t T, int32_t L, lora_segment_layout_t *out);

/*
 * Segment build: the active tokens sorted stably by slot, with the start of
 * each slot's run and the work tiles of both paths.  This is the token
 * grouping that segmented LoRA GEMMs run on ([SGL] header credit to S-LoRA
 * and Punica, "triton" backend; prepare_lora_batch builds the batch's slot
 * list once and shares it across layers).  One launch up to 4096 tokens, two
 * past that (per-work-group key counts, then the scatter); bit-exact and
 * deterministic either way.
 */
lora_status_t lora_build_segments(const int32_t *idx, const int32_t *slot_rank, int32_t T,
                                  int32_t L, int32_t R, void *ws, size_t ws_bytes, void *stream);

/*
 * Shrink ([vLLM] RowParallelLinearWithShardedLoRA.apply, the add_shrink call
 * into a float32 buffer of shape (n_slices, tokens, rank) with scale 1.0):
 *   buf[s][t][j] = sum_i x[t][i] * A[s][idx[t]][j][i]   for active t, j < r
 *   buf[s][t][j] = 0                                      otherwise
 * buf: device fp32 [S][T][R], overwritten entirely (active entries only with
 * LORA_FLAG_ACTIVE_ONLY).  x: device [T][ldx].
 */
lora_status_t lora_shrink(float *buf, const void *x, int64_t ldx, int32_t T, int32_t K,
                          const void *const *A, int32_t S, int32_t L, int32_t R,
                          const int32_t *idx, const int32_t *slot_rank, int32_t dtype,
                          int32_t path, uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/*
 * Expand ([vLLM] RowParallelLinearWithShardedLoRA.apply, the add_expand call
 * with output_slices, offset_start and add_input=True):
 *   off_s = y_col_offset + N[0] + ... + N[s-1]
 *   y[t][off_s + n] = round(y[t][off_s + n] + scale[idx[t]] * sum_{j<r} buf[s][t][j] * B[s][idx[t]][n][j])
 * y: device [T][ldy], updated in place (rows of inactive tokens untouched).
 * buf: device fp32 [S][T][R] (entries j >= r are not read).  One rounding
 * to the storage type per output element (round to nearest even).
 */
lora_status_t lora_expand(void *y, int64_t ldy, int64_t y_col_offset, const float *buf,
                          int32_t T, const void *const *B, const int64_t *N, int32_t S,
                          int32_t L, int32_t R, const int32_t *idx, const int32_t *slot_rank,
                          const float *scale, int32_t dtype, int32_t path, uint32_t flags,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Packed apply: shrink then expand over all S slices of a merged layer, the
 * buffer kept in the workspace ([vLLM] MergedColumnParallelLinearWithLoRA,
 * MergedQKVParallelLinearWithLoRA; the shrink/expand pair of
 * RowParallelLinearWithShardedLoRA.apply on one device).  Same arguments as
 * lora_shrink and lora_expand.
 */
lora_status_t lora_apply_packed(void *y, int64_t ldy, int64_t y_col_offset, const void *x,
                                int64_t ldx, int32_t T, int32_t K, const void *const *A,
                                const void *const *B, const int64_t *N, int32_t S, int32_t L,
                                int32_t R, const int32_t *idx, const int32_t *slot_rank,
                                const float *scale, int32_t dtype, int32_t path, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * The path lora_apply_packed would take for these arguments (one of
 * LORA_PATH_TOKEN, RELAY, FUSED, GROUPED, PREFILL, DECODE), after the same checks,
 * without enqueueing anything.  Returns what lora_apply_packed would return
 * for a bad argument.
 */
lora_status_t lora_plan_packed(const void *y, int64_t ldy, int64_t y_col_offset, const void *x,
                               int64_t ldx, int32_t T, int32_t K, const void *const *A,
                               const void *const *B, const int64_t *N, int32_t S, int32_t L,
                               int32_t R, const int32_t *idx, const int32_t *slot_rank,
                               const float *scale, int32_t dtype, int32_t path, uint32_t flags,
                               const void *ws, size_t ws_bytes, int32_t *chosen_path);

/*
 * lora_apply_packed without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing and calls no
 * allocating routine.  Its scratch is one file-scope device array of
 * LORA_STATIC_SCRATCH_BYTES per GPU (held until the process ends), zero-filled
 * by the first call on each device (a fill kernel on `stream`).  Same
 * arguments and results as lora_apply_packed, with these differences:
 *   - a call whose workspace regions do not fit (lora_workspace_size() less
 *     its end region must fit in half the array, and the end region in the
 *     other half) returns LORA_E_SCRATCH before anything is enqueued; decode
 *     batches up to T 1024, K 8192, 3 slices, R 32 fit;
 *   - LORA_FLAG_SEGMENTS_READY is ignored: every call builds its segments;
 *   - every call on a GPU shares that GPU's array and leaves it as the next
 *     call needs it, so calls that overlap in time on one GPU (on different
 *     streams, or from different host threads) race; order them on one
 *     stream;
 *   - lora_workspace_check(NULL, 0, stream) reports a RELAY give-up in it.
 */
#define LORA_STATIC_SCRATCH_BYTES (32u << 20)
lora_status_t lora_apply_packed_noalloc(void *y, int64_t ldy, int64_t y_col_offset,
                                        const void *x, int64_t ldx, int32_t T, int32_t K,
                                        const void *const *A, const void *const *B,
                                        const int64_t *N, int32_t S, int32_t L, int32_t R,
                                        const int32_t *idx, const int32_t *slot_rank,
                                        const float *scale, int32_t dtype, int32_t path,
                                        uint32_t flags, void *stream);

/* ------------------------------------------------------------------------
 * Fused-MoE LoRA ([vLLM] FusedMoEWithLoRA; shared-outer layout from [PR]
 * item 4).  Items are the T * top_k (token, k) pairs p = t * top_k + j with
 * expert topk_ids[p]; pairs whose expert is outside [0, E) carry no delta.
 * bf16 only; R % 16 == 0; L * E <= 1024.
 * ------------------------------------------------------------------------ */
#define MOE_LORA_W13 0   /* delta into the pre-activation gate_up buffer     */
#define MOE_LORA_W2  1   /* delta into the per-(token, k) w2 output           */

/* Workspace bytes of moe_lora_align / moe_lora_apply for these sizes. */
lora_status_t moe_lora_workspace_size(int32_t T, int32_t top_k, int32_t S, int32_t R, int32_t L,
                                      int32_t E, size_t *bytes);

/* Entries per slot of moe_lora_align's padded output:
 * round_up(T * top_k + E * (block_m - 1), block_m). */
lora_status_t moe_lora_align_capacity(int32_t T, int32_t top_k, int32_t E, int32_t block_m,
                                      int32_t *cap);

/* Whether moe_lora_apply, called without LORA_FLAG_SEGMENTS_READY for T
 * tokens, top_k, rank R and reduce_k, takes the path without alignment
 * (*unsorted = 1; see moe_lora_apply) or builds the alignment in its
 * workspace (*unsorted = 0).  The same rule as moe_lora_apply; launches
 * nothing.  LORA_E_SHAPE when T < 0 or top_k < 1, LORA_E_NULL when unsorted
 * is NULL. */
lora_status_t moe_lora_plan(int32_t T, int32_t top_k, int32_t R, int32_t reduce_k,
                            int32_t *unsorted);

/*
 * Alignment ([vLLM] FusedMoEWithLoRA, the moe_lora_align_block_size call
 * and its per-slot views): groups the pairs of every slot by expert, experts
 * ascending, pair ids ascending inside an expert, each expert's run padded
 * with the sentinel T * top_k to a multiple of block_m.  The pages give only
 * the call; this layout is the plain reading of its outputs.
 *   sorted_ids      device int32 [L][cap]          pair ids and sentinels
 *   block_expert    device int32 [L][cap / block_m] expert of each block, -1 unused
 *   num_post_padded device int32 [L]                used entries per slot
 * The three outputs may all be NULL: the call then only builds, in `ws`, the
 * token and pair segments that moe_lora_apply reuses with
 * LORA_FLAG_SEGMENTS_READY (the w2 hook reuses the w13 hook's alignment).
 */
lora_status_t moe_lora_align(const int32_t *topk_ids, const int32_t *idx, const int32_t *slot_rank,
                             int32_t T, int32_t top_k, int32_t E, int32_t L, int32_t R,
                             int32_t block_m, int32_t *sorted_ids, int32_t *block_expert,
                             int32_t *num_post_padded, void *ws, size_t ws_bytes, void *stream);

/*
 * Fused-MoE LoRA delta, in place.
 *   kind MOE_LORA_W13: x [T][ldx] hidden states; y [T*top_k][ldy] gate_up
 *       (slices side by side); y[p][off_s + n] += scale[s] * (x[t] A_s[s][ea]^T) B_s[s][e]^T
 *   kind MOE_LORA_W2:  x [T*top_k][ldx] activation output; y [T*top_k][ldy] w2 output,
 *       weighted by topk_w[p] (NULL = 1); with reduce_k (needs E_b == 1)
 *       y is [T][ldy] and receives the sum over the token's k pairs.
 *   A[s]: device [L][E_a][R][K] with E_a in {1, E}; B[s]: device [L][E_b][N[s]][R]
 *   with E_b in {1, E}; expert dim 1 = shared-outer (expert index pinned to 0).
 *   topk_ids device int32 [T][top_k]; topk_w device float [T][top_k] or NULL.
 * ws: moe_lora_workspace_size() bytes; flags: LORA_FLAG_SEGMENTS_READY when
 * ws holds this batch's alignment (moe_lora_align or a previous apply).
 * Without that flag, a call of at most 1024 pairs at R == 16 without reduce_k
 * skips the alignment ([vLLM] FusedMoEWithLoRA's naive regime for small
 * batches): one work-group per (pair, chunk of 512, 1024 or 2048 output
 * columns of a slice); moe_lora_plan reports which.  Small batches that are
 * aligned run their shrink split over K.
 */
lora_status_t moe_lora_apply(int32_t kind, void *y, int64_t ldy, int32_t reduce_k, const void *x,
                             int64_t ldx, int32_t T, int32_t top_k, int32_t K,
                             const void *const *A, int32_t E_a, const void *const *B, int32_t E_b,
                             const int64_t *N, int32_t S, int32_t E, int32_t L, int32_t R,
                             const int32_t *topk_ids, const float *topk_w, const int32_t *idx,
                             const int32_t *slot_rank, const float *scale, int32_t dtype,
                             uint32_t flags, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ADAPTER_APPLY_H */
