/*
 * CPU oracle for the multi-LoRA delta -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library.  It shares no code with the HIP library: it is a plain
 * fp32 loop over tokens, written from the definitions on the pages, built
 * with -O2 -ffp-contract=off (no FMA contraction, no fast-math) so that every
 * multiply and add is a separately rounded IEEE fp32 operation in the order
 * written here.
 *
 * Sources (cited by page title and section):
 *   [vLLM]  "vllm.lora.layers" API page.
 *   [SGL]   SGLang "lora_manager.py" source page.
 *   [PR]    "PR #48884 report" page on vLLM's Inkling LoRA support.
 *
 * Conventions shared by every function:
 *   - lora_a of slice sigma is [L][R][K] row-major, lora_b is [L][N_sigma][R]
 *     ([vLLM] MergedColumnParallelLinearWithLoRA, create_lora_weights; the
 *     page's singleton second dim is dropped).
 *   - A token whose slot index is negative, >= L, or names a slot of rank 0
 *     carries no adapter and its output row is not touched ([vLLM] the
 *     adapter_enabled vector of max_loras+1 entries, FusedMoEWithLoRA
 *     create_lora_weights; [SGL] prepare_lora_batch, rank 0 for the base
 *     model's slot).
 *   - Rank j of slot s is used only for j < slot_rank[s]; the stored slot is
 *     zero beyond its rank ([vLLM] reset_lora followed by set_lora).
 *   - scale[s] multiplies the expand result once per output element ([SGL]
 *     prepare_lora_batch passes per-slot scalings; [vLLM] passes 1.0 to
 *     add_shrink, so the scale is not folded into the shrink).
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static int slot_of(const int32_t *idx, const int32_t *slot_rank, int32_t L,
                   int32_t R, int64_t t, int32_t *rank) {
    int32_t s = idx[t];
    if (s < 0 || s >= L) return -1;
    int32_t r = slot_rank ? slot_rank[s] : R;
    if (r <= 0) return -1;
    if (r > R) r = R;
    *rank = r;
    return s;
}

/*
 * Shrink ([vLLM] RowParallelLinearWithShardedLoRA.apply: a float32 buffer of
 * shape (n_slices, tokens, rank) is zero-filled and add_shrink accumulates
 * x . lora_a^T into it with scale 1.0).
 *   buf[sig][t][j] = sum_{i<K} x[t][i] * A_sig[s][j][i]     for j < rank(s)
 *   buf[sig][t][j] = 0                                       otherwise
 * buf is [S][T][R]; the sum runs over i ascending in one fp32 accumulator.
 */
void oracle_lora_shrink(float *buf, const float *x, int64_t ldx, int32_t T, int32_t K,
                        const float *const *A, int32_t S, int32_t L, int32_t R,
                        const int32_t *idx, const int32_t *slot_rank) {
    memset(buf, 0, sizeof(float) * (size_t)S * (size_t)T * (size_t)R);
    for (int64_t t = 0; t < T; ++t) {
        int32_t r;
        int32_t s = slot_of(idx, slot_rank, L, R, t, &r);
        if (s < 0) continue;
        const float *xr = x + t * ldx;
        for (int32_t sig = 0; sig < S; ++sig) {
            for (int32_t j = 0; j < r; ++j) {
                const float *ar = A[sig] + ((int64_t)s * R + j) * K;
                float acc = 0.0f;
                for (int32_t i = 0; i < K; ++i) acc = acc + xr[i] * ar[i];
                buf[((int64_t)sig * T + t) * R + j] = acc;
            }
        }
    }
}

/*
 * Expand ([vLLM] RowParallelLinearWithShardedLoRA.apply, the add_expand call
 * with output_slices, offset_start and add_input=True; the slices of a merged
 * layer sit side by side in the output, MergedColumnParallelLinearWithLoRA and
 * MergedQKVParallelLinearWithLoRA sections):
 *   off_sig = y_col_offset + sum_{sig' < sig} N[sig']
 *   d = sum_{j < rank(s)} buf[sig][t][j] * B_sig[s][n][j]     (j ascending)
 *   y[t][off_sig + n] = y[t][off_sig + n] + scale[s] * d
 * y is fp32 [T][ldy] and is kept in fp32 (no rounding to a storage type).
 */
void oracle_lora_expand(float *y, int64_t ldy, int64_t y_col_offset, const float *buf,
                        int32_t T, const float *const *B, const int64_t *N, int32_t S,
                        int32_t L, int32_t R, const int32_t *idx, const int32_t *slot_rank,
                        const float *scale) {
    for (int64_t t = 0; t < T; ++t) {
        int32_t r;
        int32_t s = slot_of(idx, slot_rank, L, R, t, &r);
        if (s < 0) continue;
        float *yr = y + t * ldy;
        int64_t off = y_col_offset;
        for (int32_t sig = 0; sig < S; ++sig) {
            const float *b = buf + ((int64_t)sig * T + t) * R;
            for (int64_t n = 0; n < N[sig]; ++n) {
                const float *br = B[sig] + ((int64_t)s * N[sig] + n) * R;
                float d = 0.0f;
                for (int32_t j = 0; j < r; ++j) d = d + b[j] * br[j];
                yr[off + n] = yr[off + n] + scale[s] * d;
            }
            off += N[sig];
        }
    }
}

/*
 * Packed apply: the shrink into a zero-filled fp32 buffer followed by the
 * expand into the base layer's output, as in the apply body of
 * [vLLM] RowParallelLinearWithShardedLoRA (single device: no all-reduce).
 * buf_out ([S][T][R], caller-owned) receives the intermediate buffer.
 */
void oracle_lora_apply(float *y, int64_t ldy, int64_t y_col_offset, const float *x,
                       int64_t ldx, int32_t T, int32_t K, const float *const *A,
                       const float *const *B, const int64_t *N, int32_t S, int32_t L,
                       int32_t R, const int32_t *idx, const int32_t *slot_rank,
                       const float *scale, float *buf_out) {
    oracle_lora_shrink(buf_out, x, ldx, T, K, A, S, L, R, idx, slot_rank);
    oracle_lora_expand(y, ldy, y_col_offset, buf_out, T, B, N, S, L, R, idx, slot_rank,
                       scale);
}

/*
 * Segment build: active tokens (see slot_of) sorted stably by slot, the
 * token grouping that segmented LoRA GEMMs work on ([SGL] the header's
 * S-LoRA/Punica credit and the "triton" backend's segment kernels;
 * prepare_lora_batch builds the per-request slot list once per batch).
 *   slot_start[s]   = number of active tokens with slot < s   (L+1 entries)
 *   perm[slot_start[s] .. slot_start[s+1]) = tokens of slot s, ascending
 *   *n_invalid      = number of tokens whose index is >= L
 * perm has room for T entries; entries past slot_start[L] are set to -1.
 */
void oracle_segments(const int32_t *idx, const int32_t *slot_rank, int32_t T, int32_t L,
                     int32_t R, int32_t *perm, int32_t *slot_start, int32_t *n_invalid) {
    int32_t inv = 0;
    for (int32_t s = 0; s <= L; ++s) slot_start[s] = 0;
    for (int32_t t = 0; t < T; ++t) {
        int32_t r;
        if (idx[t] >= L) ++inv;
        int32_t s = slot_of(idx, slot_rank, L, R, t, &r);
        if (s >= 0) slot_start[s + 1] += 1;
    }
    for (int32_t s = 0; s < L; ++s) slot_start[s + 1] += slot_start[s];
    for (int32_t t = 0; t < T; ++t) perm[t] = -1;
    int32_t pos = 0;
    for (int32_t s = 0; s < L; ++s) {
        for (int32_t t = 0; t < T; ++t) {
            int32_t r;
            if (slot_of(idx, slot_rank, L, R, t, &r) == s) perm[pos++] = t;
        }
    }
    *n_invalid = inv;
}

/*
 * MoE alignment: for each slot s carrying an adapter, the (token, k) pair ids
 * p = t*k + j with idx[t] == s grouped by expert topk_ids[t][j] (experts
 * ascending, pair ids ascending within an expert), each expert's run padded
 * with the sentinel T*k up to a multiple of block_m ([vLLM]
 * FusedMoEWithLoRA, the moe_lora_align_block_size call and the per-slot
 * views of sorted_token_ids_lora / expert_ids_lora; the page gives only the
 * call, this is the plain reading of its outputs).
 *   sorted_ids[s][0 .. num_post_padded[s])  pair ids and sentinels
 *   block_expert[s][b] = expert of block b, -1 for unused blocks
 * cap entries per slot are written (unused ones hold the sentinel); pairs
 * whose expert is outside [0, E) are dropped.
 */
void oracle_moe_align(const int32_t *topk_ids, const int32_t *idx, const int32_t *slot_rank,
                      int32_t T, int32_t k, int32_t E, int32_t L, int32_t R, int32_t block_m,
                      int32_t cap, int32_t *sorted_ids, int32_t *block_expert,
                      int32_t *num_post_padded) {
    const int32_t P = T * k;
    const int32_t nb = cap / block_m;
    for (int32_t s = 0; s < L; ++s) {
        int32_t *so = sorted_ids + (int64_t)s * cap;
        int32_t *be = block_expert + (int64_t)s * nb;
        for (int32_t i = 0; i < cap; ++i) so[i] = P;
        for (int32_t b = 0; b < nb; ++b) be[b] = -1;
        int32_t pos = 0;
        int32_t active = (slot_rank ? slot_rank[s] : R) > 0;
        if (active) {
            for (int32_t e = 0; e < E; ++e) {
                int32_t start = pos;
                for (int32_t p = 0; p < P; ++p) {
                    if (idx[p / k] == s && topk_ids[p] == e) so[pos++] = p;
                }
                if (pos > start) {
                    while (pos % block_m) so[pos++] = P;
                    for (int32_t b = start / block_m; b < pos / block_m; ++b) be[b] = e;
                }
            }
        }
        num_post_padded[s] = pos;
    }
}

/*
 * Fused-MoE LoRA delta ([vLLM] FusedMoEWithLoRA: the activation hook adds
 * the w13 delta into the pre-activation gate_up buffer, the moe_sum hook adds
 * the w2 delta into the per-(token, k) w2 output, then sums over k; the
 * positional True passed in the w2 call is read as "multiply by the routing
 * weight").  Shared-outer layout ([PR] item 4: w13 lora_a and w2 lora_b have
 * expert dim 1 and the expert index is pinned to 0).
 *
 *   kind 0 (w13): input row x[t] ([T][K]); output row y[t*k + j]
 *   kind 1 (w2) : input row x[t*k + j] ([T*k][K]); output row y[t*k + j], or
 *                 y[t] when reduce_k (sum over j ascending)
 *   A[sig] : [L][E_a][R][K], expert e_a = (E_a == 1 ? 0 : e)
 *   B[sig] : [L][E_b][N_sig][R], expert e_b = (E_b == 1 ? 0 : e)
 *   coef   = scale[s] (kind 1 with topk_w: scale[s] * topk_w[t][j])
 *   y[row][off_sig + n] += coef * sum_j (sum_i xrow[i] A[s][e_a][j][i]) * B[s][e_b][n][j]
 */
void oracle_moe_lora_apply(int32_t kind, float *y, int64_t ldy, int32_t reduce_k,
                           const float *x, int64_t ldx, int32_t T, int32_t k, int32_t K,
                           const float *const *A, int32_t E_a, const float *const *B,
                           int32_t E_b, const int64_t *N, int32_t S, int32_t E, int32_t L,
                           int32_t R, const int32_t *topk_ids, const float *topk_w,
                           const int32_t *idx, const int32_t *slot_rank, const float *scale,
                           float *bvec /* scratch, R floats */) {
    for (int64_t t = 0; t < T; ++t) {
        int32_t r;
        int32_t s = slot_of(idx, slot_rank, L, R, t, &r);
        if (s < 0) continue;
        for (int32_t j = 0; j < k; ++j) {
            int64_t p = t * k + j;
            int32_t e = topk_ids[p];
            if (e < 0 || e >= E) continue;
            int32_t ea = (E_a == 1) ? 0 : e;
            int32_t eb = (E_b == 1) ? 0 : e;
            const float *xr = x + (kind == 0 ? t : p) * ldx;
            float *yr = y + ((kind == 1 && reduce_k) ? t : p) * ldy;
            float coef = scale[s];
            if (kind == 1 && topk_w) coef = coef * topk_w[p];
            int64_t off = 0;
            for (int32_t sig = 0; sig < S; ++sig) {
                const float *a = A[sig] + (((int64_t)s * E_a + ea) * R) * K;
                const float *b = B[sig] + (((int64_t)s * E_b + eb) * N[sig]) * R;
                for (int32_t q = 0; q < r; ++q) {
                    float acc = 0.0f;
                    for (int32_t i = 0; i < K; ++i) acc = acc + xr[i] * a[(int64_t)q * K + i];
                    bvec[q] = acc;
                }
                for (int64_t n = 0; n < N[sig]; ++n) {
                    float d = 0.0f;
                    for (int32_t q = 0; q < r; ++q) d = d + bvec[q] * b[n * R + q];
                    yr[off + n] = yr[off + n] + coef * d;
                }
                off += N[sig];
            }
        }
    }
}
