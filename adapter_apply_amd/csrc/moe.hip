// Fused-MoE LoRA: (token, k) alignment by (slot, expert) and the w13 / w2
// deltas, on the grouped MFMA kernels.  Declarations and contracts:
// include/adapter_apply.h.
#include "../../include/adapter_apply.h"
#include "common.hpp"

namespace aa {

namespace {

constexpr int kAlignThreads = 256;

// Per slot (blockIdx.y): the pair ids of each expert in ascending order (the
// pair segments), each run padded with the sentinel T*k to a multiple of bm,
// the expert of every block, and the padded length.  Work-group blockIdx.x
// fills positions [256 x, 256 x + 256) of the slot; the padded offsets of the
// slot's experts come from a block scan (E <= 1024).
__global__ __launch_bounds__(kAlignThreads) void k_moe_align_out(SegPtrs pair, int32_t T, int32_t k,
                                                                 int32_t E, int32_t bm, int32_t cap,
                                                                 int32_t *sorted_ids,
                                                                 int32_t *block_expert,
                                                                 int32_t *num_post_padded) {
    extern __shared__ int32_t off[];   // [E + 1] padded offsets of the experts in this slot
    __shared__ int32_t wsum[kAlignThreads / kWave + 1];
    const int s = blockIdx.y;
    const int P = T * k;
    const int32_t *start = pair.slot_start + (int64_t)s * E;   // key s * E + e
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // exclusive scan of the padded run lengths, E in chunks of 256
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kAlignThreads) {
        const int e = e0 + tid;
        const int c = e < E ? start[e + 1] - start[e] : 0;
        const int v = (c + bm - 1) / bm * bm;
        int incl = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        if (lane == kWave - 1) wsum[w] = incl;
        __syncthreads();
        int before = 0;
        for (int q = 0; q < w; ++q) before += wsum[q];
        int chunk_total = 0;
        for (int q = 0; q < kAlignThreads / kWave; ++q) chunk_total += wsum[q];
        if (e < E) off[e] = carry + before + incl - v;
        carry += chunk_total;
        __syncthreads();
    }
    if (tid == 0) {
        off[E] = carry;
        if (blockIdx.x == 0) num_post_padded[s] = carry;
    }
    __syncthreads();
    const int total = off[E];
    const int i = blockIdx.x * kAlignThreads + tid;
    if (i >= cap) return;
    int32_t *so = sorted_ids + (int64_t)s * cap;
    int32_t *be = block_expert + (int64_t)s * (cap / bm);
    int v = P;
    if (i < total) {
        int lo = 0, hi = E - 1;                 // expert e with off[e] <= i < off[e+1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int j = i - off[lo];
        if (j < start[lo + 1] - start[lo]) v = pair.perm[start[lo] + j];
        if (i % bm == 0) be[i / bm] = lo;
    } else if (i % bm == 0) {
        be[i / bm] = -1;
    }
    so[i] = v;
}

}  // namespace

hipError_t launch_moe_align_out(const SegPtrs &pair, int32_t T, int32_t k, int32_t E, int32_t L,
                                int32_t bm, int32_t *sorted_ids, int32_t *block_expert,
                                int32_t *num_post_padded, hipStream_t st) {
    const int cap = moe_align_capacity(T, k, E, bm);
    const dim3 grid((unsigned)((cap + kAlignThreads - 1) / kAlignThreads), (unsigned)L);
    hipLaunchKernelGGL(k_moe_align_out, grid, dim3(kAlignThreads), sizeof(int32_t) * (E + 1), st,
                       pair, T, k, E, bm, cap, sorted_ids, block_expert, num_post_padded);
    return hipGetLastError();
}

}  // namespace aa

using namespace aa;

namespace {

inline bool al(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline lora_status_t launched(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_E_LAUNCH; }

#define CHECK(expr)                          \
    do {                                     \
        lora_status_t _st = (expr);          \
        if (_st != LORA_OK) return _st;      \
    } while (0)

lora_status_t moe_check_meta(int32_t T, int32_t k, int32_t E, int32_t L, int32_t R) {
    if (T < 0 || k < 1 || E < 1 || L < 1 || L > LORA_MAX_SLOTS) return LORA_E_SHAPE;
    if ((int64_t)L * E > 1024) return LORA_E_SHAPE;           // slot-expert keys sorted in one pass
    if ((int64_t)T * k > (1 << 30)) return LORA_E_SHAPE;
    if (R < 1 || R > LORA_MAX_RANK) return LORA_E_RANK;
    if (max_tiles(T * k, L * E, kDecTile) > (1 << 24)) return LORA_E_SHAPE;
    return LORA_OK;
}

lora_status_t moe_segments(const int32_t *topk_ids, const int32_t *idx, const int32_t *slot_rank,
                           int32_t T, int32_t k, int32_t E, int32_t L, int32_t R,
                           const MoeWsLayout &ml, void *ws, size_t ws_bytes, hipStream_t st) {
    if (T == 0) {
        CHECK(launched(launch_segments_keyed(idx, slot_rank, nullptr, 1, 1, T, L, R,
                                             seg_ptrs(ws, ml.tok), st)));
        return launched(launch_segments_keyed(idx, slot_rank, topk_ids, k, E, T * k, L, R,
                                              seg_ptrs(ws, ml.pair), st));
    }
    // the token and the (token, k) pair segments together: one launch when
    // their exchange regions fit in the end area (above the buffers), else a
    // pair of launches
    SegPtrs tok = seg_ptrs(ws, ml.tok), pair = seg_ptrs(ws, ml.pair);
    const size_t xp = seg_x_bytes(T * k, L * E), xt = seg_x_bytes(T, L);
    const size_t floor = ml.end - xp - xt - 256;
    attach_seg_x(pair, ws, ws_bytes, T * k, L * E, 0, floor);
    attach_seg_x(tok, ws, ws_bytes, T, L, xp, floor);
    const SegJob jobs[2] = {seg_job_of(nullptr, 1, 1, T, tok), seg_job_of(topk_ids, k, E, T * k, pair)};
    return launched(launch_segments_split(idx, slot_rank, L, R, jobs, 2, st));
}

}  // namespace

extern "C" {

lora_status_t moe_lora_workspace_size(int32_t T, int32_t top_k, int32_t S, int32_t R, int32_t L,
                                      int32_t E, size_t *bytes) {
    if (!bytes) return LORA_E_NULL;
    CHECK(moe_check_meta(T, top_k, E, L, R));
    if (S < 1 || S > LORA_MAX_SLICES) return LORA_E_SLICES;
    *bytes = moe_ws_layout(T, top_k, S, R, L, E).end;
    return LORA_OK;
}

lora_status_t moe_lora_align_capacity(int32_t T, int32_t top_k, int32_t E, int32_t block_m,
                                      int32_t *cap) {
    if (!cap) return LORA_E_NULL;
    if (T < 0 || top_k < 1 || E < 1 || block_m < 1) return LORA_E_SHAPE;
    *cap = moe_align_capacity(T, top_k, E, block_m);
    return LORA_OK;
}

lora_status_t moe_lora_plan(int32_t T, int32_t top_k, int32_t R, int32_t reduce_k,
                            int32_t *unsorted) {
    if (!unsorted) return LORA_E_NULL;
    if (T < 0 || top_k < 1) return LORA_E_SHAPE;
    *unsorted = moe_small_takes((int32_t)std::min<int64_t>((int64_t)T * top_k, INT32_MAX), R,
                                reduce_k) ? 1 : 0;
    return LORA_OK;
}

lora_status_t moe_lora_align(const int32_t *topk_ids, const int32_t *idx, const int32_t *slot_rank,
                             int32_t T, int32_t top_k, int32_t E, int32_t L, int32_t R,
                             int32_t block_m, int32_t *sorted_ids, int32_t *block_expert,
                             int32_t *num_post_padded, void *ws, size_t ws_bytes, void *stream) {
    CHECK(moe_check_meta(T, top_k, E, L, R));
    if (block_m < 1) return LORA_E_SHAPE;
    if (T > 0 && (!topk_ids || !idx)) return LORA_E_NULL;
    const bool want_out = sorted_ids || block_expert || num_post_padded;
    if (want_out && !(sorted_ids && block_expert && num_post_padded)) return LORA_E_NULL;
    if (!ws) return LORA_E_NULL;
    if (!al(ws, 256)) return LORA_E_ALIGN;
    const MoeWsLayout ml = moe_ws_layout(T, top_k, 1, R, L, E);
    if (ws_bytes < ml.pair.end) return LORA_E_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    CHECK(moe_segments(topk_ids, idx, slot_rank, T, top_k, E, L, R, ml, ws, ws_bytes, st));
    if (!want_out) return LORA_OK;
    return launched(launch_moe_align_out(seg_ptrs(ws, ml.pair), T, top_k, E, L, block_m, sorted_ids,
                                         block_expert, num_post_padded, st));
}

lora_status_t moe_lora_apply(int32_t kind, void *y, int64_t ldy, int32_t reduce_k, const void *x,
                             int64_t ldx, int32_t T, int32_t top_k, int32_t K,
                             const void *const *A, int32_t E_a, const void *const *B, int32_t E_b,
                             const int64_t *N, int32_t S, int32_t E, int32_t L, int32_t R,
                             const int32_t *topk_ids, const float *topk_w, const int32_t *idx,
                             const int32_t *slot_rank, const float *scale, int32_t dtype,
                             uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
    if (kind != MOE_LORA_W13 && kind != MOE_LORA_W2) return LORA_E_SHAPE;
    if (dtype != LORA_DT_BF16) return LORA_E_DTYPE;
    CHECK(moe_check_meta(T, top_k, E, L, R));
    if (R % 16) return LORA_E_ALIGN;
    if (S < 1 || S > LORA_MAX_SLICES) return LORA_E_SLICES;
    if (K < 1 || ldx < K) return LORA_E_SHAPE;
    if (K % 8 || ldx % 8) return LORA_E_ALIGN;
    if ((E_a != 1 && E_a != E) || (E_b != 1 && E_b != E)) return LORA_E_SHAPE;
    if (reduce_k && (kind != MOE_LORA_W2 || E_b != 1)) return LORA_E_SHAPE;
    if (!N) return LORA_E_NULL;
    int64_t ntot = 0;
    for (int s = 0; s < S; ++s) {
        if (N[s] < 1) return LORA_E_SHAPE;
        if (N[s] % 4) return LORA_E_ALIGN;
        ntot += N[s];
    }
    if (ldy < ntot) return LORA_E_SHAPE;
    if (ldy % 4) return LORA_E_ALIGN;
    if (T == 0) return LORA_OK;
    if (!y || !x || !idx || !scale || !topk_ids || !A || !B) return LORA_E_NULL;
    for (int s = 0; s < S; ++s) {
        if (!A[s] || !B[s]) return LORA_E_NULL;
        if (!al(A[s], 16) || !al(B[s], 16)) return LORA_E_ALIGN;
    }
    if (!al(y, 16) || !al(x, 16)) return LORA_E_ALIGN;
    if (!ws) return LORA_E_NULL;
    if (!al(ws, 256)) return LORA_E_ALIGN;
    const MoeWsLayout ml = moe_ws_layout(T, top_k, S, R, L, E);
    if (ws_bytes < ml.end) return LORA_E_WORKSPACE;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int32_t P = T * top_k;
    if (!(flags & LORA_FLAG_SEGMENTS_READY) && moe_small_takes(P, R, reduce_k)) {
        // a few pairs: no alignment, one work-group per (pair, column chunk)
        Slices s1{};
        int64_t o = 0;
        for (int s = 0; s < S; ++s) {
            s1.a[s] = A[s]; s1.b[s] = B[s]; s1.n[s] = N[s]; s1.off[s] = o; o += N[s];
        }
        for (int s = S; s <= kMaxSlices; ++s) s1.off[s] = o;
        const bool w13 = kind == MOE_LORA_W13;
        return launched(launch_moe_small(y, ldy, x, ldx, T, top_k, K, s1, S, E, L, R, E_a, E_b,
                                         w13 ? top_k : 1, topk_ids, w13 ? nullptr : topk_w, idx,
                                         slot_rank, scale, st));
    }
    if (!(flags & LORA_FLAG_SEGMENTS_READY))
        CHECK(moe_segments(topk_ids, idx, slot_rank, T, top_k, E, L, R, ml, ws, ws_bytes, st));
    const SegPtrs tok = seg_ptrs(ws, ml.tok), pair = seg_ptrs(ws, ml.pair);
    float *buf = reinterpret_cast<float *>(static_cast<char *>(ws) + ml.buf);
    Slices sl{};
    int64_t off = 0;
    for (int s = 0; s < S; ++s) {
        sl.a[s] = A[s]; sl.b[s] = B[s]; sl.n[s] = N[s]; sl.off[s] = off; off += N[s];
    }
    for (int s = S; s <= kMaxSlices; ++s) sl.off[s] = off;

    GroupMap sh, ex;
    const SegPtrs *sh_seg, *ex_seg;
    if (kind == MOE_LORA_W13 && E_a == 1) {
        // shared lora_a: one shrink per token, the expand per (token, k) pair
        sh.Ekey = 1; sh.Ew = 1; sh.buf_rows = T; sh_seg = &tok;
        ex.Ekey = E; ex.Ew = E_b; ex.buf_div = top_k; ex.buf_rows = T; ex_seg = &pair;
    } else {
        // per-expert lora_a: the shrink per pair (w13 reads x of the pair's token)
        sh.Ekey = E; sh.Ew = E_a; sh.x_div = kind == MOE_LORA_W13 ? top_k : 1; sh.buf_rows = P;
        sh_seg = &pair;
        if (reduce_k) {
            // sum_j w[t,j] * buf[t*k + j], expanded once per token with the shared lora_b
            ex.Ekey = 1; ex.Ew = 1; ex.buf_rows = P; ex.coef = topk_w; ex.ksum = top_k;
            ex_seg = &tok;
        } else if (kind == MOE_LORA_W2 && E_b == 1) {
            // one lora_b for every expert ([PR] shared-outer): the expand
            // needs the pairs grouped by slot only, and a token's pairs share
            // its slot, so it walks full runs of 64 pairs of the token tiles
            // instead of the (slot, expert) tiles, half empty on average
            ex.Ekey = 1; ex.Ew = 1; ex.buf_rows = P; ex.coef = topk_w;
            ex.pair_k = top_k; ex.pair_ids = topk_ids; ex.pair_E = E;
            ex_seg = &tok;
        } else {
            ex.Ekey = E; ex.Ew = E_b; ex.buf_rows = P;
            ex.coef = kind == MOE_LORA_W2 ? topk_w : nullptr;
            ex_seg = &pair;
        }
    }
    // A small batch has few tiles, each streaming all of K through one CU:
    // the shrink is then split over K into partials in the workspace, summed
    // in order into the buffer by the reduce kernel.
    const int32_t n_items = sh.buf_rows;                   // tokens or (token, k) pairs
    int32_t kspl = 1;
    if (n_items <= kMoeSplitItems) {
        const int32_t cap = (int32_t)(ml.part_bytes / (sizeof(float) * (size_t)n_items * S * R));
        kspl = pre_kspl(n_items, K, S, R, L * sh.Ekey, sh_seg->max_tiles_pre, cap);
    }
    if (kspl > 1) {
        float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + ml.part);
        CHECK(launched(launch_pre_shrink(x, ldx, T, K, sl, S, L, R, slot_rank, *sh_seg, nullptr, st, sh,
                                         part, &kspl)));
        CHECK(launched(launch_grp_reduce(n_items, S, L, R, idx, slot_rank, part, kspl, buf, sh_seg, st,
                                         sh.Ekey)));
    } else {
        CHECK(launched(launch_pre_shrink(x, ldx, T, K, sl, S, L, R, slot_rank, *sh_seg, buf, st, sh)));
    }
    return launched(launch_pre_expand(y, ldy, buf, T, sl, S, L, R, slot_rank, scale, *ex_seg, st, ex));
}

}  // extern "C"
