// C-ABI entry points: argument checks (all before any launch), workspace
// carving and path dispatch.  Declarations and contracts: include/adapter_apply.h.
#include <cmath>

#include "../../include/adapter_apply.h"
#include "common.hpp"

using namespace aa;

namespace {

// Auto path: MFMA prefill once slots carry long token runs.
constexpr int32_t kPrefillMinTokens = 512;
constexpr int32_t kPrefillMinPerSlot = 64;
// Decode: the expand adds the shrink's K-chunk partials itself (one launch
// fewer) while a tile's partials stay small; beyond that a reduce kernel runs.
constexpr int32_t kFoldMaxChunkRank = 512;   // n_kchunks * R
// Auto's K-split single launch for narrow outputs: expected 32-token groups at
// most this many, or at least this many tokens per slot that draws any.
constexpr double kRelayFewGroups = 12.0;
constexpr double kRelayMinPerSlot = 24.0;
// Auto: the grouped kernels at rank 16 for narrow outputs up to this many tokens.
constexpr int32_t kGrpR16MaxTokens = 4096;

inline bool al(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline lora_status_t launched(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_E_LAUNCH; }

lora_status_t check_sizes(int32_t T, int32_t S, int32_t L, int32_t R, int32_t dtype) {
    if (dtype != LORA_DT_F32 && dtype != LORA_DT_BF16) return LORA_E_DTYPE;
    if (T < 0 || L < 1 || L > LORA_MAX_SLOTS) return LORA_E_SHAPE;
    if (R < 1 || R > LORA_MAX_RANK) return LORA_E_RANK;
    if (S < 1 || S > LORA_MAX_SLICES) return LORA_E_SLICES;
    if (R % (dtype == LORA_DT_BF16 ? 8 : 4)) return LORA_E_ALIGN;
    // decode tiles index grid.y / grid.z
    if (max_tiles(T, L, kDecTile) > 65535) return LORA_E_SHAPE;
    return LORA_OK;
}

lora_status_t check_k(int32_t K, int64_t ldx) {
    if (K < 1 || ldx < K) return LORA_E_SHAPE;
    if (K % 8 || ldx % 8) return LORA_E_ALIGN;
    return LORA_OK;
}

lora_status_t check_n(const int64_t *N, int32_t S, int64_t ldy, int64_t y_col_offset,
                      int64_t *total) {
    if (!N) return LORA_E_NULL;
    int64_t t = 0;
    for (int s = 0; s < S; ++s) {
        if (N[s] < 1) return LORA_E_SHAPE;
        if (N[s] % 4) return LORA_E_ALIGN;
        t += N[s];
    }
    if (y_col_offset < 0 || ldy < y_col_offset + t) return LORA_E_SHAPE;
    if (ldy % 4 || y_col_offset % 4) return LORA_E_ALIGN;
    *total = t;
    return LORA_OK;
}

lora_status_t check_ptrs(const void *const *P, int32_t S) {
    if (!P) return LORA_E_NULL;
    for (int s = 0; s < S; ++s) {
        if (!P[s]) return LORA_E_NULL;
        if (!al(P[s], 16)) return LORA_E_ALIGN;
    }
    return LORA_OK;
}

#define CHECK(expr)                          \
    do {                                     \
        lora_status_t _st = (expr);          \
        if (_st != LORA_OK) return _st;      \
    } while (0)

// y rows are read and written 16 bytes (8 columns) at a time
bool rows_of_8(const int64_t *N, int32_t S, int64_t ldy, int64_t y_col_offset) {
    if (ldy % 8 || y_col_offset % 8) return false;
    for (int s = 0; s < S; ++s)
        if (N[s] % 8) return false;
    return true;
}

bool can_fuse(int32_t T, int32_t K, int32_t R, const int64_t *N, int32_t S, int64_t ldy,
              int64_t y_col_offset, int32_t dtype) {
    if (dtype != LORA_DT_BF16 || R % 16 || R > kFusedMaxRank || T > kFusedMaxTokens) return false;
    if (K % 1024) return false;                  // 16 waves x whole 64-element lines of K
    return rows_of_8(N, S, ldy, y_col_offset);
}

// Single-launch decode with the shrink split over K (relay.hip): one-wave
// group discovery (L <= 64, T <= 1024), whole 256-column K chunks.
bool can_relay(int32_t T, int32_t K, int32_t R, int32_t L, const int64_t *N, int32_t S,
               int64_t ldy, int64_t y_col_offset, int32_t dtype) {
    if (dtype != LORA_DT_BF16 || (R != 16 && R != 32) || T > 1024 || L > 64) return false;
    if (K % kRelayKc || K / kRelayKc > kRelayMaxKc) return false;
    return rows_of_8(N, S, ldy, y_col_offset);
}

// Slot-grouped kernels: the shrink side (K) and the expand side (y rows).
bool can_group_sizes(int32_t T, int32_t R, int32_t dtype) {
    return dtype == LORA_DT_BF16 && R % 16 == 0 && R <= kGrpMaxRank && T <= kGrpMaxTokens;
}
bool can_group_k(int32_t K) { return K % 64 == 0 && grp_kchunks(K) <= kMaxKcGrp; }

bool can_group(int32_t T, int32_t K, int32_t R, const int64_t *N, int32_t S, int64_t ldy,
               int64_t y_col_offset, int32_t dtype) {
    return can_group_sizes(T, R, dtype) && can_group_k(K) && rows_of_8(N, S, ldy, y_col_offset);
}

// Workspace int32 that carries the grouped shrink's K-chunk count to a later
// expand call (slot 5 of the segment header; the segment kernel uses 0..4).
int32_t *grp_kc_slot(void *ws, const SegLayout &l) {
    return reinterpret_cast<int32_t *>(static_cast<char *>(ws) + l.header) + 5;
}

// The row-oriented MFMA shrink into the token-ordered buffer, split over K
// (partials, then the reduce kernel summing the splits in order) when
// pre_kspl says so.
lora_status_t pre_shrink_buf(const void *x, int64_t ldx, int32_t T, int32_t K, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, const SegPtrs &seg, const WsLayout &wl,
                             void *ws, float *buf, hipStream_t st) {
    int32_t kspl = pre_kspl(T, K, S, R, L, seg.max_tiles_pre, wl.n_kchunks);
    if (kspl <= 1)
        return launched(launch_pre_shrink(x, ldx, T, K, sl, S, L, R, slot_rank, seg, buf, st));
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.partial);
    CHECK(launched(launch_pre_shrink(x, ldx, T, K, sl, S, L, R, slot_rank, seg, nullptr, st,
                                     GroupMap(), part, &kspl)));
    return launched(launch_grp_reduce(T, S, L, R, idx, slot_rank, part, kspl, buf, &seg, st));
}

// Grouped shrink that writes K-chunk partials for the reduce kernel; the chunk
// count comes back in *n_kc.  With the segment table and ranks past the
// partial-sum limit, the row-oriented MFMA shrink runs split over K: it keeps
// loads in flight across K stages where the grouped shrink loads one
// 512-column chunk per work-group.
lora_status_t grp_shrink_part(const void *x, int64_t ldx, int32_t T, int32_t K, const Slices &sl,
                              int32_t S, int32_t L, int32_t R, const int32_t *idx,
                              const int32_t *slot_rank, float *part, const WsLayout &wl,
                              const SegPtrs *gseg, hipStream_t st, int32_t *n_kc) {
    if (gseg && R > kGrpMaxPartialRank) {
        int32_t kspl = pre_kspl(T, K, S, R, L, gseg->max_tiles_pre, wl.n_kchunks);
        const lora_status_t e = launched(launch_pre_shrink(x, ldx, T, K, sl, S, L, R, slot_rank,
                                                           *gseg, nullptr, st, GroupMap(), part, &kspl));
        *n_kc = kspl;
        return e;
    }
    *n_kc = grp_kchunks(K);
    return launched(launch_grp_shrink(x, ldx, T, K, sl, S, L, R, idx, slot_rank, part, nullptr,
                                      gseg, st));
}

// TOKEN's grid is T x (256-column chunks); each work-group reads its slot's
// K x R lora_a block.  It fits while a work-group reads at most 1 MB of
// lora_a and the rounds of 1024 work-groups (four per CU) times the 16-row
// passes of the rank stay within 4; auto takes it while the lora_a bytes of
// all work-groups stay within the dtype's bound.
// The grid's work-groups, or -1 past what one launch takes (2^31 - 1).
int64_t token_wgs(int32_t T, const int64_t *N, int32_t S) {
    int64_t c = 0;
    for (int s = 0; s < S; ++s) {
        c += (N[s] + kTokenCols - 1) / kTokenCols;
        if (c > INT32_MAX) return -1;
    }
    const int64_t w = (int64_t)T * c;
    return w > INT32_MAX ? -1 : w;
}
bool token_fits(int64_t wgs, int32_t K, int32_t R, int32_t dtype) {
    const int64_t a_wg = (int64_t)K * R * (dtype == LORA_DT_BF16 ? 2 : 4);
    const int64_t rounds = (wgs + kTokenRound - 1) / kTokenRound;
    return wgs >= 0 && a_wg <= kTokenMaxWgBytes && rounds * ((R + 15) / 16) <= kTokenMaxRoundPasses;
}

lora_status_t choose_path(int32_t path, int32_t T, int32_t L, int32_t R, int32_t dtype,
                          int *use_prefill) {
    const bool can_prefill = dtype == LORA_DT_BF16 && R % 16 == 0;
    if (path == LORA_PATH_DECODE || path == LORA_PATH_FUSED || path == LORA_PATH_GROUPED ||
        path == LORA_PATH_RELAY) {
        *use_prefill = 0;
        return LORA_OK;
    }
    if (path == LORA_PATH_PREFILL) {
        if (!can_prefill) return LORA_E_PATH;
        *use_prefill = 1;
        return LORA_OK;
    }
    if (path != LORA_PATH_AUTO) return LORA_E_PATH;
    const int32_t slots = T < L ? T : L;
    *use_prefill = can_prefill && T >= kPrefillMinTokens && slots > 0 &&
                   T / slots >= kPrefillMinPerSlot;
    return LORA_OK;
}

// Auto for lora_shrink / lora_expand called apart, without LORA_FLAG_PARTIAL:
// batches of many slots or high ranks take the tile kernels (the buffer
// between the calls is the same token-ordered fp32 [S][T][R] on every path, so
// the two calls need not agree on the path).
bool auto_tiles_apart(int32_t path, uint32_t flags, int32_t L, int32_t R, int32_t dtype) {
    return path == LORA_PATH_AUTO && !(flags & LORA_FLAG_PARTIAL) && dtype == LORA_DT_BF16 &&
           (L > 64 || R > 64) && (R == 16 || R == 32 || R == 64 || R == 128);
}

lora_status_t check_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (!ws) return LORA_E_NULL;
    if (!al(ws, 256)) return LORA_E_ALIGN;
    if (ws_bytes < need) return LORA_E_WORKSPACE;
    return LORA_OK;
}

Slices make_slices(const void *const *A, const void *const *B, const int64_t *N, int32_t S,
                   int64_t y_col_offset) {
    Slices sl{};
    int64_t off = y_col_offset;
    for (int s = 0; s < S; ++s) {
        sl.a[s] = A ? A[s] : nullptr;
        sl.b[s] = B ? B[s] : nullptr;
        sl.n[s] = N ? N[s] : 0;
        sl.off[s] = off;
        off += sl.n[s];
    }
    for (int s = S; s <= kMaxSlices; ++s) sl.off[s] = off;
    return sl;
}

}  // namespace

namespace aa {

// Every check of lora_apply_packed and its choice of path, on the host; it
// enqueues nothing.  The auto rule, the first that holds:
//   1. TOKEN while its work-groups' recomputed shrinks read little lora_a;
//   2. RELAY with a workspace of lora_workspace_size() bytes: for relay
//      batches of narrow outputs, and for every wide output it takes;
//   3. GROUPED at rank 16 for narrow outputs up to 4096 tokens and 128 slots;
//   4. PREFILL when slots carry long token runs (choose_path);
//   5. FUSED where its shapes allow, the output is narrow and L <= 64;
//   6. GROUPED where its shapes allow, L <= 64, R <= 64 and the output is
//      narrow;
//   7. PREFILL for bf16 with R in {16, 32, 64, 128} and rows of 8 columns;
//   8. DECODE.
// "Narrow": the slices sum to at most 16384 columns.
int32_t packed_plan(const void *y, int64_t ldy, int64_t y_col_offset, const void *x, int64_t ldx,
                    int32_t T, int32_t K, const void *const *A, const void *const *B,
                    const int64_t *N, int32_t S, int32_t L, int32_t R, const int32_t *idx,
                    const int32_t *slot_rank, const float *scale, int32_t dtype, int32_t path,
                    uint32_t flags, const void *ws, size_t ws_bytes, PackedPlan *out) {
    (void)slot_rank;
    (void)flags;
    CHECK(check_sizes(T, S, L, R, dtype));
    CHECK(check_k(K, ldx));
    int64_t ntot = 0;
    CHECK(check_n(N, S, ldy, y_col_offset, &ntot));
    // TOKEN (one work-group per token and 256 columns, each recomputing its
    // token's shrink) while the lora_a bytes those shrinks read stay small.
    // Measured with the inputs in HBM against RELAY on bf16: QKV shape 1 to
    // 12 tokens 5.5-6.9 against 6.3-7.3 us, 16 tokens 8.1 against 7.4, 24
    // tokens 9.4 against 7.5 (so narrow outputs that RELAY could take keep a
    // lower bound); a 32000-column lm_head at 4 tokens 7.4 against 7.6, 8
    // tokens 10.1 against 9.0; rank-64 gate_up at 1 token 11.9 against 21.5
    // for the grouped kernels (RELAY takes ranks 16 and 32 only).  Against
    // DECODE's three launches on fp32: QKV shape 80 tokens 28.3 against 31.1,
    // 96 tokens 33.6 against 31.4; hidden 64, 4096 tokens 8.0 against 22.0.
    const int64_t tok_wgs = token_wgs(T, N, S);
    if (path == LORA_PATH_TOKEN && tok_wgs < 0) return LORA_E_PATH;
    const bool relay_fits = can_relay(T, K, R, L, N, S, ldy, y_col_offset, dtype) && ws &&
                            ws_bytes >= ws_layout(T, K, S, R, L).end;
    const int64_t tok_max = dtype != LORA_DT_BF16             ? kTokenMaxBytesF32
                            : ntot <= kAutoMaxDecodeCols && relay_fits ? kTokenMaxBytesNarrow
                                                                    : kTokenMaxBytesBf16;
    // (token_fits bounds the work-groups to 4096 and each one's lora_a bytes
    // to 1 MB, so the product below stays far inside int64)
    const bool token = path == LORA_PATH_TOKEN ||
                       (path == LORA_PATH_AUTO && token_fits(tok_wgs, K, R, dtype) &&
                        tok_wgs * K * R * (dtype == LORA_DT_BF16 ? 2 : 4) <= tok_max);
    int use_prefill = 0;
    if (!token) CHECK(choose_path(path, T, L, R, dtype, &use_prefill));
    if (token) {
        out->path = LORA_PATH_TOKEN;
        out->shared_a = 0;
        out->noop = T == 0 ? 1 : 0;
        if (T == 0) return LORA_OK;
        if (!y || !x || !idx || !scale) return LORA_E_NULL;
        CHECK(check_ptrs(A, S));
        CHECK(check_ptrs(B, S));
        if (!al(y, 16) || !al(x, 16)) return LORA_E_ALIGN;
        return LORA_OK;   // no workspace needed
    }
    // Auto takes the single-launch kernel with the K-split shrink when the
    // workspace is there: for decode batches of narrow outputs, and for every
    // wide output (an lm_head's vocabulary) it takes, where its 16-token
    // expand items of up to four column chunks beat the tile kernels.
    // Without a workspace narrow outputs take the other single-launch kernel,
    // and wide outputs go to the tile kernels (the single-launch kernel
    // without a workspace recomputes a group's shrink for every 1024-column
    // chunk).
    const bool narrow = ntot <= kAutoMaxDecodeCols;
    const bool relay_ok = can_relay(T, K, R, L, N, S, ldy, y_col_offset, dtype);
    if (path == LORA_PATH_RELAY && !relay_ok) return LORA_E_PATH;
    // The K-split single launch runs a fixed set of work-groups per 32-token
    // slot group (at the QKV shape 16 K chunks x 3 slices of shrink and 12
    // column chunks x 4 token blocks of expand), however few tokens the group
    // holds; the other single-launch kernel recomputes the shrink of each
    // 8-token group per 1024-column chunk.  So for narrow outputs auto takes
    // the K-split launch when the expected groups are few or full: at most
    // kRelayFewGroups of them, or at least kRelayMinPerSlot tokens per slot
    // that draws any (slots drawn uniformly).  Measured (QKV shape, rank 16):
    // 8 slots, 1 to 1024 tokens, it is the faster one (T 512: 12.9 against
    // 16.7 us; T 1024: 24.2 against 26.1); 64 slots at T 64 and 256, and 32
    // slots at T 512, the other (10.5, 18.3, 17.1 against 20.2, 31.0, 19.9 us).
    const double used = L * (1.0 - exp(-(double)T / L));
    const bool relay_batch = used + T / (double)kRelayGroup <= kRelayFewGroups ||
                             T >= kRelayMinPerSlot * used;
    const bool relay_ws = ws && ws_bytes >= ws_layout(T, K, S, R, L).end;
    // Wide outputs (an lm_head's vocabulary) take it wherever it runs: measured
    // against the tile kernels on vocabularies of 32000 to 256000 columns, 64
    // to 1024 tokens over 8 to 64 slots, ranks 16 and 32, it is the faster
    // (128256 columns: 256 tokens 36.0 against 50.3 us, 1024 tokens 104.8
    // against 117.6, 256 tokens over 64 slots 118.4 against 153.0; 1024
    // tokens of 32000 columns over 64 slots 52.8 against 64.4).
    const bool relay_wide = !narrow;
    const bool relay_auto = relay_ok && relay_ws && ((narrow && relay_batch) || relay_wide);
    // Decode-sized batches of long slot runs take it too, before the tile
    // kernels (8 slots, T 512: 12.9 against 27.1 us; T 1024: 24.2 against 30.3).
    if (path == LORA_PATH_AUTO && use_prefill && relay_auto) use_prefill = 0;
    const bool relay = path == LORA_PATH_RELAY || (path == LORA_PATH_AUTO && !use_prefill && relay_auto);
    // The other single launch up to 64 slots: past that each of many small
    // groups streams its slot's lora_a once per column chunk (1024 tokens over
    // 128 slots at rank 32: 95.6 us against 64.1 for the tile kernels).
    const bool fuse = !use_prefill && !relay && can_fuse(T, K, R, N, S, ldy, y_col_offset, dtype) &&
                      (path == LORA_PATH_FUSED || (path == LORA_PATH_AUTO && narrow && L <= 64));
    if (path == LORA_PATH_FUSED && !fuse) return LORA_E_PATH;
    // Auto takes the grouped kernels while their in-kernel discovery is the
    // one-wave kind (L <= 64) and the expand sums the K-chunk partials itself;
    // and at rank 16 for narrow outputs up to 4096 tokens and 128 slots, also
    // before the tile kernels (QKV shape: 2048 tokens over 16 slots 36.8
    // against 40.1 us, 1536 over 128 slots 44.2 against 51.9; at ranks 32 and
    // 64 the tile kernels are faster).
    const bool group_r16 = R == 16 && narrow && T <= kGrpR16MaxTokens && L <= 128;
    const bool group_auto = (L <= 64 && R <= kGrpMaxPartialRank && narrow) || group_r16;
    const bool group_ok = can_group(T, K, R, N, S, ldy, y_col_offset, dtype);
    if (path == LORA_PATH_AUTO && use_prefill && !relay && group_r16 && group_ok) use_prefill = 0;
    const bool group = !use_prefill && !fuse && !relay && group_ok &&
                       (path == LORA_PATH_GROUPED || (path == LORA_PATH_AUTO && group_auto));
    if (path == LORA_PATH_GROUPED && !group) return LORA_E_PATH;
    // Auto, past the single-launch and discovering grouped kernels (more than
    // 64 slots, ranks past 64, or wide outputs): the MFMA prefill kernels, the
    // shrink split over K when its tiles are few, while the persistent expand
    // takes the rank.
    if (path == LORA_PATH_AUTO && !use_prefill && !fuse && !group && !relay && dtype == LORA_DT_BF16 &&
        (R == 16 || R == 32 || R == 64 || R == 128) && rows_of_8(N, S, ldy, y_col_offset))
        use_prefill = 1;
    out->path = relay ? LORA_PATH_RELAY : fuse ? LORA_PATH_FUSED : group ? LORA_PATH_GROUPED
              : use_prefill ? LORA_PATH_PREFILL : LORA_PATH_DECODE;
    // One lora_a for every slice (the same pointer in each, as a merged layer
    // holds when its checkpoint has a single lora_a: [vLLM]
    // MergedQKVParallelLinearWithLoRA duplicates it per slice).
    bool shared_a = S > 1 && A;
    for (int s = 1; s < S && shared_a; ++s) shared_a = A[s] == A[0];
    out->shared_a = shared_a ? 1 : 0;
    out->noop = T == 0 ? 1 : 0;
    if (T == 0) return LORA_OK;
    if (!y || !x || !idx || !scale) return LORA_E_NULL;
    CHECK(check_ptrs(A, S));
    CHECK(check_ptrs(B, S));
    if (!al(y, 16) || !al(x, 16)) return LORA_E_ALIGN;
    if (!fuse) CHECK(check_ws(ws, ws_bytes, ws_layout(T, K, S, R, L).end));
    return LORA_OK;
}

// Enqueues the kernels of a checked plan.
int32_t packed_run(const PackedPlan &p, void *y, int64_t ldy, int64_t y_col_offset, const void *x,
                   int64_t ldx, int32_t T, int32_t K, const void *const *A, const void *const *B,
                   const int64_t *N, int32_t S, int32_t L, int32_t R, const int32_t *idx,
                   const int32_t *slot_rank, const float *scale, int32_t dtype, uint32_t flags,
                   void *ws, size_t ws_bytes, hipStream_t st) {
    if (p.noop) return LORA_OK;
    if (p.path == LORA_PATH_FUSED) {
        // one launch; no workspace and no segments needed
        const Slices sl = make_slices(A, B, N, S, y_col_offset);
        return launched(launch_dec_fused(y, ldy, x, ldx, T, K, sl, S, L, R, idx, slot_rank, scale, st));
    }
    if (p.path == LORA_PATH_TOKEN) {
        // one launch; no workspace and no segments needed
        const Slices sl = make_slices(A, B, N, S, y_col_offset);
        return launched(launch_dec_token(dtype, y, ldy, x, ldx, T, K, sl, S, L, R, idx, slot_rank,
                                         scale, st));
    }
    const WsLayout wl = ws_layout(T, K, S, R, L);
    SegPtrs seg = seg_ptrs(ws, wl.seg);
    // the single-launch segment build's region in the end area, above this
    // call's own regions
    attach_seg_x(seg, ws, ws_bytes, T, L, 0, wl.buf + align256(sizeof(float) * (size_t)S * T * R));
    const Slices sl = make_slices(A, B, N, S, y_col_offset);
    float *buf = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.buf);
    if (p.path == LORA_PATH_RELAY) {
        // one launch; partials and counters in the region at the end of ws
        const RelayRegion rr = relay_region(ws_bytes, T, K, S, R, L);
        char *w = static_cast<char *>(ws);
        return launched(launch_dec_relay(y, ldy, x, ldx, T, K, sl, S, L, R, idx, slot_rank, scale,
                                         reinterpret_cast<float *>(w + rr.part),
                                         reinterpret_cast<int32_t *>(w + rr.sync),
                                         reinterpret_cast<int32_t *>(w + rr.err),
                                         (flags & LORA_FLAG_RELAY_GIVE_UP) != 0, st));
    }
    if (p.path == LORA_PATH_GROUPED) {
        // two launches that derive their token groups from idx, or the
        // segment build and launches that read the groups from its table;
        // a shared lora_a is shrunk once (slice 0) and every slice's expand
        // adds that shrink
        const SegPtrs *gseg = grp_discovers(T, L) ? nullptr : &seg;
        if (gseg && !(flags & LORA_FLAG_SEGMENTS_READY))
            CHECK(launched(launch_segments(idx, slot_rank, T, L, R, seg, st)));
        float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.partial);
        const int32_t Ssh = p.shared_a ? 1 : S;
        const Slices slsh = p.shared_a ? make_slices(A, B, N, 1, y_col_offset) : sl;
        const bool sh = p.shared_a != 0;
        if (R > kGrpMaxPartialRank) {
            // large ranks: the K chunks are summed into the token-ordered buffer first
            int32_t n_kc = 0;
            CHECK(grp_shrink_part(x, ldx, T, K, slsh, Ssh, L, R, idx, slot_rank, part, wl, gseg, st, &n_kc));
            CHECK(launched(launch_grp_reduce(T, Ssh, L, R, idx, slot_rank, part, n_kc, buf, gseg, st)));
            return launched(launch_grp_expand(y, ldy, T, 1, sl, S, L, R, idx, slot_rank, scale,
                                              nullptr, buf, nullptr, gseg, st, sh));
        }
        CHECK(launched(launch_grp_shrink(x, ldx, T, K, slsh, Ssh, L, R, idx, slot_rank, part, nullptr,
                                         gseg, st)));
        return launched(launch_grp_expand(y, ldy, T, grp_kchunks(K), sl, S, L, R, idx, slot_rank,
                                          scale, part, nullptr, nullptr, gseg, st, sh));
    }
    if (!(flags & LORA_FLAG_SEGMENTS_READY))
        CHECK(launched(launch_segments(idx, slot_rank, T, L, R, seg, st)));
    if (p.path == LORA_PATH_PREFILL) {
        // a shared lora_a: the shrink runs once and every slice's expand reads its buffer
        if (p.shared_a) {
            const Slices sl1 = make_slices(A, B, N, 1, y_col_offset);
            CHECK(pre_shrink_buf(x, ldx, T, K, sl1, 1, L, R, idx, slot_rank, seg, wl, ws, buf, st));
            GroupMap gm;
            gm.buf_sstride = 0;
            return launched(launch_pre_expand(y, ldy, buf, T, sl, S, L, R, slot_rank, scale, seg, st, gm));
        }
        CHECK(pre_shrink_buf(x, ldx, T, K, sl, S, L, R, idx, slot_rank, seg, wl, ws, buf, st));
        return launched(launch_pre_expand(y, ldy, buf, T, sl, S, L, R, slot_rank, scale, seg, st));
    }
    float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.partial);
    CHECK(launched(launch_dec_shrink(dtype, x, ldx, T, K, sl, S, L, R, slot_rank, seg, partial,
                                     wl.n_kchunks, st)));
    if (wl.n_kchunks * R <= kFoldMaxChunkRank)
        return launched(launch_dec_expand(dtype, y, ldy, nullptr, partial, wl.n_kchunks, T, sl, S,
                                          L, R, slot_rank, scale, seg, st));
    CHECK(launched(launch_dec_reduce(T, S, L, R, slot_rank, seg, partial, wl.n_kchunks, buf, st)));
    return launched(launch_dec_expand(dtype, y, ldy, buf, nullptr, 0, T, sl, S, L, R, slot_rank,
                                      scale, seg, st));
}

}  // namespace aa

extern "C" {

const char *lora_status_string(lora_status_t s) {
    switch (s) {
        case LORA_OK: return "ok";
        case LORA_E_NULL: return "a required pointer is NULL";
        case LORA_E_SHAPE: return "a size is out of range or a leading dimension is too small";
        case LORA_E_DTYPE: return "unknown dtype";
        case LORA_E_RANK: return "rank outside [1, 512]";
        case LORA_E_SLICES: return "slice count outside [1, 8]";
        case LORA_E_WORKSPACE: return "workspace smaller than lora_workspace_size()";
        case LORA_E_ALIGN: return "pointer or stride alignment not met";
        case LORA_E_PATH: return "the requested path cannot run these arguments";
        case LORA_E_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case LORA_E_TIMEOUT:
            return "a hand-over wait of the single-launch K-split decode gave up; the results "
                   "of the calls since the last check are not valid (the workspace was zero-filled)";
        case LORA_E_RUNTIME: return "a HIP runtime call failed";
        case LORA_E_SCRATCH:
            return "the call needs more scratch than lora_apply_packed_noalloc's static array holds";
        default: return "unknown status";
    }
}

lora_status_t lora_workspace_size(int32_t T, int32_t K, int32_t S, int32_t R, int32_t L,
                                  size_t *bytes) {
    if (!bytes) return LORA_E_NULL;
    CHECK(check_sizes(T, S, L, R, LORA_DT_F32));
    if (K < 1) return LORA_E_SHAPE;
    *bytes = ws_layout(T, K, S, R, L).end;
    return LORA_OK;
}

lora_status_t lora_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return LORA_E_NULL;
    if (!al(ws, 256)) return LORA_E_ALIGN;
    return launched(launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

lora_status_t lora_workspace_check(void *ws, size_t ws_bytes, void *stream) {
    if (!ws && ws_bytes == 0) return static_scratch_check(static_cast<hipStream_t>(stream));
    if (!ws) return LORA_E_NULL;
    if (!al(ws, 256)) return LORA_E_ALIGN;
    if (ws_bytes < 256) return LORA_E_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t word = 0;
    const char *e = static_cast<const char *>(ws) + err_word_offset(ws_bytes);
    if (hipMemcpyAsync(&word, e, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess)
        return LORA_E_RUNTIME;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_E_RUNTIME;
    if (word == 0) return LORA_OK;
    // a wait gave up: late partials may sit in the region, so start over
    if (launch_fill_zero(ws, ws_bytes, st) != hipSuccess) return LORA_E_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_E_RUNTIME;
    return LORA_E_TIMEOUT;
}

lora_status_t lora_segment_layout(int32_t T, int32_t L, lora_segment_layout_t *out) {
    if (!out) return LORA_E_NULL;
    if (T < 0 || L < 1 || L > LORA_MAX_SLOTS) return LORA_E_SHAPE;
    const SegLayout l = seg_layout(T, L);
    out->header = (int64_t)l.header;
    out->slot_start = (int64_t)l.slot_start;
    out->perm = (int64_t)l.perm;
    out->tiles_decode = (int64_t)l.tiles_dec;
    out->tiles_prefill = (int64_t)l.tiles_pre;
    out->tile_decode_tokens = kDecTile;
    out->tile_prefill_tokens = kPreTile;
    return LORA_OK;
}

lora_status_t lora_build_segments(const int32_t *idx, const int32_t *slot_rank, int32_t T,
                                  int32_t L, int32_t R, void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || L < 1 || L > LORA_MAX_SLOTS) return LORA_E_SHAPE;
    if (R < 1 || R > LORA_MAX_RANK) return LORA_E_RANK;
    if (max_tiles(T, L, kDecTile) > 65535) return LORA_E_SHAPE;
    if (T > 0 && !idx) return LORA_E_NULL;
    const SegLayout l = seg_layout(T, L);
    CHECK(check_ws(ws, ws_bytes, l.end));
    SegPtrs seg = seg_ptrs(ws, l);
    attach_seg_x(seg, ws, ws_bytes, T, L, 0, l.end);
    return launched(launch_segments(idx, slot_rank, T, L, R, seg, static_cast<hipStream_t>(stream)));
}

lora_status_t lora_shrink(float *buf, const void *x, int64_t ldx, int32_t T, int32_t K,
                          const void *const *A, int32_t S, int32_t L, int32_t R,
                          const int32_t *idx, const int32_t *slot_rank, int32_t dtype,
                          int32_t path, uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
    if (path == LORA_PATH_FUSED || path == LORA_PATH_RELAY || path == LORA_PATH_TOKEN)
        return LORA_E_PATH;
    CHECK(check_sizes(T, S, L, R, dtype));
    CHECK(check_k(K, ldx));
    int use_prefill = 0;
    CHECK(choose_path(path, T, L, R, dtype, &use_prefill));
    if (auto_tiles_apart(path, flags, L, R, dtype)) use_prefill = 1;
    const bool group = path == LORA_PATH_GROUPED;
    if (group && !(can_group_sizes(T, R, dtype) && can_group_k(K))) return LORA_E_PATH;
    if (group && (flags & LORA_FLAG_PARTIAL) && R > kGrpMaxPartialRank) return LORA_E_PATH;
    if (T == 0) return LORA_OK;
    if (!buf || !x || !idx) return LORA_E_NULL;
    CHECK(check_ptrs(A, S));
    if (!al(buf, 16) || !al(x, 16)) return LORA_E_ALIGN;
    const WsLayout wl = ws_layout(T, K, S, R, L);
    CHECK(check_ws(ws, ws_bytes, wl.end));

    hipStream_t st = static_cast<hipStream_t>(stream);
    const SegPtrs seg = seg_ptrs(ws, wl.seg);
    const Slices sl = make_slices(A, nullptr, nullptr, S, 0);
    // buf is written unless the decode path keeps partials in the workspace
    const bool writes_buf = use_prefill || !(flags & LORA_FLAG_PARTIAL);
    if (group) {
        // groups come from idx inside the kernels, or from the segment table
        const SegPtrs *gseg = grp_discovers(T, L) ? nullptr : &seg;
        if (gseg && !(flags & LORA_FLAG_SEGMENTS_READY))
            CHECK(launched(launch_segments(idx, slot_rank, T, L, R, seg, st)));
        if (writes_buf && !(flags & LORA_FLAG_ACTIVE_ONLY))
            CHECK(launched(launch_fill_zero(buf, sizeof(float) * (size_t)S * T * R, st)));
        float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.partial);
        if (!writes_buf)
            return launched(launch_grp_shrink(x, ldx, T, K, sl, S, L, R, idx, slot_rank, part,
                                              grp_kc_slot(ws, wl.seg), gseg, st));
        int32_t n_kc = 0;
        CHECK(grp_shrink_part(x, ldx, T, K, sl, S, L, R, idx, slot_rank, part, wl, gseg, st, &n_kc));
        return launched(launch_grp_reduce(T, S, L, R, idx, slot_rank, part, n_kc, buf, gseg, st));
    }
    if (!(flags & LORA_FLAG_SEGMENTS_READY))
        CHECK(launched(launch_segments(idx, slot_rank, T, L, R, seg, st)));
    if (writes_buf && !(flags & LORA_FLAG_ACTIVE_ONLY))
        CHECK(launched(launch_fill_zero(buf, sizeof(float) * (size_t)S * T * R, st)));
    if (use_prefill)
        return pre_shrink_buf(x, ldx, T, K, sl, S, L, R, idx, slot_rank, seg, wl, ws, buf, st);
    float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.partial);
    CHECK(launched(launch_dec_shrink(dtype, x, ldx, T, K, sl, S, L, R, slot_rank, seg, partial,
                                     wl.n_kchunks, st)));
    if (flags & LORA_FLAG_PARTIAL) return LORA_OK;
    return launched(launch_dec_reduce(T, S, L, R, slot_rank, seg, partial, wl.n_kchunks, buf, st));
}

lora_status_t lora_expand(void *y, int64_t ldy, int64_t y_col_offset, const float *buf,
                          int32_t T, const void *const *B, const int64_t *N, int32_t S,
                          int32_t L, int32_t R, const int32_t *idx, const int32_t *slot_rank,
                          const float *scale, int32_t dtype, int32_t path, uint32_t flags,
                          void *ws, size_t ws_bytes, void *stream) {
    if (path == LORA_PATH_FUSED || path == LORA_PATH_RELAY || path == LORA_PATH_TOKEN)
        return LORA_E_PATH;
    CHECK(check_sizes(T, S, L, R, dtype));
    int64_t ntot = 0;
    CHECK(check_n(N, S, ldy, y_col_offset, &ntot));
    int use_prefill = 0;
    CHECK(choose_path(path, T, L, R, dtype, &use_prefill));
    if (auto_tiles_apart(path, flags, L, R, dtype) && rows_of_8(N, S, ldy, y_col_offset))
        use_prefill = 1;
    const bool group = path == LORA_PATH_GROUPED;
    if (group && !(can_group_sizes(T, R, dtype) && rows_of_8(N, S, ldy, y_col_offset)))
        return LORA_E_PATH;
    if (group && (flags & LORA_FLAG_PARTIAL) && R > kGrpMaxPartialRank) return LORA_E_PATH;
    if (T == 0) return LORA_OK;
    if (!y || !buf || !idx || !scale) return LORA_E_NULL;
    CHECK(check_ptrs(B, S));
    if (!al(y, 16) || !al(buf, 16)) return LORA_E_ALIGN;
    const SegLayout sgl = seg_layout(T, L);
    CHECK(check_ws(ws, ws_bytes, sgl.end));

    hipStream_t st = static_cast<hipStream_t>(stream);
    const SegPtrs seg = seg_ptrs(ws, sgl);
    const Slices sl = make_slices(nullptr, B, N, S, y_col_offset);
    if (group) {
        const SegPtrs *gseg = grp_discovers(T, L) ? nullptr : &seg;
        if (gseg && !(flags & LORA_FLAG_SEGMENTS_READY))
            CHECK(launched(launch_segments(idx, slot_rank, T, L, R, seg, st)));
        if (!(flags & LORA_FLAG_PARTIAL))
            return launched(launch_grp_expand(y, ldy, T, 1, sl, S, L, R, idx, slot_rank, scale,
                                              nullptr, buf, nullptr, gseg, st));
        // partials right after the segments; the chunk count comes from the
        // shrink, capped by what this workspace holds
        const float *part = reinterpret_cast<const float *>(static_cast<char *>(ws) + sgl.end);
        const size_t chunk_bytes = sizeof(float) * (size_t)T * S * R;
        const int64_t fit = (int64_t)((ws_bytes - sgl.end) / chunk_bytes);
        if (fit < 1) return LORA_E_WORKSPACE;
        const int32_t cap = (int32_t)(fit < kMaxKcGrp ? fit : kMaxKcGrp);
        return launched(launch_grp_expand(y, ldy, T, cap, sl, S, L, R, idx, slot_rank, scale, part,
                                          nullptr, grp_kc_slot(ws, sgl), gseg, st));
    }
    if (!(flags & LORA_FLAG_SEGMENTS_READY))
        CHECK(launched(launch_segments(idx, slot_rank, T, L, R, seg, st)));
    if (use_prefill)
        return launched(launch_pre_expand(y, ldy, buf, T, sl, S, L, R, slot_rank, scale, seg, st));
    if (flags & LORA_FLAG_PARTIAL) {
        // partial sums sit right after the segments (ws_layout), K-chunk count in the header
        const float *partial = reinterpret_cast<const float *>(static_cast<char *>(ws) + sgl.end);
        // the kernel never reads more chunks than this workspace holds
        const size_t chunk_bytes = sizeof(float) * (size_t)T * S * R;
        const int32_t fit = (int32_t)((ws_bytes - sgl.end) / chunk_bytes);
        if (fit < 1) return LORA_E_WORKSPACE;
        return launched(launch_dec_expand(dtype, y, ldy, nullptr, partial, fit, T, sl, S, L, R,
                                          slot_rank, scale, seg, st));
    }
    return launched(launch_dec_expand(dtype, y, ldy, buf, nullptr, 0, T, sl, S, L, R, slot_rank,
                                      scale, seg, st));
}

lora_status_t lora_plan_packed(const void *y, int64_t ldy, int64_t y_col_offset, const void *x,
                               int64_t ldx, int32_t T, int32_t K, const void *const *A,
                               const void *const *B, const int64_t *N, int32_t S, int32_t L,
                               int32_t R, const int32_t *idx, const int32_t *slot_rank,
                               const float *scale, int32_t dtype, int32_t path, uint32_t flags,
                               const void *ws, size_t ws_bytes, int32_t *chosen_path) {
    if (!chosen_path) return LORA_E_NULL;
    PackedPlan p;
    CHECK(packed_plan(y, ldy, y_col_offset, x, ldx, T, K, A, B, N, S, L, R, idx, slot_rank, scale,
                      dtype, path, flags, ws, ws_bytes, &p));
    *chosen_path = p.path;
    return LORA_OK;
}

lora_status_t lora_apply_packed(void *y, int64_t ldy, int64_t y_col_offset, const void *x,
                                int64_t ldx, int32_t T, int32_t K, const void *const *A,
                                const void *const *B, const int64_t *N, int32_t S, int32_t L,
                                int32_t R, const int32_t *idx, const int32_t *slot_rank,
                                const float *scale, int32_t dtype, int32_t path, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream) {
    PackedPlan p;
    CHECK(packed_plan(y, ldy, y_col_offset, x, ldx, T, K, A, B, N, S, L, R, idx, slot_rank, scale,
                      dtype, path, flags, ws, ws_bytes, &p));
    return packed_run(p, y, ldy, y_col_offset, x, ldx, T, K, A, B, N, S, L, R, idx, slot_rank,
                      scale, dtype, flags, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
