// Shared definitions of the HIP library: storage-type helpers, the
// workspace layout and the kernel argument blocks.  gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aa {

constexpr int kWave = 64;
constexpr int kMaxSlices = 8;
constexpr int kMaxRank = 512;
constexpr int kMaxSlots = 1024;

// Tile sizes (tokens of one slot handled together).
// Segment build: threads of its work-groups; item counts past kSegSplitItems
// use the two-pass build over ceil(items / kSegThreads) work-groups.
constexpr int kSegThreads = 1024;
constexpr int kSegSplitItems = 4096;
constexpr int kDecTile = 32;   // decode (VALU) path: one token per lane half
constexpr int kPreTile = 64;   // prefill (MFMA) path: two 32-row MFMA blocks

// Decode shrink: K columns per work-group chunk and rank rows per work-group.
constexpr int kDecKc = 256;    // 4 waves x 64 columns
constexpr int kDecRows = 16;   // rows of the (slice, rank) space per work-group

// Single-launch decode (fused shrink + expand).
constexpr int kFusedGroup = 8;         // tokens of one slot per work-group
constexpr int kFusedCols = 1024;       // output columns per work-group
constexpr int kFusedMaxRank = 32;
constexpr int kFusedMaxTokens = 1024;  // idx staged in LDS
// lora_apply_packed's auto path keeps the fused and grouped decode kernels to
// outputs of at most this many columns per token (sum over slices)
constexpr int64_t kAutoMaxDecodeCols = 16384;
constexpr int kFusedXcds = 8;

// Single-launch decode with the shrink split over K (relay.hip).
constexpr int kRelayGroup = 32;        // tokens of one slot per shrink item
constexpr int kRelayKc = 256;          // K columns per shrink item
constexpr int kRelayCols = 512;        // output columns per expand item
constexpr int kRelayMaxKc = 32;        // K <= 8192

// Slot-grouped split decode (split-K MFMA shrink, then expand).
constexpr int kGrpTokens = 32;         // tokens of one slot per group
constexpr int kGrpCols = 512;          // output columns per expand work-group
constexpr int kGrpMaxTokens = 4096;    // idx staged in LDS
constexpr int kGrpMaxRank = 128;
constexpr int kGrpMaxPartialRank = 64;   // the expand adds K-chunk partials itself up to this rank
constexpr int kMaxKcGrp = 16;          // K chunks of 512: K <= 8192

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest, ties to even (gfx950 converts a pair in one
// instruction, v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t b = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Loads in the pipelined loops are unconditional, from addresses clamped to a
// valid row; results that belong to padding rows/columns are discarded or
// zeroed where they are written.  A load under a branch would make the
// compiler wait for every outstanding load (vmcnt(0)) at the next use and
// serialise the prefetch.
template <typename V, typename E>
__device__ __forceinline__ V ldg(const E *p) { return *reinterpret_cast<const V *>(p); }

// Streamed-once data (y rows): 16-byte loads and stores with the
// non-temporal hint, so that they do not push reused lora_a / lora_b rows and
// x rows out of the L2.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <typename E>
__device__ __forceinline__ uint4 ldg_nt(const E *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename E>
__device__ __forceinline__ void stg_nt(E *p, const uint4 &v) {
    const u32x4_t u = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t *>(p));
}

// Sum over the 64 lanes of a wave, the same value on every lane: DPP sums
// within each 16-lane row (quad swaps, then half-row and row mirrors), then
// the four row sums in row order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_f32<0xb1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4e>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x141>(v);   // row_half_mirror
    v += dpp_f32<0x140>(v);   // row_mirror
    const int b = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
}

// Work-group barrier for LDS traffic only: global loads, stores and atomics
// stay in flight across it (__syncthreads() may also wait for every
// outstanding global access, which puts a memory round trip on the path).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned).
// ---------------------------------------------------------------------------
struct SegLayout {
    size_t header;        // int32[8]: active, invalid, decode tiles, prefill tiles,
                          //           K chunks of the last decode shrink
    size_t slot_start;    // int32[L+1]
    size_t perm;          // int32[T]
    size_t tiles_dec;     // int4[max_tiles_dec]: slot, begin, end, 0
    size_t tiles_pre;     // int4[max_tiles_pre]
    size_t counts;        // int32[ceil(T / kSegThreads)][L + 1]: two-launch build, per work-group
    size_t end;
    int32_t max_tiles_dec;
    int32_t max_tiles_pre;
};

struct WsLayout {
    SegLayout seg;
    size_t partial;       // fp32 [n_kchunks][T][S*R]
    size_t buf;           // fp32 [S][T][R]
    size_t relay;         // bytes of the single-launch split decode's region (see relay_region)
    size_t end;           // the regions above, the relay region, the error word's line
    int32_t n_kchunks;
};

int32_t relay_sync_ints(int32_t T, int32_t L, int32_t S);


inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The error word of the single-launch split decode's bounded waits: the first
// int32 of the workspace's last 256-byte line (inside the buffer whatever
// ws_bytes is).  Set when a wait gives up; read and cleared by
// lora_workspace_check.  No kernel writes anything else to that line.
inline size_t err_word_offset(size_t ws_bytes) { return (ws_bytes - sizeof(int32_t)) & ~size_t(255); }

// The single-launch split decode's region: its fp32 partials [S][K/256][T][R]
// and then its counters.  The kernel needs it all zero on entry and leaves it
// all zero, so nothing else may write there: it sits at the END of the
// caller's buffer, just before the error word's line, while every other
// region starts at offset 0.  Every region grows with each size argument, so
// a workspace of lora_workspace_size() at the largest sizes a caller uses
// keeps this region clear of every other call's regions, whatever their
// shapes.
struct RelayRegion {
    size_t part;          // offset of the partials
    size_t sync;          // offset of the counters
    size_t err;           // offset of the error word
};
inline size_t relay_part_bytes(int32_t T, int32_t K, int32_t S, int32_t R) {
    return align256(sizeof(float) * (size_t)((K + kRelayKc - 1) / kRelayKc) * T * S * R);
}
inline size_t relay_bytes(int32_t T, int32_t K, int32_t S, int32_t R, int32_t L) {
    return relay_part_bytes(T, K, S, R) + align256(sizeof(int32_t) * (size_t)relay_sync_ints(T, L, S));
}
inline RelayRegion relay_region(size_t ws_bytes, int32_t T, int32_t K, int32_t S, int32_t R, int32_t L) {
    RelayRegion r;
    r.err = err_word_offset(ws_bytes);
    r.part = (r.err - relay_bytes(T, K, S, R, L)) & ~size_t(255);
    r.sync = r.part + relay_part_bytes(T, K, S, R);
    return r;
}

// The single-launch segment build (more than kSegSplitItems items, at most
// kSegOneMaxWg work-groups) exchanges its work-groups' per-key counts through
// a region that, like the relay region, must be zero on entry and is left
// zero: [counts int32 [n_wg][keys + 1]][one 256-byte line: done counter].  It
// sits at the end of the workspace, just below the error word's line (it may
// overlap the relay region: both are zero between calls).  Past
// kSegOneMaxWg work-groups the build takes two launches, but the region stays
// reserved, so that the size grows with every argument.  (A lone build of at
// most kSegSplitItems items runs in one work-group and does not use it; the
// token job of the fused-MoE alignment, built beside the pair job, does.)
constexpr int kSegOneMaxWg = 16;
inline size_t seg_x_bytes(int32_t n_items, int32_t nkeys) {
    int64_t n_wg = ((int64_t)n_items + kSegThreads - 1) / kSegThreads;
    if (n_wg < 1) n_wg = 1;
    if (n_wg > kSegOneMaxWg) n_wg = kSegOneMaxWg;
    return align256(sizeof(int32_t) * (size_t)n_wg * (nkeys + 1)) + 256;
}

inline int32_t max_tiles(int32_t T, int32_t L, int32_t tile) {
    // sum over slots of ceil(c_s / tile) <= T / tile + (number of non-empty slots)
    int64_t m = (int64_t)T / tile + (T < L ? T : L) + 1;
    return (int32_t)m;
}

inline int32_t row_groups(int32_t S, int32_t R) {
    return (S * R + kDecRows - 1) / kDecRows;
}

// T items (tokens, or token-expert pairs), L keys (slots, or slot-expert pairs),
// placed at byte offset `base` of the workspace.
inline SegLayout seg_layout(int32_t T, int32_t L, size_t base = 0) {
    SegLayout l{};
    size_t o = base;
    l.header = o;     o = align256(o + 16 * sizeof(int32_t));
    l.slot_start = o; o = align256(o + sizeof(int32_t) * (size_t)(L + 1));
    l.perm = o;       o = align256(o + sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    l.max_tiles_dec = max_tiles(T, L, kDecTile);
    l.max_tiles_pre = max_tiles(T, L, kPreTile);
    l.tiles_dec = o;  o = align256(o + 16 * (size_t)l.max_tiles_dec);
    l.tiles_pre = o;  o = align256(o + 16 * (size_t)l.max_tiles_pre);
    l.counts = o;     o = align256(o + sizeof(int32_t) * (size_t)((T + kSegThreads - 1) / kSegThreads) * (L + 1));
    l.end = o;
    return l;
}

inline WsLayout ws_layout(int32_t T, int32_t K, int32_t S, int32_t R, int32_t L) {
    WsLayout w{};
    w.seg = seg_layout(T, L);
    size_t o = w.seg.end;
    w.n_kchunks = (K + kDecKc - 1) / kDecKc;
    w.partial = o; o = align256(o + sizeof(float) * (size_t)w.n_kchunks * (size_t)T * S * R);
    w.buf = o;     o = align256(o + sizeof(float) * (size_t)S * T * R);
    w.relay = relay_bytes(T, K, S, R, L);
    // the end area (relay region and the single-launch segment build's
    // region, which may overlap), then the error word's line
    const size_t x = seg_x_bytes(T, L);
    w.end = o + (w.relay > x ? w.relay : x) + 256;
    return w;
}

// Fused-MoE workspace: token segments (by slot), pair segments (by slot and
// expert) and the fp32 buffer [S][T*k][R].
// K-split partials of the MoE shrink: kMoeSplitChunks chunks of up to
// kMoeSplitItems items (the split serves small batches, whose few tiles would
// otherwise stream K through a few CUs).
constexpr int kMoeSplitChunks = 16;
constexpr int kMoeSplitItems = 4096;

struct MoeWsLayout {
    SegLayout tok;
    SegLayout pair;
    size_t buf;
    size_t part;          // fp32 [S][chunks][items][R], items <= kMoeSplitItems
    size_t part_bytes;
    size_t end;
};

inline MoeWsLayout moe_ws_layout(int32_t T, int32_t k, int32_t S, int32_t R, int32_t L, int32_t E) {
    MoeWsLayout m{};
    m.tok = seg_layout(T, L, 0);
    m.pair = seg_layout(T * k, L * E, m.tok.end);
    m.buf = m.pair.end;
    m.part = align256(m.buf + sizeof(float) * (size_t)S * T * k * R);
    const int64_t items = (int64_t)T * k < kMoeSplitItems ? (int64_t)T * k : kMoeSplitItems;
    m.part_bytes = sizeof(float) * (size_t)kMoeSplitChunks * items * S * R;
    // the single-launch segment build's regions of the pair and token jobs,
    // then the error word's line
    m.end = align256(m.part + m.part_bytes) + seg_x_bytes(T * k, L * E) + seg_x_bytes(T, L) + 256;
    return m;
}

inline int32_t moe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t bm) {
    const int64_t c = (int64_t)T * k + (int64_t)E * (bm - 1);
    return (int32_t)((c + bm - 1) / bm * bm);
}

// Device view of the segments.
struct SegPtrs {
    int32_t *header;
    int32_t *slot_start;
    int32_t *perm;
    int4 *tiles_dec;
    int4 *tiles_pre;
    int32_t *counts;
    int32_t *xcounts;     // single-launch build's region (see seg_x_bytes), or null:
    int32_t *xdone;       //   the build takes two launches
    int32_t *err;         // the workspace's error word (a wait of the build gave up)
    int32_t max_tiles_dec;
    int32_t max_tiles_pre;
};

inline SegPtrs seg_ptrs(void *ws, const SegLayout &l) {
    char *b = static_cast<char *>(ws);
    SegPtrs p;
    p.header = reinterpret_cast<int32_t *>(b + l.header);
    p.slot_start = reinterpret_cast<int32_t *>(b + l.slot_start);
    p.perm = reinterpret_cast<int32_t *>(b + l.perm);
    p.tiles_dec = reinterpret_cast<int4 *>(b + l.tiles_dec);
    p.tiles_pre = reinterpret_cast<int4 *>(b + l.tiles_pre);
    p.counts = reinterpret_cast<int32_t *>(b + l.counts);
    p.xcounts = p.xdone = p.err = nullptr;
    p.max_tiles_dec = l.max_tiles_dec;
    p.max_tiles_pre = l.max_tiles_pre;
    return p;
}

// Gives `seg` the single-launch build's region of (n_items, nkeys) at the end
// of a workspace of ws_bytes, `below` bytes under the error word's line, when
// the build takes one launch and the region stays above byte `floor` (the
// caller's own regions).  Otherwise the build keeps two launches.
inline void attach_seg_x(SegPtrs &seg, void *ws, size_t ws_bytes, int32_t n_items, int32_t nkeys,
                         size_t below, size_t floor) {
    const size_t xb = seg_x_bytes(n_items, nkeys);
    const size_t err = err_word_offset(ws_bytes);
    const int64_t n_wg = ((int64_t)n_items + kSegThreads - 1) / kSegThreads;
    if (n_wg > kSegOneMaxWg || err < below + xb || err - below - xb < floor) return;
    char *b = static_cast<char *>(ws);
    seg.xcounts = reinterpret_cast<int32_t *>(b + err - below - xb);
    seg.xdone = reinterpret_cast<int32_t *>(b + err - below - 256);
    seg.err = reinterpret_cast<int32_t *>(b + err);
}

// Per-slice pointers and widths passed by value to kernels.
struct Slices {
    const void *a[kMaxSlices];   // lora_a [L][R][K]
    const void *b[kMaxSlices];   // lora_b [L][N_s][R]
    int64_t n[kMaxSlices];       // N_s
    int64_t off[kMaxSlices + 1]; // column offset of each slice in y (incl. y_col_offset)
};

// A fused-MoE call of at most this many (token, k) pairs, rank 16, without
// the k-reduction and without a prebuilt alignment skips the alignment
// (moe_small.hip).
constexpr int kMoeSmallPairs = 1024;
bool moe_small_takes(int32_t pairs, int32_t R, int32_t reduce_k);
hipError_t launch_moe_small(void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T, int32_t top_k,
                            int32_t K, const Slices &sl, int32_t S, int32_t E, int32_t L, int32_t R,
                            int32_t Ea, int32_t Eb, int32_t x_div, const int32_t *topk_ids,
                            const float *coef, const int32_t *idx, const int32_t *slot_rank,
                            const float *scale, hipStream_t st);


// lora_apply_packed in two steps (abi.hip): packed_plan runs every argument
// check and chooses the path without enqueueing anything; packed_run enqueues
// the plan's kernels.  Both return a LORA_* status.
struct PackedPlan {
    int32_t path;       // LORA_PATH_RELAY, FUSED, GROUPED, PREFILL or DECODE
    int32_t shared_a;   // every slice passes the same lora_a pointer
    int32_t noop;       // T == 0
};
int32_t packed_plan(const void *y, int64_t ldy, int64_t y_col_offset, const void *x, int64_t ldx,
                    int32_t T, int32_t K, const void *const *A, const void *const *B,
                    const int64_t *N, int32_t S, int32_t L, int32_t R, const int32_t *idx,
                    const int32_t *slot_rank, const float *scale, int32_t dtype, int32_t path,
                    uint32_t flags, const void *ws, size_t ws_bytes, PackedPlan *out);
int32_t packed_run(const PackedPlan &p, void *y, int64_t ldy, int64_t y_col_offset, const void *x,
                   int64_t ldx, int32_t T, int32_t K, const void *const *A, const void *const *B,
                   const int64_t *N, int32_t S, int32_t L, int32_t R, const int32_t *idx,
                   const int32_t *slot_rank, const float *scale, int32_t dtype, uint32_t flags,
                   void *ws, size_t ws_bytes, hipStream_t st);

// lora_workspace_check on lora_apply_packed_noalloc's array of the current
// device (static_scratch.hip): LORA_OK, or LORA_E_TIMEOUT after zero-filling it.
int32_t static_scratch_check(hipStream_t st);

// Launchers (host side), defined next to their kernels.
hipError_t launch_segments(const int32_t *idx, const int32_t *slot_rank, int32_t T, int32_t L,
                           int32_t R, const SegPtrs &seg, hipStream_t st);
// Items are tokens (topk == nullptr) or (token, k) pairs keyed by slot * E + expert.
hipError_t launch_segments_keyed(const int32_t *idx, const int32_t *slot_rank,
                                 const int32_t *topk, int32_t k, int32_t E, int32_t n_items,
                                 int32_t L, int32_t R, const SegPtrs &seg, hipStream_t st);
// One build of the two-pass (split) segment form: items are tokens (topk
// null) or (token, k) pairs keyed by slot * E + expert, counted by n_wg
// work-groups of kSegThreads items into `counts`, placed into `seg`.
struct SegJob {
    const int32_t *topk;
    int32_t k, E, n_items, n_wg;
    int32_t *counts;
    SegPtrs seg;
};
struct SegJobs {
    const int32_t *idx;
    const int32_t *slot_rank;
    int32_t L, R, n_jobs;
    SegJob job[2];
};
SegJob seg_job_of(const int32_t *topk, int32_t k, int32_t E, int32_t n_items, const SegPtrs &seg);
// Up to two builds over the same idx in one pair of launches (count, place).
hipError_t launch_segments_split(const int32_t *idx, const int32_t *slot_rank, int32_t L, int32_t R,
                                 const SegJob *jobs, int n_jobs, hipStream_t st);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);

// Writes the K-chunk partial sums; launch_dec_reduce (or the expand) adds them.
hipError_t launch_dec_shrink(int dtype, const void *x, int64_t ldx, int32_t T, int32_t K,
                             const Slices &sl, int32_t S, int32_t L, int32_t R,
                             const int32_t *slot_rank, const SegPtrs &seg, float *partial,
                             int32_t n_kchunks, hipStream_t st);
hipError_t launch_dec_reduce(int32_t T, int32_t S, int32_t L, int32_t R,
                             const int32_t *slot_rank, const SegPtrs &seg, const float *partial,
                             int32_t n_kchunks, float *buf, hipStream_t st);
// buf == nullptr: the expand sums the K-chunk partials itself (count read from
// the segment header, at most n_kchunks).
// TOKEN: one launch, work-group = (token, kTokenCols output columns) (k_dec_token).
constexpr int kTokenCols = 256;
constexpr int64_t kTokenRound = 1024;                 // work-groups resident at once (4 per CU)
constexpr int64_t kTokenMaxRoundPasses = 4;
constexpr int64_t kTokenMaxWgBytes = 1 << 20;         // lora_a bytes per work-group
constexpr int64_t kTokenMaxBytesBf16 = 72LL << 20;    // auto: lora_a bytes of all work-groups
constexpr int64_t kTokenMaxBytesNarrow = 44LL << 20;  // the same, bf16 outputs that RELAY could take
constexpr int64_t kTokenMaxBytesF32 = 512LL << 20;
hipError_t launch_dec_token(int dtype, void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T,
                            int32_t K, const Slices &sl, int32_t S, int32_t L, int32_t R,
                            const int32_t *idx, const int32_t *slot_rank, const float *scale,
                            hipStream_t st);
hipError_t launch_dec_expand(int dtype, void *y, int64_t ldy, const float *buf,
                             const float *partial, int32_t n_kchunks, int32_t T,
                             const Slices &sl, int32_t S, int32_t L, int32_t R,
                             const int32_t *slot_rank, const float *scale, const SegPtrs &seg,
                             hipStream_t st);

hipError_t launch_moe_align_out(const SegPtrs &pair, int32_t T, int32_t k, int32_t E, int32_t L,
                                int32_t bm, int32_t *sorted_ids, int32_t *block_expert,
                                int32_t *num_post_padded, hipStream_t st);

int32_t fused_max_groups(int32_t T, int32_t L);
hipError_t launch_dec_fused(void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T,
                            int32_t K, const Slices &sl, int32_t S, int32_t L, int32_t R,
                            const int32_t *idx, const int32_t *slot_rank, const float *scale,
                            hipStream_t st);

int32_t relay_max_groups(int32_t T, int32_t L);
// part: fp32 [S][K / kRelayKc][T][R]; sync: relay_sync_ints() int32; both zero
// on entry and left at zero.  err: set to 1 when a wait runs past its bound
// (or at once with give_up, a test hook); never cleared by the kernel.
hipError_t launch_dec_relay(void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T,
                            int32_t K, const Slices &sl, int32_t S, int32_t L, int32_t R,
                            const int32_t *idx, const int32_t *slot_rank, const float *scale,
                            float *part, int32_t *sync, int32_t *err, bool give_up,
                            hipStream_t st);

int32_t grp_max_groups(int32_t T, int32_t L);
int32_t grp_kchunks(int32_t K);
// Whether the grouped kernels find their groups from idx in one wave (else
// they read the segment table's decode tiles).
inline bool grp_discovers(int32_t T, int32_t L) { return L <= 64 && T <= 1024; }
// seg (nullable): the segment table the groups are read from, already built
// on the stream; null: each work-group discovers its group from idx.
// Partials: fp32 [S][grp_kchunks(K)][T][R], rows by slot-sorted position.
// n_kc_out (nullable) receives the chunk count for a later expand call.
hipError_t launch_grp_shrink(const void *x, int64_t ldx, int32_t T, int32_t K, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, float *part, int32_t *n_kc_out,
                             const SegPtrs *seg, hipStream_t st);
// Adds the partials (n_kc chunks, or the count at n_kc_in capped at n_kc) or,
// when buf is given, the token-ordered buffer [S][T][R]; shared_a: every slice
// adds slice 0's (the shrink of one lora_a shared by all slices).
hipError_t launch_grp_expand(void *y, int64_t ldy, int32_t T, int32_t n_kc, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, const float *scale, const float *part,
                             const float *buf, const int32_t *n_kc_in, const SegPtrs *seg,
                             hipStream_t st, bool shared_a = false);
// With a segment table of keyed tiles (slot * ekey + expert), pass ekey; T is
// the number of items (positions of the partials, rows of buf).
hipError_t launch_grp_reduce(int32_t T, int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, const float *part, int32_t n_kc,
                             float *buf, const SegPtrs *seg, hipStream_t st, int32_t ekey = 1);

// Grouped-problem mapping of the MFMA kernels.  A tile's key is
// slot * Ekey + expert (Ekey = 1 for token tiles); the lora tensor it reads is
// group slot * Ew + (Ew == 1 ? 0 : expert).  An item of the row list maps to
// x row item / x_div, buffer row item / buf_div and y row item / y_div.
struct GroupMap {
    int32_t Ekey = 1;
    int32_t Ew = 1;
    int32_t x_div = 1;
    int32_t buf_div = 1;
    int32_t y_div = 1;
    int32_t buf_rows = 0;          // rows of the [S][buf_rows][R] buffer
    int32_t buf_sstride = -1;      // expand: rows between the buffer's slices (-1: buf_rows,
                                   // 0: every slice reads slice 0, the shrink of a shared lora_a)
    const float *coef = nullptr;   // per-item factor (routing weight), or null
    int32_t ksum = 0;              // expand: buffer row of token t = sum_j coef[t*ksum+j] * buf[t*ksum+j]
    // expand, pair view (pair_k = k > 0): the segments are token tiles keyed
    // by slot, and the items are their (token, k) pairs, 64 to a tile; a pair
    // whose expert pair_ids[p] lies outside [0, pair_E) carries no delta
    int32_t pair_k = 0;
    const int32_t *pair_ids = nullptr;
    int32_t pair_E = 0;
};

// K splits of the row-oriented MFMA shrink.  A batch with few 64-token tiles
// for the CUs (many slots with a few tokens each) would stream each slot's
// lora_a through one CU; splitting K gives about 1024 work-groups, each with
// at least 8 stages of 64 columns, while the fp32 partials (written and read
// once) stay under an eighth of the shrink's input bytes.  1: no split.
inline int32_t pre_kspl(int32_t T, int32_t K, int32_t S, int32_t R, int32_t L, int32_t max_tiles,
                 int32_t cap_chunks) {
    const int32_t sr = S * R, ncb = sr <= 32 ? 1 : sr <= 64 ? 2 : 4;
    const int32_t n_cb = (sr + 32 * ncb - 1) / (32 * ncb);
    const int32_t nst = (K + 63) / 64;
    int32_t k = (1024 + max_tiles * n_cb - 1) / (max_tiles * n_cb);
    if (k > nst / 8) k = nst / 8;
    if (k > kMaxKcGrp) k = kMaxKcGrp;
    if (k > cap_chunks) k = cap_chunks;
    const double in_bytes = 2.0 * K * ((double)T + (double)(T < L ? T : L) * S * R);
    while (k > 1 && 8.0 * k * T * S * R > in_bytes / 8) --k;
    return k < 1 ? 1 : k;
}

// part (nullable): split K into *kspl_io chunks (fewer if K has fewer
// 64-column stages; the count used is written back) and write fp32 partials
// [S][kspl][T][R] by slot-sorted position instead of buf.
hipError_t launch_pre_shrink(const void *x, int64_t ldx, int32_t T, int32_t K, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *slot_rank,
                             const SegPtrs &seg, float *buf, hipStream_t st,
                             const GroupMap &gm = GroupMap(), float *part = nullptr,
                             int32_t *kspl_io = nullptr);
hipError_t launch_pre_expand(void *y, int64_t ldy, const float *buf, int32_t T, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *slot_rank,
                             const float *scale, const SegPtrs &seg, hipStream_t st,
                             const GroupMap &gm = GroupMap());

}  // namespace aa
