// Tile path: MFMA kernels over tiles of at most 64 tokens of one key (slot,
// or slot and expert for MoE) -- the SGMV regime of long per-slot runs, and
// batches of many slots or high ranks, whose shrink is then split over K.
//
// Tokens are grouped by key into tiles of 64 (two 32-row MFMA blocks).  The
// kernels use v_mfma_f32_32x32x16_bf16 (bf16 in, fp32 accumulate).  An operand
// fragment is 16 bytes per lane: row (l % 32), 8 consecutive k values starting
// at 8 * (l / 32).  The accumulator layout of a 32x32 block: lane l holds
// column (l % 32) and rows 8 * (i / 4) + 4 * (l / 32) + (i % 4), i = 0..15.
//
// Shrink (k_pre_shrink_rows): work-group = (tile, up to 128 of the S*R buffer
// columns, K split), x and lora_a rows staged through LDS in 64-column K
// stages; with a K split it writes fp32 partials that the grouped reduce
// kernel sums in order.
//
// Expand: work-group = (tile, group of output columns of one slice), the
// product formed transposed, D[n][t] = B[n][:] . buf[t][:], with the y tile,
// the lora_b block and the buffer rows staged through LDS so that every
// global access is row-contiguous: k_pre_expand_pipe (persistent, ranks 16,
// 32, 64, 128), k_pre_expand_rows (one item per work-group, ranks up to 64,
// per-item factors and the k-reduction); other ranks use k_pre_expand, whose
// lanes read and write y 8 bytes at a time in the MFMA layout.  Column groups
// are dealt to the 8 XCDs so each XCD keeps its slice of lora_b hot in its
// own L2 across a slot's tiles.
#include "common.hpp"

namespace aa {

namespace {

constexpr int kThreads = 256;
constexpr int kExpGroupCols = 512;     // output columns per expand work-group
constexpr int kExpWaveCols = kExpGroupCols / 4;
constexpr int kXcds = 8;

struct PreShrinkArgs {
    const uint16_t *x;
    int64_t ldx;
    int32_t T, K, S, L, R, n_cb;
    int32_t kspl, st_per;      // K splits and 64-column stages per split
    const int32_t *slot_rank;
    SegPtrs seg;
    Slices sl;
    float *buf;
    float *part;               // or null: fp32 [S][kspl][buf_rows][R] by slot-sorted position
    GroupMap gm;
};

struct PreExpandArgs {
    uint16_t *y;
    int64_t ldy;
    const float *buf;
    int32_t T, S, L, R, n_cg, per_xcd;
    const int32_t *slot_rank;
    const float *scale;
    SegPtrs seg;
    Slices sl;
    int32_t group_start[kMaxSlices + 1];
    GroupMap gm;
};

__device__ __forceinline__ bf16x8_t as_frag(const uint4 &u) { return __builtin_bit_cast(bf16x8_t, u); }

// 16-byte unit u of row n of an LDS block with U units per row.  16/U rows
// share one 256-byte bank window; the unit is XOR-ed with the row's window
// index so that the 16 rows read together by a quarter-wave fragment load (one
// unit each) hit 16 different 16-byte bank groups.  Whole-row writes stay
// conflict-free.  (U = 6 is not swizzled.)
__device__ __forceinline__ int swz(int n, int u, int U) {
    const int m = (U & (U - 1)) == 0 ? (n / (16 / U)) & (U - 1) : 0;
    return (n * U + (u ^ m)) << 4;
}

// Shrink: work-group = (64-item tile, block of 32 * NCB buffer columns), 8
// waves.  K advances in stages of 64 columns: a stage is the tile's x rows and
// the block's lora_a rows, 128 bytes each, loaded row-contiguously (one wave
// instruction = 8 whole rows), with 4 stages in flight in registers and two
// LDS buffers (one barrier per stage, LDS traffic only).  The 2 * NCB output
// blocks of 32 x 32 are shared by the 8 waves, each block's K steps split
// over 4 / NCB waves (v_mfma_f32_32x32x16_bf16).  Writes fp32 buf[s][t][j]
// for every column of the block that exists (zeros for j >= rank);
// K % 8 == 0, any rank.  With one column block (S * R <= 32) a tile's x rows
// are read by one work-group only and are loaded non-temporally, so that
// they do not push the lora_a rows other tiles reuse out of the L2 (the
// fused-MoE step 153 -> 147 us); with more blocks the work-groups of a tile
// share its x rows through the L2 (non-temporal there: prefill shrink 37 ->
// 45 us).
constexpr int kShThreads = 512;
constexpr int kShStageK = 64;          // K columns per stage (128 bytes of a row)
constexpr int kShNpf = 4;              // stages in flight

template <int NCB>
__global__ __launch_bounds__(kShThreads) void k_pre_shrink_rows(PreShrinkArgs a) {
    constexpr int ROWS = 64 + 32 * NCB;                // x rows, then lora_a rows
    constexpr int UNITS = ROWS * 8;                    // 16-byte units per stage
    constexpr int NU = (UNITS + kShThreads - 1) / kShThreads;
    // every thread stores all NU of its units (rows past ROWS are never read),
    // so no store of a stage sits under a branch
    __shared__ __attribute__((aligned(16))) char s_stage[2][NU * kShThreads * 16];
    static_assert((4 / NCB - 1) * 2 * NCB * 16 * 64 * 4 <= 2 * NU * kShThreads * 16,
                  "the staging area holds the K parts summed after the last stage");
    __shared__ int64_t s_brow[64];

    // Work-group i runs on XCD i % 8; XCD x takes a contiguous range of the
    // (slot-ordered) tiles, so each XCD's L2 holds the lora_a rows of only
    // the few slots its tiles belong to.
    const int xcd = blockIdx.x % kXcds;
    const int local = blockIdx.x / kXcds;
    const int cb = local % a.n_cb;
    const int ks = (local / a.n_cb) % a.kspl;     // K split: stages [sb, sb + nst)
    const int n_tiles = a.seg.header[3];
    const int per = (n_tiles + kXcds - 1) / kXcds;
    const int lt = local / (a.n_cb * a.kspl);
    if (lt >= per) return;
    const int tile = xcd * per + lt;
    if (tile >= n_tiles) return;
    const int4 tl = a.seg.tiles_pre[tile];
    const int s = tl.x / a.gm.Ekey, e = tl.x - s * a.gm.Ekey, p0 = tl.y, ntok = tl.z - tl.y;
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    const int64_t grp = (int64_t)s * a.gm.Ew + (a.gm.Ew == 1 ? 0 : e);
    const int SRf = a.S * a.R;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    if (tid < 64) s_brow[tid] = a.seg.perm[p0 + (tid < ntok ? tid : 0)] / a.gm.buf_div;

    // The rows this thread loads (fixed over K): clamped to valid ones.
    const uint16_t *rowp[NU];
    int uoff[NU];
#pragma unroll
    for (int v = 0; v < NU; ++v) {
        const int q = min(v * kShThreads + tid, UNITS - 1);
        const int row = q >> 3;
        uoff[v] = 8 * (q & 7);
        if (row < 64) {
            const int item = a.seg.perm[p0 + (row < ntok ? row : 0)];
            rowp[v] = a.x + (int64_t)(item / a.gm.x_div) * a.ldx;
        } else {
            const int c = cb * 32 * NCB + row - 64;
            const int sg = c / a.R, j = c - sg * a.R;
            const bool ok = c < SRf && j < r;
            rowp[v] = static_cast<const uint16_t *>(a.sl.a[ok ? sg : 0]) +
                      (grp * a.R + (ok ? j : 0)) * (int64_t)a.K;
        }
    }
    const int sb = ks * a.st_per;
    const int nst = min((a.K + kShStageK - 1) / kShStageK - sb, a.st_per);   // >= 1 (host)
    uint4 ring[kShNpf][NU];
    auto issue = [&](int slot, int st) {
#pragma unroll
        for (int v = 0; v < NU; ++v) {
            const int k = min((sb + st) * kShStageK + uoff[v], a.K - 8);
            // unit 0 of every thread is an x row (64 rows x 8 units = the
            // first 512); with one column block its rows are read by this
            // work-group only, and are streamed so as not to evict lora_a rows
            ring[slot][v] = NCB == 1 && v == 0 ? ldg_nt(rowp[v] + k) : ldg<uint4>(rowp[v] + k);
        }
    };
    // The store takes the loaded value through a mask, not a select: a select
    // of a load result becomes a branch, and the compiler waits for every
    // load in flight (the prefetched stages included) before it.
    auto put = [&](int slot, int st, char *buf) {
#pragma unroll
        for (int v = 0; v < NU; ++v) {
            const int q = v * kShThreads + tid;
            // stages past this split's last (padding to a multiple of
            // kShNpf) belong to the next split or lie past K: zeros
            const bool kin = st < nst && (sb + st) * kShStageK + uoff[v] < a.K;
            const uint32_t m = 0u - (uint32_t)kin;
            const uint4 u = ring[slot][v];
            *reinterpret_cast<uint4 *>(buf + swz(q >> 3, q & 7, 8)) = make_uint4(u.x & m, u.y & m, u.z & m, u.w & m);
        }
    };
    // Every wave computes: wave w takes the 32 x 32 block (token block w & 1,
    // column block cbk) over KSW of the stage's 4 K steps (part kp); the
    // KSPLIT parts of a block are summed in order after the last stage.  A
    // wave reads all its fragments of a stage before its first MFMA.
    constexpr int KSPLIT = 4 / NCB, KSW = kShStageK / 16 / KSPLIT;
    const int tb = w & 1, cbk = (w >> 1) % NCB, kp = (w >> 1) / NCB;
    floatx16_t acc = {};
    auto mma = [&](const char *buf) {
        uint4 xf[KSW], af[KSW];
#pragma unroll
        for (int i = 0; i < KSW; ++i) {
            const int u = 2 * (kp * KSW + i) + half;
            xf[i] = *reinterpret_cast<const uint4 *>(buf + swz(32 * tb + l32, u, 8));
            af[i] = *reinterpret_cast<const uint4 *>(buf + swz(64 + 32 * cbk + l32, u, 8));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < KSW; ++i)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(xf[i]), as_frag(af[i]), acc, 0, 0, 0);
    };
    // Stages past the split's last one (padding to a multiple of kShNpf) stage
    // zeros.  No branch around the loads.
    // The prologue issues the stages in ring order, as the loop refills them
    // (kept by scheduling barriers): the loop's first store then waits only
    // for its own stage.  Issued in another order, the loads of stage 0 could
    // be the youngest in flight when the loop is entered, and the wait at the
    // loop's head would drain every stage on each pass.
#pragma unroll
    for (int u = 0; u < kShNpf; ++u) {
        issue(u, min(u, nst - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int st0 = 0; st0 < nst; st0 += kShNpf) {
#pragma unroll
        for (int u = 0; u < kShNpf; ++u) {
            const int st = st0 + u;
            char *buf = s_stage[st & 1];
            put(u, st, buf);
            lds_barrier();
            issue(u, min(st + kShNpf, nst - 1));   // refill the slot just consumed
            mma(buf);
        }
    }
    __syncthreads();   // s_brow visible (and every stage consumed)
    if (KSPLIT > 1) {
        // parts 1 .. KSPLIT-1 of each block through the (now free) staging
        // area, added to part 0 in order
        float *s_red = reinterpret_cast<float *>(&s_stage[0][0]);
        const int blk = tb + 2 * cbk;
        if (kp > 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s_red[(((kp - 1) * 2 * NCB + blk) * 16 + i) * 64 + lane] = acc[i];
        }
        __syncthreads();
        if (kp > 0) return;
#pragma unroll
        for (int q = 1; q < KSPLIT; ++q)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] += s_red[(((q - 1) * 2 * NCB + blk) * 16 + i) * 64 + lane];
    }

    // acc[i]: token 32*tb + 8*(i/4) + 4*half + (i%4), column 32*(NCB*cb + cbk) + l32
    const int c = cb * 32 * NCB + 32 * cbk + l32;
    if (c >= SRf) return;
    const int sg = c / a.R, j = c - sg * a.R;
    if (a.part) {
        float *dst = a.part + (((int64_t)sg * a.kspl + ks) * a.gm.buf_rows + p0) * a.R + j;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 32 * tb + 8 * (i >> 2) + 4 * half + (i & 3);
            if (t < ntok) dst[(int64_t)t * a.R] = j < r ? acc[i] : 0.0f;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 32 * tb + 8 * (i >> 2) + 4 * half + (i & 3);
        if (t < ntok) a.buf[((int64_t)sg * a.gm.buf_rows + s_brow[t]) * a.R + j] = j < r ? acc[i] : 0.0f;
    }
}

// The tiles an expand walks.  Normally the segment table's prefill tiles; in
// the pair view (gm.pair_k = k > 0) the table holds token tiles keyed by slot
// and expand tile j is the (j % k)-th run of kPreTile (token, k) pairs of
// token tile j / k: position p of a token tile's pair run is pair
// perm[p / k] * k + p % k (the pairs of a token share its slot).  A run past
// the token tile's pairs is empty.
__device__ __forceinline__ int exp_n_tiles(const PreExpandArgs &a) {
    return a.seg.header[3] * (a.gm.pair_k ? a.gm.pair_k : 1);
}
__device__ __forceinline__ int4 exp_tile(const PreExpandArgs &a, int j) {
    const int k = a.gm.pair_k;
    if (!k) return a.seg.tiles_pre[j];
    const int4 t = a.seg.tiles_pre[j / k];
    const int b = t.y * k + kPreTile * (j % k);
    return make_int4(t.x, b, min(t.z * k, b + kPreTile), 0);
}
__device__ __forceinline__ int exp_perm(const PreExpandArgs &a, int p) {
    const int k = a.gm.pair_k;
    return k ? a.seg.perm[p / k] * k + p % k : a.seg.perm[p];
}
// whether an item of a tile carries a delta (pair view: its expert in range)
__device__ __forceinline__ bool exp_live(const PreExpandArgs &a, int item) {
    return !a.gm.pair_k || (uint32_t)a.gm.pair_ids[item] < (uint32_t)a.gm.pair_E;
}

// Per-lane view of one token block of an expand tile: the item, its y row, its
// scale factor and the 8 buffer values of rank group jj (k-summed if asked).
struct ExpItem {
    int item;
    bool ok;
    int64_t yrow;
    float scl;
};

__device__ __forceinline__ ExpItem exp_item(const PreExpandArgs &a, int p0, int row, int ntok,
                                            float sc) {
    ExpItem it;
    const bool in = row < ntok;
    it.item = exp_perm(a, p0 + (in ? row : 0));   // clamped: never stored
    it.ok = in && exp_live(a, it.item);
    it.yrow = it.item / a.gm.y_div;
    const float cf = (a.gm.coef && !a.gm.ksum) ? a.gm.coef[it.item] : 1.0f;
    it.scl = sc * cf;
    return it;
}

// 8 buffer values (ranks jj .. jj+7) of an item for slice sg, as two float4
// (the caller zeroes ranks at or past the slot's rank when it packs them: an
// expand-only caller may leave them arbitrary).
__device__ __forceinline__ void buf_vals(const PreExpandArgs &a, int sg, int item, int jj,
                                         float4 &v0, float4 &v1) {
    if (a.gm.ksum) {
        v0 = make_float4(0, 0, 0, 0);
        v1 = make_float4(0, 0, 0, 0);
        for (int j = 0; j < a.gm.ksum; ++j) {
            const int64_t br = (int64_t)item * a.gm.ksum + j;
            const float w = a.gm.coef ? a.gm.coef[br] : 1.0f;
            const float *bp = a.buf + ((int64_t)sg * a.gm.buf_sstride + br) * a.R + jj;
            const float4 u0 = ldg<float4>(bp), u1 = ldg<float4>(bp + 4);
            v0.x += w * u0.x; v0.y += w * u0.y; v0.z += w * u0.z; v0.w += w * u0.w;
            v1.x += w * u1.x; v1.y += w * u1.y; v1.z += w * u1.z; v1.w += w * u1.w;
        }
    } else {
        const float *bp = a.buf + ((int64_t)sg * a.gm.buf_sstride + item / a.gm.buf_div) * a.R + jj;
        v0 = ldg<float4>(bp);
        v1 = ldg<float4>(bp + 4);
    }
}

__device__ __forceinline__ uint4 pack_frag(const float4 &v0, const float4 &v1, int jj, int r) {
    return make_uint4(pack_bf16x2(jj + 0 < r ? v0.x : 0.f, jj + 1 < r ? v0.y : 0.f),
                      pack_bf16x2(jj + 2 < r ? v0.z : 0.f, jj + 3 < r ? v0.w : 0.f),
                      pack_bf16x2(jj + 4 < r ? v1.x : 0.f, jj + 5 < r ? v1.y : 0.f),
                      pack_bf16x2(jj + 6 < r ? v1.z : 0.f, jj + 7 < r ? v1.w : 0.f));
}

// Generic expand, any rank (passes of up to 128 accumulate before the single
// rounding of y).
__global__ __launch_bounds__(kThreads) void k_pre_expand(PreExpandArgs a) {
    const int xcd = blockIdx.x % kXcds;
    const int local = blockIdx.x / kXcds;
    const int tile = local / a.per_xcd;
    const int cg = (local - tile * a.per_xcd) * kXcds + xcd;
    if (cg >= a.n_cg) return;
    if (tile >= exp_n_tiles(a)) return;
    const int4 tl = exp_tile(a, tile);
    if (tl.z <= tl.y) return;
    const int s = tl.x / a.gm.Ekey, e = tl.x - s * a.gm.Ekey, p0 = tl.y, ntok = tl.z - tl.y;
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    const int64_t grp = (int64_t)s * a.gm.Ew + (a.gm.Ew == 1 ? 0 : e);
    int sg = 0;
    while (sg + 1 < a.S && cg >= a.group_start[sg + 1]) ++sg;
    const int64_t Ns = a.sl.n[sg];
    const float sc = a.scale[s];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int nks = (r + 15) >> 4;                      // rank steps of 16
    const int nbase = (cg - a.group_start[sg]) * kExpGroupCols + w * kExpWaveCols;
    if (nbase >= Ns) return;

    ExpItem it[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) it[tb] = exp_item(a, p0, tb * 32 + l32, ntok, sc);
    const uint16_t *bbase = static_cast<const uint16_t *>(a.sl.b[sg]) + grp * Ns * a.R;
    uint16_t *ybase = a.y + a.sl.off[sg];

    uint4 bfrag[2][8];
    auto load_bfrag = [&](int kp, int nk) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int jj = (kp + ks) * 16 + 8 * half;
                uint4 f = make_uint4(0, 0, 0, 0);
                if (ks < nk) {
                    float4 v0, v1;
                    buf_vals(a, sg, it[tb].item, jj, v0, v1);
                    f = pack_frag(v0, v1, jj, r);
                }
                bfrag[tb][ks] = f;
            }
    };
    const bool one_pass = nks <= 8;
    if (one_pass) load_bfrag(0, nks);

    for (int nb = 0; nb < kExpWaveCols / 32; ++nb) {
        const int n0 = nbase + nb * 32;
        if (n0 >= Ns) break;
        const int nrow = min(n0 + l32, (int)Ns - 1);     // A-operand row (output column)
        const uint16_t *brow = bbase + (int64_t)nrow * a.R;
        floatx16_t acc[2] = {{}, {}};
        for (int kp = 0; kp < nks; kp += 8) {
            const int nk = min(8, nks - kp);
            if (!one_pass) load_bfrag(kp, nk);
            uint4 afrag[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                afrag[ks] = ks < nk ? ldg<uint4>(brow + (kp + ks) * 16 + 8 * half) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks < nk) {
                    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(afrag[ks]), as_frag(bfrag[0][ks]), acc[0], 0, 0, 0);
                    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(afrag[ks]), as_frag(bfrag[1][ks]), acc[1], 0, 0, 0);
                }
            }
        }
        // Lane holds columns n0 + 8g + 4*half + {0..3} of its item in each token block.
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            if (!it[tb].ok) continue;
            uint16_t *yrow = ybase + it[tb].yrow * a.ldy;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 8 * g + 4 * half;
                if (n < Ns) {
                    uint2 *yp = reinterpret_cast<uint2 *>(yrow + n);
                    const uint2 yv = *yp;
                    const float c = it[tb].scl;
                    uint2 o;
                    o.x = pack_bf16x2(bf16_lo(yv.x) + c * acc[tb][4 * g + 0],
                                      bf16_hi(yv.x) + c * acc[tb][4 * g + 1]);
                    o.y = pack_bf16x2(bf16_lo(yv.y) + c * acc[tb][4 * g + 2],
                                      bf16_hi(yv.y) + c * acc[tb][4 * g + 3]);
                    *yp = o;
                }
            }
        }
    }
}

// Row-oriented expand for ranks <= 64 (R = 16 * NKS): work-group = (64-token
// tile, 256 output columns of one slice), 4 waves, two work-groups per CU.
// Every global access is row-contiguous: the y tile is read into LDS with
// each wave instruction covering two 512-byte row pieces, the lora_b rows of
// the 256 columns are one contiguous block, the buffer rows are whole rows.
// The product D[n][t] = B[n][:] . buf[t][:] (v_mfma_f32_32x32x16_bf16) is
// added to the y tile in LDS, which is then written back row by row.
constexpr int kRowTok = 64;                  // tokens per tile (kPreTile)
constexpr int kRowCols = 256;                // output columns per work-group
constexpr int kRowYStride = kRowCols + 8;    // bf16 elements per LDS y row (528 B)

template <int NKS>
__global__ __launch_bounds__(kThreads, 2) void k_pre_expand_rows(PreExpandArgs a) {
    constexpr int R = 16 * NKS;
    constexpr int U = R / 8;                       // 16-byte units per lora_b / buffer row
    constexpr int YU = kRowCols / 8;               // 16-byte units per y row piece (32)
    constexpr int NY = kRowTok * YU / kThreads;    // y units per thread (8)
    constexpr int NBU = kRowCols * U / kThreads;   // lora_b units per thread (R / 8)
    constexpr int NFU = kRowTok * (R / 4) / kThreads;   // fp32 buffer units (float4) per thread
    static_assert(NFU >= 1, "rank too small for one buffer unit per thread");
    __shared__ __attribute__((aligned(16))) uint16_t s_y[kRowTok * kRowYStride];
    __shared__ __attribute__((aligned(16))) char s_b[kRowCols * U * 16];
    __shared__ __attribute__((aligned(16))) char s_buf[kRowTok * U * 16];
    __shared__ int64_t s_yrow[kRowTok];
    __shared__ float s_scl[kRowTok];
    __shared__ int s_live[kRowTok];

    const int xcd = blockIdx.x % kXcds;
    const int local = blockIdx.x / kXcds;
    const int tile = local / a.per_xcd;
    const int cg = (local - tile * a.per_xcd) * kXcds + xcd;
    if (cg >= a.n_cg) return;
    if (tile >= exp_n_tiles(a)) return;
    const int4 tl = exp_tile(a, tile);
    if (tl.z <= tl.y) return;
    const int s = tl.x / a.gm.Ekey, e = tl.x - s * a.gm.Ekey, p0 = tl.y, ntok = tl.z - tl.y;
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    const int64_t grp = (int64_t)s * a.gm.Ew + (a.gm.Ew == 1 ? 0 : e);
    int sg = 0;
    while (sg + 1 < a.S && cg >= a.group_start[sg + 1]) ++sg;
    const int Ns = (int)a.sl.n[sg];
    const int n_base = (cg - a.group_start[sg]) * kRowCols;
    const float sc = a.scale[s];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    // ---- per-token row, scale and buffer item (tokens past the tile: clamped)
    if (tid < kRowTok) {
        const int row = tid < ntok ? tid : 0;
        const int item = exp_perm(a, p0 + row);
        s_yrow[tid] = item / a.gm.y_div;
        s_scl[tid] = sc * ((a.gm.coef && !a.gm.ksum) ? a.gm.coef[item] : 1.0f);
        s_live[tid] = tid < ntok && exp_live(a, item);
    }
    __syncthreads();

    // ---- all loads -------------------------------------------------------
    uint16_t *ybase = a.y + a.sl.off[sg];
    uint4 yv[NY];
#pragma unroll
    for (int i = 0; i < NY; ++i) {
        // rows past the tile's tokens all read one 16-byte unit: an
        // instruction of padding rows costs one request
        const int q = i * kThreads + tid;
        const int row = q / YU, col = n_base + 8 * (q % YU);
        yv[i] = ldg_nt(ybase + s_yrow[row] * a.ldy + (row < ntok ? min(col, Ns - 8) : n_base));
    }
    const char *bblk = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.sl.b[sg]) + grp * Ns * R);
    uint4 bv[NBU];
#pragma unroll
    for (int i = 0; i < NBU; ++i) {
        const int q = i * kThreads + tid;
        const int n = min(n_base + q / U, Ns - 1);
        bv[i] = ldg<uint4>(reinterpret_cast<const uint4 *>(bblk + ((int64_t)n * U + q % U) * 16));
    }
    float4 fv[NFU];
    int frow[NFU];
#pragma unroll
    for (int i = 0; i < NFU; ++i) {
        const int q = i * kThreads + tid;
        const int t = q / (R / 4), j = 4 * (q % (R / 4));
        frow[i] = t;
        const int row = t < ntok ? t : 0;
        const int item = exp_perm(a, p0 + row);
        if (!a.gm.ksum) {
            fv[i] = ldg<float4>(a.buf + ((int64_t)sg * a.gm.buf_sstride + item / a.gm.buf_div) * R + j);
        } else {
            // the k-reduced buffer row of token `item`: sum_j coef * buf over its pairs
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int kk = 0; kk < a.gm.ksum; ++kk) {
                const int64_t br = (int64_t)item * a.gm.ksum + kk;
                const float cw = a.gm.coef ? a.gm.coef[br] : 1.0f;
                const float4 u = ldg<float4>(a.buf + ((int64_t)sg * a.gm.buf_sstride + br) * R + j);
                acc.x += cw * u.x; acc.y += cw * u.y; acc.z += cw * u.z; acc.w += cw * u.w;
            }
            fv[i] = acc;
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- into LDS --------------------------------------------------------
#pragma unroll
    for (int i = 0; i < NY; ++i) {
        const int q = i * kThreads + tid;
        *reinterpret_cast<uint4 *>(&s_y[(q / YU) * kRowYStride + 8 * (q % YU)]) = yv[i];
    }
#pragma unroll
    for (int i = 0; i < NBU; ++i) {
        const int q = i * kThreads + tid;
        *reinterpret_cast<uint4 *>(s_b + swz(q / U, q % U, U)) = bv[i];
    }
#pragma unroll
    for (int i = 0; i < NFU; ++i) {
        const int q = i * kThreads + tid;
        const int t = frow[i], j = 4 * (q % (R / 4));
        const bool ok = t < ntok;
        uint2 o;
        o.x = pack_bf16x2(ok && j < r ? fv[i].x : 0.f, ok && j + 1 < r ? fv[i].y : 0.f);
        o.y = pack_bf16x2(ok && j + 2 < r ? fv[i].z : 0.f, ok && j + 3 < r ? fv[i].w : 0.f);
        // 8-byte half of unit j / 8 of row t
        *reinterpret_cast<uint2 *>(s_buf + swz(t, j >> 3, U) + ((j & 4) << 1)) = o;
    }
    __syncthreads();

    // ---- D[n][t]: wave w takes columns 64w .. 64w + 63, both token blocks ----
    floatx16_t acc[2][2] = {{{}, {}}, {{}, {}}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int u = 2 * ks + half;
        uint4 bf[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) bf[tb] = *reinterpret_cast<const uint4 *>(s_buf + swz(32 * tb + l32, u, U));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const uint4 af = *reinterpret_cast<const uint4 *>(s_b + swz(64 * w + 32 * nb + l32, u, U));
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(af), as_frag(bf[tb]), acc[nb][tb], 0, 0, 0);
        }
    }
    // lane: token 32*tb + l32, columns 64w + 32nb + 8g + 4*half + {0..3}
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = 32 * tb + l32;
        if (t < ntok) {
            const float c = s_scl[t];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 *yp = reinterpret_cast<uint2 *>(&s_y[t * kRowYStride + 64 * w + 32 * nb + 8 * g + 4 * half]);
                    const uint2 y0 = *yp;
                    uint2 o;
                    o.x = pack_bf16x2(bf16_lo(y0.x) + c * acc[nb][tb][4 * g + 0], bf16_hi(y0.x) + c * acc[nb][tb][4 * g + 1]);
                    o.y = pack_bf16x2(bf16_lo(y0.y) + c * acc[nb][tb][4 * g + 2], bf16_hi(y0.y) + c * acc[nb][tb][4 * g + 3]);
                    *yp = o;
                }
        }
    }
    __syncthreads();

    // ---- write the tile back, row by row (rows that carry a delta) ---------
#pragma unroll
    for (int i = 0; i < NY; ++i) {
        const int q = i * kThreads + tid;
        const int row = q / YU, col = n_base + 8 * (q % YU);
        if (s_live[row] && col < Ns)
            stg_nt(ybase + s_yrow[row] * a.ldy + col,
                   *reinterpret_cast<const uint4 *>(&s_y[row * kRowYStride + 8 * (q % YU)]));
    }
}

// Persistent, software-pipelined form of k_pre_expand_rows for the common case
// (no per-item factor, no k-reduction): two or three work-groups per CU, each
// walking a strided list of (tile, column group) items of its XCD.  The y /
// lora_b / buffer loads of item k+1 are in flight while item k is multiplied,
// added and stored; the per-item token lists (tile descriptor -> perm gather
// -> y and buffer rows) run two and three items ahead in registers and reach
// the loads through double-buffered LDS slots, so no dependent load sits on
// the critical path.  Items are ordered tile first: the work-groups of an XCD
// work at any time on a few consecutive (slot-ordered) tiles with all the
// XCD's column groups, so each tile's buffer rows and the few slots' lora_b
// blocks are fetched into its L2 once (ordered column group first, the
// lora_b blocks of a slot were evicted between its tiles and fetched again:
// about one more pass over lora_b on the prefill gate_up workload).  Item
// f = tile * n_cg + cg runs on XCD f % 8: with n_cg a multiple of 8 each XCD
// keeps the same column groups for every tile (its lora_b columns stay in its
// L2); otherwise the XCDs still get equal shares and no item is empty.
// Ranks up to 128 (R = 16 * NKS); CW output columns per item (256 up to rank
// 64, 128 above, so that two work-groups still fit a CU's LDS).  Of each
// lora_b row only the first 2 * ceil(r / 16) units (rounded up to a power of
// two) are read, r the item's slot rank: slots of low rank in a tensor padded
// to a high rank do not pay for the padding.
// A load at a wave-uniform address of data no work-group of the launch
// writes, through the scalar cache (s_load: counted by lgkmcnt, so waits for
// the vector loads in flight do not depend on it).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 ldg_uniform(const int4 *p) {
    const i32x4_t v = *reinterpret_cast<const __attribute__((address_space(4))) i32x4_t *>(
        reinterpret_cast<uintptr_t>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}

template <int NKS, int CW>
__global__ __launch_bounds__(kThreads, NKS == 1 ? 3 : 2) void k_pre_expand_pipe(PreExpandArgs a) {
    constexpr int R = 16 * NKS;
    constexpr int U = R / 8;                       // 16-byte units per lora_b row (power of two)
    constexpr int LGU = U == 2 ? 1 : U == 4 ? 2 : U == 8 ? 3 : 4;
    constexpr int YS = CW + 8;                     // bf16 elements per LDS y row
    constexpr int YU = CW / 8;
    constexpr int NY = kRowTok * YU / kThreads;
    constexpr int NBU = CW * U / kThreads;
    constexpr int NFU = kRowTok * (R / 4) / kThreads;
    constexpr int WC = CW / 4;                     // columns per wave
    constexpr int NB = WC / 32;                    // 32-column MFMA blocks per wave
    // Ranks 32 to 128 take the loop whose every pass issues the same memory
    // operations (below); rank 16 keeps the one with skipped loads and stores,
    // which needs fewer registers (165 against 184), so that three
    // work-groups fit a CU as its grid assumes.
    constexpr bool kStatic = NKS > 1;
    constexpr bool kPutLive = NKS >= 8;
    static_assert((U & (U - 1)) == 0 && U <= 16, "lora_b rows of 2, 4, 8 or 16 units");
    __shared__ __attribute__((aligned(16))) uint16_t s_y[kRowTok * YS];
    __shared__ __attribute__((aligned(16))) char s_b[CW * U * 16];
    __shared__ __attribute__((aligned(16))) char s_buf[kRowTok * U * 16];
    __shared__ int64_t s_yrow[2][kRowTok];
    __shared__ int64_t s_brow[2][kRowTok];
    __shared__ float s_sc[2];
    __shared__ int s_rk[2];

    const int xcd = blockIdx.x % kXcds;
    const int lw = blockIdx.x / kXcds;
    const int nw = gridDim.x / kXcds;
    const int n_tiles = a.seg.header[3];
    // items f = tile * n_cg + cg, dealt round-robin to the XCDs (f % 8)
    const int64_t n_items = (int64_t)n_tiles * a.n_cg;
    const int n_x = n_items > xcd ? (int)((n_items - xcd + kXcds - 1) / kXcds) : 0;
    const int cnt = lw < n_x ? (n_x - lw + nw - 1) / nw : 0;
    if (cnt == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    // item k of this work-group (clamped to its last one): tile and column group
    auto item_of = [&](int k) { return (int64_t)(lw + min(k, cnt - 1) * nw) * kXcds + xcd; };
    auto tile_of = [&](int k) { return (int)(item_of(k) / a.n_cg); };
    auto cg_of = [&](int k) { return (int)(item_of(k) % a.n_cg); };
    struct Col { int sg, Ns, n_base; };
    auto col_of = [&](int k) {
        const int cg = cg_of(k);
        Col c;
        c.sg = 0;
        while (c.sg + 1 < a.S && cg >= a.group_start[c.sg + 1]) ++c.sg;
        c.Ns = (int)a.sl.n[c.sg];
        c.n_base = (cg - a.group_start[c.sg]) * CW;
        return c;
    };
    // log2 of the lora_b units per row an item reads: 2 * ceil(r / 16) rounded up
    auto lg_units = [&](int r) { return min(32 - __clz(2 * ((r + 15) >> 4) - 1), LGU); };
    // metadata loads of item k: its token (thread < 64), slot rank and scale
    struct Meta { int item; int rank; float sc; };
    auto meta_load = [&](const int4 &tl) {
        Meta m;
        const int ntok = tl.z - tl.y;
        m.item = a.seg.perm[tl.y + min(tid & 63, ntok - 1)];
        const int sl = tl.x / a.gm.Ekey;
        // through the global address space (a select between slot_rank and
        // the argument R would make it a FLAT load, which the compiler's
        // waits treat as unordered: every wait after it would be for zero)
        const int32_t *rk = a.slot_rank ? a.slot_rank + sl : reinterpret_cast<const int32_t *>(a.scale + sl);
        const int32_t rv = *reinterpret_cast<const __attribute__((address_space(1))) int32_t *>(
            reinterpret_cast<uintptr_t>(rk));
        m.rank = a.slot_rank ? rv : a.R;
        m.sc = a.scale[sl];
        return m;
    };
    auto meta_put = [&](const Meta &m, int slot) {
        if (tid < kRowTok) {
            s_yrow[slot][tid] = m.item / a.gm.y_div;
            s_brow[slot][tid] = m.item / a.gm.buf_div;
        }
        if (tid == 0) {
            s_rk[slot] = max(1, min(m.rank, a.R));
            s_sc[slot] = m.sc;
        }
    };
    // (zero at the start: lanes whose loads are masked off keep them)
    uint4 yv[NY], bv[NBU];
    float4 fv[NFU];
#pragma unroll
    for (int i = 0; i < NY; ++i) yv[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < NBU; ++i) bv[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < NFU; ++i) fv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    // data loads of item k (its metadata in LDS slot k & 1)
    auto data_load = [&](const int4 &tl, const Col &c, int slot) {
        const int s = tl.x / a.gm.Ekey, e = tl.x - s * a.gm.Ekey;
        const int64_t grp = (int64_t)s * a.gm.Ew + (a.gm.Ew == 1 ? 0 : e);
        const uint16_t *ybase = a.y + a.sl.off[c.sg];
        // At ranks 32 to 128 each load is masked per lane to the units that
        // exist (token rows of the tile, units of the slot's rank, buffer
        // entries below it): an instruction with no lane left is skipped, the
        // others address only their useful lanes (the texture addresser's
        // time per instruction goes with its lanes: 20 full instructions per
        // item were most of an item's time), and the compiler still counts
        // every load, so each wait covers only what it needs.  Lanes left out
        // keep stale registers that nothing reads.  At rank 16 the
        // work-group's y instructions past the tile's tokens are skipped and
        // padding rows read one 16-byte unit of the last token row.
        const int ntk = tl.z - tl.y;
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            const int q = i * kThreads + tid;
            const int col = q / YU < ntk ? min(c.n_base + 8 * (q % YU), c.Ns - 8) : c.n_base;
            if (kStatic ? q / YU < ntk : i * (kThreads / YU) < ntk)   // rank 16: instruction i holds a token row
                yv[i] = ldg_nt(ybase + s_yrow[slot][q / YU] * a.ldy + col);
        }
        // units q < CW * Ue of the block, Ue = 1 << lgu per row; the rest repeat the last
        const int lgu = lg_units(s_rk[slot]);
        const int last = (CW << lgu) - 1;
        const char *bblk = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.sl.b[c.sg]) + grp * c.Ns * R);
#pragma unroll
        for (int i = 0; i < NBU; ++i) {
            const int q = min(i * kThreads + tid, last);
            const int n = min(c.n_base + (q >> lgu), c.Ns - 1);
            if (!kStatic || i * kThreads + tid <= last)
                bv[i] = ldg<uint4>(reinterpret_cast<const uint4 *>(bblk + ((int64_t)n * U + (q & ((1 << lgu) - 1))) * 16));
        }
        // buffer rows: entries j >= r are dropped, so their loads repeat the
        // last needed float4 of the row (no extra cache lines)
        const int jmax = 4 * ((s_rk[slot] + 3) / 4 - 1);
#pragma unroll
        for (int i = 0; i < NFU; ++i) {
            const int q = i * kThreads + tid;
            const int t = q / (R / 4), j = 4 * (q % (R / 4));
            if (!kStatic || (t < ntk && j <= jmax))
                fv[i] = ldg<float4>(a.buf + ((int64_t)c.sg * a.gm.buf_sstride + s_brow[slot][t]) * R + min(j, jmax));
        }
    };

    // ---- prologue: items 0, 1, 2 ------------------------------------------
    int4 tl0 = ldg_uniform(&a.seg.tiles_pre[tile_of(0)]);
    int4 tl1 = ldg_uniform(&a.seg.tiles_pre[tile_of(1)]);
    int4 tl2 = ldg_uniform(&a.seg.tiles_pre[tile_of(2)]);
    meta_put(meta_load(tl0), 0);
    Meta m1 = meta_load(tl1);
    Col c0 = col_of(0), c1 = col_of(1);
    __syncthreads();
    data_load(tl0, c0, 0);

    if constexpr (!kStatic) {
        for (int k = 0; k < cnt; ++k) {
            const int slot = k & 1, nslot = slot ^ 1;
            const int ntok = tl0.z - tl0.y;
            const int r = s_rk[slot];
            const int nks = (r + 15) >> 4;
            // 1. item k into LDS; item k+1's metadata into its slot
            {
#pragma unroll
                for (int i = 0; i < NY; ++i) {
                    const int q = i * kThreads + tid;
                    *reinterpret_cast<uint4 *>(&s_y[(q / YU) * YS + 8 * (q % YU)]) = yv[i];
                }
                const int lgu = lg_units(r);
#pragma unroll
                for (int i = 0; i < NBU; ++i) {
                    const int q = i * kThreads + tid;
                    if (q < (CW << lgu))
                        *reinterpret_cast<uint4 *>(s_b + swz(q >> lgu, q & ((1 << lgu) - 1), U)) = bv[i];
                }
#pragma unroll
                for (int i = 0; i < NFU; ++i) {
                    const int q = i * kThreads + tid;
                    const int t = q / (R / 4), j = 4 * (q % (R / 4));
                    const bool ok = t < ntok;
                    uint2 o;
                    o.x = pack_bf16x2(ok && j < r ? fv[i].x : 0.f, ok && j + 1 < r ? fv[i].y : 0.f);
                    o.y = pack_bf16x2(ok && j + 2 < r ? fv[i].z : 0.f, ok && j + 3 < r ? fv[i].w : 0.f);
                    *reinterpret_cast<uint2 *>(s_buf + swz(t, j >> 3, U) + ((j & 4) << 1)) = o;
                }
                meta_put(m1, nslot);
            }
            __syncthreads();
            // 2. loads of item k+1, metadata of item k+2, descriptor of item k+3
            const float sc = s_sc[slot];
            const Col ck = c0;
            if (k + 1 < cnt) data_load(tl1, c1, nslot);   // the last item has none (a reload of it
                                                          // would fetch its y rows once more)
            const Meta m2 = meta_load(tl2);
            const int4 tl3 = ldg<int4>(&a.seg.tiles_pre[tile_of(k + 3)]);
            // 3. D[n][t] for item k over its slot's rank steps, added into the y tile
            {
                floatx16_t acc[NB][2];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[nb][0] = acc[nb][1] = floatx16_t{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if (ks < nks) {
                        const int u = 2 * ks + half;
                        uint4 bfr[2];
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) bfr[tb] = *reinterpret_cast<const uint4 *>(s_buf + swz(32 * tb + l32, u, U));
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const uint4 af = *reinterpret_cast<const uint4 *>(s_b + swz(WC * w + 32 * nb + l32, u, U));
#pragma unroll
                            for (int tb = 0; tb < 2; ++tb)
                                acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(af), as_frag(bfr[tb]), acc[nb][tb], 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const int t = 32 * tb + l32;
                    if (t < ntok) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                uint2 *yp = reinterpret_cast<uint2 *>(&s_y[t * YS + WC * w + 32 * nb + 8 * g + 4 * half]);
                                const uint2 y0 = *yp;
                                uint2 o;
                                o.x = pack_bf16x2(bf16_lo(y0.x) + sc * acc[nb][tb][4 * g + 0], bf16_hi(y0.x) + sc * acc[nb][tb][4 * g + 1]);
                                o.y = pack_bf16x2(bf16_lo(y0.y) + sc * acc[nb][tb][4 * g + 2], bf16_hi(y0.y) + sc * acc[nb][tb][4 * g + 3]);
                                *yp = o;
                            }
                    }
                }
            }
            __syncthreads();
            // 4. item k back to y, row by row
            {
                uint16_t *ybase = a.y + a.sl.off[ck.sg];
#pragma unroll
                for (int i = 0; i < NY; ++i) {
                    const int q = i * kThreads + tid;
                    const int row = q / YU, col = ck.n_base + 8 * (q % YU);
                    if (row < ntok && col < ck.Ns)
                        stg_nt(ybase + s_yrow[slot][row] * a.ldy + col,
                               *reinterpret_cast<const uint4 *>(&s_y[row * YS + 8 * (q % YU)]));
                }
            }
            __syncthreads();
            tl0 = tl1; tl1 = tl2; tl2 = tl3;
            m1 = m2;
            c0 = c1; c1 = col_of(k + 2);
        }
    } else {
        // One item (k): the last has no prefetch; every other pass issues the
        // same memory operations, so the wait at its head is for item k's data only.
        auto item = [&](int k, auto prefetch) {
            constexpr bool kPrefetch = decltype(prefetch)::value;
            const int slot = k & 1, nslot = slot ^ 1;
            // descriptor of item k+3 through the scalar cache, issued before the
            // wait for item k's data
            const int4 tl3 = ldg_uniform(&a.seg.tiles_pre[tile_of(k + 3)]);
            const int ntok = tl0.z - tl0.y;
            const int r = s_rk[slot];
            const int nks = (r + 15) >> 4;
            // 1. item k into LDS; item k+1's metadata into its slot
            {
                // at rank 128 only the rows and rank entries that are read: the
                // tile's token rows (the y tile's others are never stored back,
                // and the buffer's only reach discarded products) and the
                // buffer entries of the slot's rank steps (zero past r); the
                // LDS writes of a tile of a few tokens were a sixth of an item's
                // time in batches of many slots (at lower ranks the masks cost
                // more than they save)
#pragma unroll
                for (int i = 0; i < NY; ++i) {
                    const int q = i * kThreads + tid;
                    if (!kPutLive || q / YU < ntok)
                        *reinterpret_cast<uint4 *>(&s_y[(q / YU) * YS + 8 * (q % YU)]) = yv[i];
                }
                const int lgu = lg_units(r);
#pragma unroll
                for (int i = 0; i < NBU; ++i) {
                    const int q = i * kThreads + tid;
                    if (q < (CW << lgu))
                        *reinterpret_cast<uint4 *>(s_b + swz(q >> lgu, q & ((1 << lgu) - 1), U)) = bv[i];
                }
#pragma unroll
                for (int i = 0; i < NFU; ++i) {
                    const int q = i * kThreads + tid;
                    const int t = q / (R / 4), j = 4 * (q % (R / 4));
                    const bool ok = kPutLive || t < ntok;
                    uint2 o;
                    o.x = pack_bf16x2(ok && j < r ? fv[i].x : 0.f, ok && j + 1 < r ? fv[i].y : 0.f);
                    o.y = pack_bf16x2(ok && j + 2 < r ? fv[i].z : 0.f, ok && j + 3 < r ? fv[i].w : 0.f);
                    if (!kPutLive || (t < ntok && j < 16 * nks))
                        *reinterpret_cast<uint2 *>(s_buf + swz(t, j >> 3, U) + ((j & 4) << 1)) = o;
                }
                meta_put(m1, nslot);
            }
            __syncthreads();
            // 2. loads of item k+1, metadata of item k+2
            const float sc = s_sc[slot];
            const Col ck = c0;
            if constexpr (kPrefetch) data_load(tl1, c1, nslot);   // the last item has none
            const Meta m2 = meta_load(tl2);
            // 3. D[n][t] for item k over its slot's rank steps, added into the y tile
            {
                floatx16_t acc[NB][2];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[nb][0] = acc[nb][1] = floatx16_t{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if (ks < nks) {
                        const int u = 2 * ks + half;
                        uint4 bfr[2];
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) bfr[tb] = *reinterpret_cast<const uint4 *>(s_buf + swz(32 * tb + l32, u, U));
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const uint4 af = *reinterpret_cast<const uint4 *>(s_b + swz(WC * w + 32 * nb + l32, u, U));
#pragma unroll
                            for (int tb = 0; tb < 2; ++tb)
                                acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(af), as_frag(bfr[tb]), acc[nb][tb], 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const int t = 32 * tb + l32;
                    if (t < ntok) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                uint2 *yp = reinterpret_cast<uint2 *>(&s_y[t * YS + WC * w + 32 * nb + 8 * g + 4 * half]);
                                const uint2 y0 = *yp;
                                uint2 o;
                                o.x = pack_bf16x2(bf16_lo(y0.x) + sc * acc[nb][tb][4 * g + 0], bf16_hi(y0.x) + sc * acc[nb][tb][4 * g + 1]);
                                o.y = pack_bf16x2(bf16_lo(y0.y) + sc * acc[nb][tb][4 * g + 2], bf16_hi(y0.y) + sc * acc[nb][tb][4 * g + 3]);
                                *yp = o;
                            }
                    }
                }
            }
            __syncthreads();
            // 4. item k back to y, row by row.  Every lane stores: rows past the
            // tile's tokens and columns past the slice store the last token row's
            // (or the last column unit's) final value again, the same bytes to the
            // same place, so no store sits under a branch.
            {
                uint16_t *ybase = a.y + a.sl.off[ck.sg];
#pragma unroll
                for (int i = 0; i < NY; ++i) {
                    const int q = i * kThreads + tid;
                    const int row = min(q / YU, ntok - 1);
                    const int cu = min(8 * (q % YU), ck.Ns - 8 - ck.n_base);
                    stg_nt(ybase + s_yrow[slot][row] * a.ldy + ck.n_base + cu,
                           *reinterpret_cast<const uint4 *>(&s_y[row * YS + cu]));
                }
            }
            __syncthreads();
            tl0 = tl1; tl1 = tl2; tl2 = tl3;
            m1 = m2;
            c0 = c1; c1 = col_of(k + 2);
        };
        // the first item is peeled too, so that the loop is entered with the
        // same operations in flight as its back edge carries
        if (cnt > 1) {
            item(0, std::true_type{});
            for (int k = 1; k + 1 < cnt; ++k) item(k, std::true_type{});
        }
        item(cnt - 1, std::false_type{});
    }
}

}  // namespace

hipError_t launch_pre_shrink(const void *x, int64_t ldx, int32_t T, int32_t K, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *slot_rank,
                             const SegPtrs &seg, float *buf, hipStream_t st, const GroupMap &gm,
                             float *part, int32_t *kspl_io) {
    PreShrinkArgs a;
    a.x = static_cast<const uint16_t *>(x); a.ldx = ldx; a.T = T; a.K = K; a.S = S; a.L = L;
    a.R = R; a.slot_rank = slot_rank; a.seg = seg; a.sl = sl; a.buf = buf;
    a.gm = gm;
    if (a.gm.buf_rows == 0) a.gm.buf_rows = T;
    // columns per work-group, in blocks of 32: all of S * R up to 64; past
    // that 128 when the shrink is split over K (many short tiles), else 64
    // (long tiles: twice the work-groups for the CUs, and half the LDS reads
    // per stage of the waves that compute)
    const int sr = S * R;
    const int ncb = sr <= 32 ? 1 : (sr <= 64 || !part) ? 2 : 4;
    a.n_cb = (sr + 32 * ncb - 1) / (32 * ncb);
    // K splits: every split gets at least one stage; the count actually used
    // goes back to the caller (the partials hold that many chunks)
    const int nst = (K + kShStageK - 1) / kShStageK;
    int kspl = part && kspl_io ? (*kspl_io < 1 ? 1 : *kspl_io) : 1;
    if (kspl > nst) kspl = nst;
    a.st_per = (nst + kspl - 1) / kspl;
    a.kspl = (nst + a.st_per - 1) / a.st_per;
    a.part = part;
    if (kspl_io) *kspl_io = a.kspl;
    dim3 grid((unsigned)(kXcds * ((seg.max_tiles_pre + kXcds - 1) / kXcds) * a.n_cb * a.kspl));
    switch (ncb) {
        case 1: hipLaunchKernelGGL(k_pre_shrink_rows<1>, grid, dim3(kShThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_pre_shrink_rows<2>, grid, dim3(kShThreads), 0, st, a); break;
        default: hipLaunchKernelGGL(k_pre_shrink_rows<4>, grid, dim3(kShThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_pre_expand(void *y, int64_t ldy, const float *buf, int32_t T, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *slot_rank,
                             const float *scale, const SegPtrs &seg, hipStream_t st,
                             const GroupMap &gm) {
    PreExpandArgs a;
    a.y = static_cast<uint16_t *>(y); a.ldy = ldy; a.buf = buf; a.T = T; a.S = S; a.L = L;
    a.R = R; a.slot_rank = slot_rank; a.scale = scale; a.seg = seg; a.sl = sl;
    a.gm = gm;
    if (a.gm.buf_rows == 0) a.gm.buf_rows = T;
    if (a.gm.buf_sstride < 0) a.gm.buf_sstride = a.gm.buf_rows;
    bool aligned = R % 16 == 0 && ldy % 8 == 0;
    for (int s = 0; s < S; ++s)
        aligned = aligned && sl.n[s] % 8 == 0 && sl.off[s] % 8 == 0;
    // the persistent kernel: ranks 16, 32, 64, 128 (power-of-two rows), no
    // per-item factor (its load would hang off the token index, inside the
    // item pipeline); the per-launch kernel: ranks up to 64; else the generic one
    const bool pipe = aligned && (R == 16 || R == 32 || R == 64 || R == 128) && !a.gm.coef && !a.gm.ksum &&
                      !a.gm.pair_k;
    const bool rows = aligned && R <= 64;
    const int cols = pipe ? (R <= 64 ? kRowCols : kRowCols / 2) : rows ? kRowCols : kExpGroupCols;
    int c = 0;
    for (int s = 0; s < S; ++s) {
        a.group_start[s] = c;
        c += (int)((sl.n[s] + cols - 1) / cols);
    }
    for (int s = S; s <= kMaxSlices; ++s) a.group_start[s] = c;
    a.n_cg = c;
    a.per_xcd = (c + kXcds - 1) / kXcds;
    const int64_t max_tiles = (int64_t)seg.max_tiles_pre * (gm.pair_k ? gm.pair_k : 1);
    dim3 grid((unsigned)(max_tiles * a.per_xcd * kXcds));
    if (pipe) {
        // 32 CUs per XCD; two work-groups per CU, three at rank 16 (whose
        // 44 KB of LDS leave room for a third: more items in flight to cover
        // the fixed cost of the small ones, e.g. the half-full (slot, expert)
        // tiles of a fused-MoE call)
        const dim3 pgrid(kXcds * (R == 16 ? 96 : 64));
        switch (R / 16) {
            case 1: hipLaunchKernelGGL((k_pre_expand_pipe<1, kRowCols>), pgrid, dim3(kThreads), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_pre_expand_pipe<2, kRowCols>), pgrid, dim3(kThreads), 0, st, a); break;
            case 4: hipLaunchKernelGGL((k_pre_expand_pipe<4, kRowCols>), pgrid, dim3(kThreads), 0, st, a); break;
            default: hipLaunchKernelGGL((k_pre_expand_pipe<8, kRowCols / 2>), pgrid, dim3(kThreads), 0, st, a); break;
        }
        return hipGetLastError();
    }
    if (!rows) {
        hipLaunchKernelGGL(k_pre_expand, grid, dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    switch (R / 16) {
        case 1: hipLaunchKernelGGL(k_pre_expand_rows<1>, grid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_pre_expand_rows<2>, grid, dim3(kThreads), 0, st, a); break;
        case 3: hipLaunchKernelGGL(k_pre_expand_rows<3>, grid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL(k_pre_expand_rows<4>, grid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace aa
