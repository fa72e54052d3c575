// Slot-grouped decode in two launches: a split-K shrink and an expand.
//
// A batch of a few hundred decode tokens moves ~10 MB, so the time goes to
// latency and to how many bytes each work-group must pull through its CU.
// A single kernel that recomputes the shrink next to every output chunk
// makes each work-group read a whole slice of lora_a; here the shrink is
// spread over K instead, and the expand sums the K-chunk partials.
//
// Groups: the slot-major runs of at most 32 tokens that a stable sort of the
// active tokens by slot gives.  While one wave can find them (at most 64
// slots and 1024 tokens) each work-group derives its group from idx itself
// (discover.hpp), so there is no separate segment kernel and the only
// dependent global loads are idx -> {x, lora_a} and idx -> {partials,
// lora_b, y}.  Beyond that the kernels read the same groups from the segment
// table (the decode tiles of the segment build): one tile and its token ids
// per work-group instead of a discovery over the whole batch in each.
//
// Shrink work-group = (group, pack of up to 4 blocks of 16 rank rows drawn
// from the S slices, K chunk of 512).  Each of the 8 waves loads its 64-column
// K slice of the 32 x rows and the pack's lora_a rows line by line (one wave
// instruction = 8 rows x 128 bytes), stages them through its own XOR-swizzled
// LDS area and runs v_mfma_f32_16x16x32_bf16; the 8 waves are summed in LDS
// in a fixed order.  Partials: fp32 [S][kc][pos][R], pos = the token's
// position in slot-sorted order.
//
// Expand work-group = (group, 512 output columns of one slice).  It sums the
// K-chunk partials of its tokens in a fixed order, rounds the buffer to bf16
// and runs v_mfma_f32_16x16x16_bf16 as D[n][t] = B[n][:] . buf[t][:]; the
// deltas go through LDS so that y is read and written along rows, 16 bytes
// per lane: y[t][n] = RNE(y + scale[s] * delta).
#include <type_traits>

#include "discover.hpp"

namespace aa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;   // 8
constexpr int kG = kGrpTokens;             // 32 tokens per group
constexpr int kSub = 64;                   // K columns per wave: one 128-byte line per row
constexpr int kKC = kWaves * kSub;         // 512 K columns per chunk
constexpr int kCols = kGrpCols;            // 512 output columns per expand work-group
constexpr int kColsW = kCols / kWaves;     // 64 per wave = 4 blocks of 16

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t frag8(const uint4 &u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ short4_t frag4(const uint2 &u) { return __builtin_bit_cast(short4_t, u); }

// Byte offset of 16-byte unit u of row r in a staging area of 128-byte rows,
// the unit XOR-swizzled with the row (fragment reads of 8 rows hit 8 bank groups).
__device__ __forceinline__ int stage_off(int r, int u) { return r * 128 + ((u ^ (r & 7)) << 4); }

using Disc = DiscLds<kG, kGrpMaxTokens, kWaves>;
struct NoDisc {};
template <bool TAB>
using DiscT = typename std::conditional<TAB, NoDisc, Disc>::type;

// Decode tiles of the segment build: (slot, begin, end) runs of at most 32
// tokens in slot-sorted order, the groups the discovery would find.
struct GrpTable {
    const int4 *tiles;
    const int32_t *perm;
    const int32_t *header;   // [2]: number of tiles
    int32_t max_tiles;
    int32_t ekey;            // tile key = slot * ekey + expert (1: the key is the slot)
};

// Group `group` of the batch (discover.hpp); *tok receives its token list.
__device__ __forceinline__ GroupSel discover(const int32_t *idx, const int32_t *slot_rank, int T, int L,
                                             int R, Disc &g, int group, const int32_t **tok) {
    *tok = g.tok;
    return find_group(idx, slot_rank, T, L, R, g, [=](int) { return group; });
}

// Group `group` from the segment table (TAB) or from idx.
template <bool TAB, typename D>
__device__ __forceinline__ GroupSel group_of(const GrpTable &tab, const int32_t *idx,
                                             const int32_t *slot_rank, int T, int L, int R, D &g,
                                             int group, const int32_t **tok) {
    if constexpr (TAB) {
        GroupSel sel{-1, 0, 0, 0, 0, 0};
        const int n = tab.header[2];
        const int4 tl = tab.tiles[min(group, tab.max_tiles - 1)];   // read before the test
        if (group >= n) return sel;
        sel.slot = tl.x;
        sel.pos0 = tl.y;
        sel.ntok = tl.z - tl.y;
        sel.n_groups = n;
        sel.rank = min(slot_rank ? slot_rank[tl.x / tab.ekey] : R, R);
        *tok = tab.perm + tl.y;
        return sel;
    } else {
        return discover(idx, slot_rank, T, L, R, g, group, tok);
    }
}

struct GrpShrinkArgs {
    const uint16_t *x;
    int64_t ldx;
    int32_t T, K, S, L, R, n_blocks, n_packs, n_kc;
    const int32_t *idx;
    const int32_t *slot_rank;
    const void *a[kMaxSlices];
    float *part;          // [S][n_kc][T][R]
    int32_t *n_kc_out;    // or null: receives n_kc (read by a separate expand call)
    GrpTable tab;
};

// NRB: blocks of 16 rank rows per work-group (1..4); TAB: groups from the segment table.
template <int NRB, bool TAB>
__global__ __launch_bounds__(kThreads) void k_grp_shrink(GrpShrinkArgs a) {
    constexpr int RR = kG + 16 * NRB;          // staged rows: 32 x rows, then lora_a rows
    constexpr int LPS = RR / 8;                // wave load instructions (8 rows x 128 B each)
    constexpr int kStage = kWaves * RR * 128;
    constexpr int kPart = kWaves * kG * (16 * NRB + 4) * 4;
    constexpr int kUnion = kStage > kPart ? kStage : kPart;
    __shared__ __attribute__((aligned(16))) char s_union[kUnion];
    __shared__ DiscT<TAB> g;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int kc = blockIdx.x % a.n_kc;
    const int pack = (blockIdx.x / a.n_kc) % a.n_packs;
    const int group = blockIdx.x / (a.n_kc * a.n_packs);
    if (blockIdx.x == 0 && tid == 0 && a.n_kc_out) *a.n_kc_out = a.n_kc;
    const int32_t *tokl;
    const GroupSel gs = group_of<TAB>(a.tab, a.idx, a.slot_rank, a.T, a.L, a.R, g, group, &tokl);
    const int s = gs.slot;
    if (s < 0) return;
    const int ntok = gs.ntok, pos0 = gs.pos0;
    const int r = gs.rank;
    const int rb = (a.R + 15) / 16;            // rank blocks per slice

    // The pack's blocks: slice and first rank row; a block past the slices or
    // the slot's rank is loaded from a valid row and never stored.
    int bsl[NRB], bj0[NRB];
    bool bok[NRB];
    bool any = false;
#pragma unroll
    for (int b = 0; b < NRB; ++b) {
        const int gb = pack * NRB + b;
        bsl[b] = gb < a.n_blocks ? gb / rb : 0;
        bj0[b] = gb < a.n_blocks ? (gb % rb) * 16 : 0;
        bok[b] = gb < a.n_blocks && bj0[b] < r;
        any |= bok[b];
    }
    if (!any) return;   // uniform: every block of the pack is past the rank

    // ---- loads: row p of the staging area -------------------------------
    const uint16_t *srcrow[LPS];
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
        const int p = 8 * i + (lane >> 3);
        if (p < kG) {
            srcrow[i] = a.x + (int64_t)tokl[p < ntok ? p : 0] * a.ldx;
        } else {
            const int b = (p - kG) >> 4, jj = (p - kG) & 15;
            const int j = min(bj0[b] + jj, r - 1);
            srcrow[i] = static_cast<const uint16_t *>(a.a[bsl[b]]) + ((int64_t)s * a.R + j) * a.K;
        }
    }
    const int k0 = kc * kKC + w * kSub;
    const bool kv = k0 < a.K;                  // K % 64 == 0: a wave's slice is all in or all out
    const int kk = (kv ? k0 : a.K - kSub) + 8 * (lane & 7);
    uint4 v[LPS];
#pragma unroll
    for (int i = 0; i < LPS; ++i) v[i] = ldg<uint4>(srcrow[i] + kk);
    __builtin_amdgcn_sched_barrier(0);

    char *stage = s_union + w * (RR * 128);
#pragma unroll
    for (int i = 0; i < LPS; ++i)
        *reinterpret_cast<uint4 *>(stage + stage_off(8 * i + (lane >> 3), lane & 7)) = v[i];

    // ---- MFMA 16x16x32: D[t][j] = x[t][:] . A[j][:] over this wave's 64 columns
    const int row = lane & 15, quad = lane >> 4;
    floatx4_t acc[2][NRB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int b = 0; b < NRB; ++b) acc[tb][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        uint4 xf[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            xf[tb] = *reinterpret_cast<const uint4 *>(stage + stage_off(16 * tb + row, 4 * ks + quad));
            if (!kv) xf[tb] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < NRB; ++b) {
            const uint4 af = *reinterpret_cast<const uint4 *>(stage + stage_off(kG + 16 * b + row, 4 * ks + quad));
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag8(xf[tb]), frag8(af), acc[tb][b], 0, 0, 0);
        }
    }
    __syncthreads();   // staging is reused for the per-wave partial sums
    // acc[tb][b][i]: token 16*tb + 4*quad + i, rank row 16*b + row of the pack
    float *s_part = reinterpret_cast<float *>(s_union);   // [wave][token][16*NRB + 4]
    constexpr int PW = 16 * NRB + 4;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int b = 0; b < NRB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_part[(w * kG + 16 * tb + 4 * quad + i) * PW + 16 * b + row] = acc[tb][b][i];
    __syncthreads();
    // Sum the 8 waves in order; one float4 of 4 rank rows per thread.
    for (int o = tid; o < kG * 4 * NRB; o += kThreads) {
        const int t = o / (4 * NRB), q = o - t * (4 * NRB);
        const int b = q >> 2, j4 = 4 * (q & 3);
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float4 p = *reinterpret_cast<const float4 *>(&s_part[(ww * kG + t) * PW + 16 * b + j4]);
            sum.x += p.x; sum.y += p.y; sum.z += p.z; sum.w += p.w;
        }
        bool okb = false;
        int sl = 0, j0 = 0;
#pragma unroll
        for (int bb = 0; bb < NRB; ++bb)
            if (bb == b) { okb = bok[bb]; sl = bsl[bb]; j0 = bj0[bb]; }
        if (okb && t < ntok && j0 + j4 < a.R) {
            float *dst = a.part + (((int64_t)sl * a.n_kc + kc) * a.T + pos0 + t) * a.R + j0 + j4;
            *reinterpret_cast<float4 *>(dst) = sum;
        }
    }
}

struct GrpExpandArgs {
    uint16_t *y;
    int64_t ldy;
    int32_t T, S, L, R, n_chunks, n_kc;
    const int32_t *idx;
    const int32_t *slot_rank;
    const float *scale;
    const float *part;       // [S][n_kc][T][R] rows by slot-sorted position, or
    const float *buf;        // [S][T][R] rows by token (then n_kc = 1)
    const int32_t *n_kc_in;  // or null: chunk count written by the shrink, at most n_kc
    int32_t shared;          // every slice reads slice 0's partials / buffer (one lora_a)
    Slices sl;
    int32_t chunk_start[kMaxSlices + 1];
    GrpTable tab;
};

// RB: R / 16 (1..8).  lora_b rows are staged per wave in passes of 64 ranks
// (128 bytes of each row); ranks past 64 need the buffer form (n_kc == 1).
// TAB: groups from the segment table.
template <int RB, bool TAB>
__global__ __launch_bounds__(kThreads) void k_grp_expand(GrpExpandArgs a) {
    constexpr int R = 16 * RB;
    constexpr int BROW = 2 * R;                       // bytes of one lora_b row
    constexpr int SROW = BROW < 128 ? BROW : 128;     // staged bytes per row and pass
    constexpr int NPASS = (BROW + 127) / 128;
    constexpr int BLD = kColsW * BROW / 1024;         // wave load instructions for its lora_b rows (2 * RB)
    constexpr bool kPow2Row = (RB & (RB - 1)) == 0;
    constexpr int kLgRowUnits = RB == 1 ? 1 : RB == 2 ? 2 : RB == 4 ? 3 : 4;   // log2(2 * RB) when kPow2Row
    constexpr int Q = kG * R / 4;                     // float4 units of one K chunk's partials
    constexpr int H = kThreads / Q > 0 ? kThreads / Q : 1;
    constexpr int NQ = (Q + kThreads - 1) / kThreads; // units per thread
    constexpr int kStage = kWaves * kColsW * SROW;
    constexpr int kDelta = kG * (kCols + 4) * 4;
    constexpr int kUnion = kStage > kDelta ? kStage : kDelta;
    __shared__ __attribute__((aligned(16))) char s_union[kUnion];
    __shared__ __attribute__((aligned(16))) float4 s_red[H][Q];
    __shared__ __attribute__((aligned(16))) uint16_t s_buf[kG][R + 8];
    __shared__ DiscT<TAB> g;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int chunk = blockIdx.x % a.n_chunks;
    const int group = blockIdx.x / a.n_chunks;
    const int n_kc = a.n_kc_in ? max(1, min(*a.n_kc_in, a.n_kc)) : a.n_kc;
    const int32_t *tokl;
    const GroupSel gs = group_of<TAB>(a.tab, a.idx, a.slot_rank, a.T, a.L, R, g, group, &tokl);
    const int s = gs.slot;
    if (s < 0) return;
    const int ntok = gs.ntok, pos0 = gs.pos0;
    const int r = gs.rank;
    int sg = 0;
    while (sg + 1 < a.S && chunk >= a.chunk_start[sg + 1]) ++sg;
    const int Ns = (int)a.sl.n[sg];
    const int n_base = (chunk - a.chunk_start[sg]) * kCols;
    const float sc = a.scale[s];

    // ---- loads, all issued before the first use ---------------------------
    // lora_b rows of this wave's 64 columns: the first U 16-byte units of each
    // row, U = 2 * ceil(r / 16) rounded up to a power of two when the padded
    // row is a power-of-two size, else the whole row.  A slot of rank 8 in a
    // tensor padded to rank 128 reads 32 of its 256 bytes per row.  Load
    // instruction i holds units 64 i .. 64 i + 63 of the wave's row block
    // (row-major); instructions past U repeat the last one.
    const int nks = (r + 15) >> 4;
    const int lgu = kPow2Row ? min(32 - __clz(2 * nks - 1), kLgRowUnits) : 0;
    const int U = kPow2Row ? 1 << lgu : 2 * RB;
    const char *bblk = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.sl.b[sg]) +
                                                      (int64_t)s * Ns * R);
    uint4 bq[BLD];
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
        const int f = 64 * min(i, U - 1) + lane;          // BLD == 2 * RB >= U
        const int rl = kPow2Row ? f >> lgu : f / U, u = kPow2Row ? f & (U - 1) : f % U;
        const int nr = min(n_base + w * kColsW + rl, Ns - 1);
        bq[i] = ldg<uint4>(reinterpret_cast<const uint4 *>(bblk + (int64_t)nr * BROW + 16 * u));
    }
    // y: wave w owns tokens w, w + 8, w + 16, w + 24 of the group, 8 columns per lane.
    const int ycol = min(n_base + 8 * lane, Ns - 8);
    uint4 yv[kG / kWaves];
#pragma unroll
    for (int i = 0; i < kG / kWaves; ++i) {
        const int t = w + kWaves * i;
        yv[i] = ldg<uint4>(a.y + (int64_t)tokl[t < ntok ? t : 0] * a.ldy + a.sl.off[sg] + ycol);
    }
    // partials (or buffer rows) of the group's tokens: thread = (float4 units
    // q = tid % Q + kThreads * v, K-chunk phase h)
    const int h = tid / Q;
    constexpr int NPL = RB > 4 ? 1 : (kMaxKcGrp + H - 1) / H;   // K-chunk loads per unit, upper bound
    float4 pv[NQ][NPL];
#pragma unroll
    for (int v = 0; v < NQ; ++v) {
        const int q = min(tid % Q + kThreads * v, Q - 1);
        const int pt = min(q / (R / 4), ntok - 1);
        const int sp = a.shared ? 0 : sg;
        const float *pbase = a.buf ? a.buf + ((int64_t)sp * a.T + tokl[pt]) * R + 4 * (q % (R / 4))
                                   : a.part + ((int64_t)sp * n_kc * a.T + pos0 + pt) * R + 4 * (q % (R / 4));
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int kcl = min(h + H * i, n_kc - 1);
            pv[v][i] = ldg<float4>(pbase + (int64_t)kcl * a.T * R);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- buffer: sum the K chunks in order, round to bf16 ------------------
    if (h < H) {
#pragma unroll
        for (int v = 0; v < NQ; ++v) {
            const int q = tid % Q + kThreads * v;
            if (q < Q) {
                float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int i = 0; i < NPL; ++i)
                    if (h + H * i < n_kc) { sum.x += pv[v][i].x; sum.y += pv[v][i].y; sum.z += pv[v][i].z; sum.w += pv[v][i].w; }
                s_red[h][q] = sum;
            }
        }
    }
    __syncthreads();
    for (int u = tid; u < Q; u += kThreads) {
        float4 sum = s_red[0][u];
#pragma unroll
        for (int hh = 1; hh < H; ++hh) {
            const float4 p = s_red[hh][u];
            sum.x += p.x; sum.y += p.y; sum.z += p.z; sum.w += p.w;
        }
        const int t = u / (R / 4), j = 4 * (u % (R / 4));
        const bool ok = t < ntok;
        uint2 o;
        o.x = pack_bf16x2(ok && j < r ? sum.x : 0.f, ok && j + 1 < r ? sum.y : 0.f);
        o.y = pack_bf16x2(ok && j + 2 < r ? sum.z : 0.f, ok && j + 3 < r ? sum.w : 0.f);
        *reinterpret_cast<uint2 *>(&s_buf[t][j]) = o;
    }
    __syncthreads();

    // ---- expand (MFMA 16x16x16): D[n][t] = B[n][:] . buf[t][:] ------------
    // The wave's lora_b rows pass through its own staging area 64 ranks at a
    // time; rank steps past the slot's rank are skipped.
    const int row = lane & 15, quad = lane >> 4;
    char *stage = s_union + w * (kColsW * SROW);
    floatx4_t out[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) out[nb][tb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int f = 64 * i + lane;
            const int rl = kPow2Row ? f >> lgu : f / U, u = kPow2Row ? f & (U - 1) : f % U;
            const int off = 16 * u - ps * 128;
            if (i < U && off >= 0 && off < SROW)
                *reinterpret_cast<uint4 *>(stage + rl * SROW + off) = bq[i];
        }
#pragma unroll
        for (int kq = 0; kq < SROW / 32; ++kq) {
            const int ks = ps * 4 + kq;
            if (ks < nks) {
                uint2 bfr[2];
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) bfr[tb] = *reinterpret_cast<const uint2 *>(&s_buf[16 * tb + row][16 * ks + 4 * quad]);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const uint2 af = *reinterpret_cast<const uint2 *>(stage + (16 * nb + row) * SROW + 32 * kq + 8 * quad);
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
                        out[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(af), frag4(bfr[tb]), out[nb][tb], 0, 0, 0);
                }
            }
        }
    }
    __syncthreads();   // every wave is done with its staging area (the deltas alias it)
    // lane: token 16*tb + row, columns 64w + 16nb + 4*quad .. +3 of the chunk
    float *s_delta = reinterpret_cast<float *>(s_union);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            *reinterpret_cast<float4 *>(s_delta + (16 * tb + row) * (kCols + 4) + w * kColsW + 16 * nb + 4 * quad) =
                make_float4(sc * out[nb][tb][0], sc * out[nb][tb][1], sc * out[nb][tb][2], sc * out[nb][tb][3]);
    __syncthreads();
    const int cl = 8 * lane;
    if (n_base + cl < Ns) {
#pragma unroll
        for (int i = 0; i < kG / kWaves; ++i) {
            const int t = w + kWaves * i;
            if (t < ntok) {
                const float4 d0 = *reinterpret_cast<const float4 *>(s_delta + t * (kCols + 4) + cl);
                const float4 d1 = *reinterpret_cast<const float4 *>(s_delta + t * (kCols + 4) + cl + 4);
                const uint4 y0 = yv[i];
                uint4 o;
                o.x = pack_bf16x2(bf16_lo(y0.x) + d0.x, bf16_hi(y0.x) + d0.y);
                o.y = pack_bf16x2(bf16_lo(y0.y) + d0.z, bf16_hi(y0.y) + d0.w);
                o.z = pack_bf16x2(bf16_lo(y0.z) + d1.x, bf16_hi(y0.z) + d1.y);
                o.w = pack_bf16x2(bf16_lo(y0.w) + d1.z, bf16_hi(y0.w) + d1.w);
                *reinterpret_cast<uint4 *>(a.y + (int64_t)tokl[t] * a.ldy + a.sl.off[sg] + n_base + cl) = o;
            }
        }
    }
}

struct GrpReduceArgs {
    int32_t T, S, L, R, n_kc;
    const int32_t *idx;
    const int32_t *slot_rank;
    const float *part;   // [S][n_kc][T][R]
    float *buf;          // [S][T][R]
    GrpTable tab;
};

// buf[s][t][j] = sum over K chunks (in order) of the group's partials; ranks
// j >= r are written as 0.  Rows of tokens without an adapter are not touched.
template <bool TAB>
__global__ __launch_bounds__(kThreads) void k_grp_reduce(GrpReduceArgs a) {
    __shared__ DiscT<TAB> g;
    const int group = blockIdx.x;
    const int32_t *tokl;
    const GroupSel gs = group_of<TAB>(a.tab, a.idx, a.slot_rank, a.T, a.L, a.R, g, group, &tokl);
    const int s = gs.slot;
    if (s < 0) return;
    const int ntok = gs.ntok, pos0 = gs.pos0, r = gs.rank;
    const int R4 = a.R / 4;
    for (int o = threadIdx.x; o < a.S * ntok * R4; o += kThreads) {
        const int sg = o / (ntok * R4), rem = o - sg * ntok * R4;
        const int t = rem / R4, j = 4 * (rem - t * R4);
        const float *p = a.part + ((int64_t)sg * a.n_kc * a.T + pos0 + t) * a.R + j;
        // every chunk's load in flight at once (n_kc <= kMaxKcGrp), summed in order
        float4 v[kMaxKcGrp];
#pragma unroll
        for (int kc = 0; kc < kMaxKcGrp; ++kc) v[kc] = ldg<float4>(p + (int64_t)min(kc, a.n_kc - 1) * a.T * a.R);
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int kc = 0; kc < kMaxKcGrp; ++kc)
            if (kc < a.n_kc) { sum.x += v[kc].x; sum.y += v[kc].y; sum.z += v[kc].z; sum.w += v[kc].w; }
        sum.x = j < r ? sum.x : 0.f;
        sum.y = j + 1 < r ? sum.y : 0.f;
        sum.z = j + 2 < r ? sum.z : 0.f;
        sum.w = j + 3 < r ? sum.w : 0.f;
        *reinterpret_cast<float4 *>(a.buf + ((int64_t)sg * a.T + tokl[t]) * a.R + j) = sum;
    }
}

GrpTable grp_table(const SegPtrs *seg, int32_t ekey = 1) {
    GrpTable t{};
    t.ekey = ekey;
    if (seg) {
        t.tiles = seg->tiles_dec;
        t.perm = seg->perm;
        t.header = seg->header;
        t.max_tiles = seg->max_tiles_dec;
    }
    return t;
}

// Work-groups per token group dimension: every possible group.
int32_t grp_groups(int32_t T, int32_t L, const SegPtrs *seg) {
    return seg ? seg->max_tiles_dec : grp_max_groups(T, L);
}

}  // namespace

int32_t grp_max_groups(int32_t T, int32_t L) {
    return (T + kGrpTokens - 1) / kGrpTokens + (T < L ? T : L);
}

int32_t grp_kchunks(int32_t K) { return (K + kKC - 1) / kKC; }

hipError_t launch_grp_shrink(const void *x, int64_t ldx, int32_t T, int32_t K, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, float *part, int32_t *n_kc_out,
                             const SegPtrs *seg, hipStream_t st) {
    GrpShrinkArgs a;
    a.tab = grp_table(seg);
    a.x = static_cast<const uint16_t *>(x); a.ldx = ldx;
    a.T = T; a.K = K; a.S = S; a.L = L; a.R = R;
    a.idx = idx; a.slot_rank = slot_rank; a.part = part; a.n_kc_out = n_kc_out;
    for (int s = 0; s < kMaxSlices; ++s) a.a[s] = s < S ? sl.a[s] : nullptr;
    a.n_blocks = S * ((R + 15) / 16);
    const int nrb = a.n_blocks < 4 ? a.n_blocks : 4;
    a.n_packs = (a.n_blocks + nrb - 1) / nrb;
    a.n_kc = grp_kchunks(K);
    dim3 grid((unsigned)(grp_groups(T, L, seg) * a.n_packs * a.n_kc));
    if (seg) {
        switch (nrb) {
            case 1: hipLaunchKernelGGL((k_grp_shrink<1, true>), grid, dim3(kThreads), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_grp_shrink<2, true>), grid, dim3(kThreads), 0, st, a); break;
            case 3: hipLaunchKernelGGL((k_grp_shrink<3, true>), grid, dim3(kThreads), 0, st, a); break;
            default: hipLaunchKernelGGL((k_grp_shrink<4, true>), grid, dim3(kThreads), 0, st, a); break;
        }
    } else {
        switch (nrb) {
            case 1: hipLaunchKernelGGL((k_grp_shrink<1, false>), grid, dim3(kThreads), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_grp_shrink<2, false>), grid, dim3(kThreads), 0, st, a); break;
            case 3: hipLaunchKernelGGL((k_grp_shrink<3, false>), grid, dim3(kThreads), 0, st, a); break;
            default: hipLaunchKernelGGL((k_grp_shrink<4, false>), grid, dim3(kThreads), 0, st, a); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_grp_expand(void *y, int64_t ldy, int32_t T, int32_t n_kc, const Slices &sl,
                             int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, const float *scale, const float *part,
                             const float *buf, const int32_t *n_kc_in, const SegPtrs *seg,
                             hipStream_t st, bool shared_a) {
    GrpExpandArgs a;
    a.shared = shared_a ? 1 : 0;
    a.tab = grp_table(seg);
    a.y = static_cast<uint16_t *>(y); a.ldy = ldy;
    a.T = T; a.S = S; a.L = L; a.R = R;
    a.idx = idx; a.slot_rank = slot_rank; a.scale = scale; a.part = part; a.buf = buf;
    a.n_kc_in = buf ? nullptr : n_kc_in; a.sl = sl;
    a.n_kc = buf ? 1 : n_kc;
    int c = 0;
    for (int s = 0; s < S; ++s) {
        a.chunk_start[s] = c;
        c += (int)((sl.n[s] + kCols - 1) / kCols);
    }
    for (int s = S; s <= kMaxSlices; ++s) a.chunk_start[s] = c;
    a.n_chunks = c;
    dim3 grid((unsigned)(grp_groups(T, L, seg) * c));
#define AA_GRP_EXPAND(RB_)                                                             \
    if (seg) hipLaunchKernelGGL((k_grp_expand<RB_, true>), grid, dim3(kThreads), 0, st, a); \
    else hipLaunchKernelGGL((k_grp_expand<RB_, false>), grid, dim3(kThreads), 0, st, a)
    switch (R / 16) {
        case 1: AA_GRP_EXPAND(1); break;
        case 2: AA_GRP_EXPAND(2); break;
        case 3: AA_GRP_EXPAND(3); break;
        case 4: AA_GRP_EXPAND(4); break;
        case 5: AA_GRP_EXPAND(5); break;
        case 6: AA_GRP_EXPAND(6); break;
        case 7: AA_GRP_EXPAND(7); break;
        default: AA_GRP_EXPAND(8); break;
    }
#undef AA_GRP_EXPAND
    return hipGetLastError();
}

hipError_t launch_grp_reduce(int32_t T, int32_t S, int32_t L, int32_t R, const int32_t *idx,
                             const int32_t *slot_rank, const float *part, int32_t n_kc,
                             float *buf, const SegPtrs *seg, hipStream_t st, int32_t ekey) {
    GrpReduceArgs a;
    a.tab = grp_table(seg, ekey);
    a.T = T; a.S = S; a.L = L; a.R = R; a.n_kc = n_kc;
    a.idx = idx; a.slot_rank = slot_rank; a.part = part; a.buf = buf;
    const dim3 grid((unsigned)grp_groups(T, L, seg));
    if (seg) hipLaunchKernelGGL(k_grp_reduce<true>, grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(k_grp_reduce<false>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace aa
