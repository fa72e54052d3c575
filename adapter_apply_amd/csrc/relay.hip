// Single-launch decode with the shrink split over K: shrink work-groups hand
// their fp32 partial sums to expand work-groups inside the same kernel.
//
// The single-launch kernel of fused.hip recomputes a group's shrink in every
// 1024-column chunk, so each of its work-groups streams the group's x rows and
// the slot's lora_a slice (192 KB at K = 4096) through one CU.  Here the shrink
// of a (group, slice) is done once, split over K chunks of 256 columns; every
// expand work-group of that (group, slice) adds the chunks' partials.
//
// Roles.  The grid has two parts, the groups a batch usually fills and then
// the rest (a group's count is known only after the discovery), each part its
// shrink blocks first, then its expand blocks; so idle work-groups of the
// second part do not hold slots ahead of working ones.  Work-groups are
// dispatched in block order (observed on gfx950: the XCC_ID register reads back
// block % 8 for every block, in order; the programming model does not promise
// it), so when an expand work-group starts waiting, every shrink work-group of
// its group has already been dispatched; shrink work-groups wait for nothing,
// so every wait ends.  The waits are bounded all the same: past kSpin polls the work-group
// sets the error word of the workspace and goes on (nothing hangs; that call's
// results are not valid, and late partials may be left in the region).
// lora_workspace_check reports the error and zero-fills the workspace.
//
// Hand-over.  A partial is stored as its fp32 bit pattern XOR kReady, a quiet
// NaN whose payload has non-zero low bits: no sum of bf16 products yields it
// (bf16 NaNs and the default NaN have zero low bits), so a stored word is never
// zero and zero means "not written yet".  Words cross work-groups only through
// agent-scope relaxed atomic stores and loads (on gfx950: global stores and
// loads with the sc1 bit), so no L2 write-back or invalidate is needed and no
// counter stands between the data and its reader: an expand work-group loads
// all its words and repeats while any is still zero.  The last expand
// work-group to read a block of tokens (a counter per block, each on its own
// 256-byte line:
// counters sharing a line serialise every poll and add of the batch on one
// memory channel) writes the block back to zero, so the workspace is left as
// it was found.
//
// Work items.
//   shrink (g, kc, s): group g of at most 32 tokens of one slot (slot-major
//     runs of a stable sort by slot), K columns [256 kc, 256 kc + 256), slice
//     s.  4 waves, 64 K columns each: the wave loads its x rows and the slot's
//     lora_a rows line by line (8 rows x 128 B per instruction), stages them
//     in swizzled LDS and runs v_mfma_f32_16x16x32_bf16 (two 16-token tiles);
//     the 4 waves are summed in order.  Output: fp32 [S][n_kc][T][R] by
//     slot-sorted token position.  When every slice passes the same lora_a
//     ([vLLM] MergedQKVParallelLinearWithLoRA copies one checkpoint lora_a
//     into every slice) only slice 0's shrink items run, and the expand items
//     of every slice add slice 0's partials.
//   expand (g, item, b): tokens 8b .. 8b + 7 of group g (16b .. 16b + 15 for
//     outputs wider than 16384 columns), CPI consecutive 512-column chunks
//     of one slice (one chunk; up to four on wide outputs, as many as keep
//     about four expand work-groups per CU).  The first chunk's lora_b rows,
//     read straight into MFMA fragments, and its y rows are loaded before the
//     wait; after it the K-chunk partials are summed in a fixed order into a
//     bf16 buffer, and v_mfma_f32_16x16x16_bf16 (16x16x32 at rank 32) forms
//     D[n][t] = B[n][:] . buf[t][:] chunk by chunk, the next chunk's loads in
//     flight meanwhile; y is read and written 16 bytes per lane along rows
//     (non-temporal).
// XCD placement (block i runs on XCD i % 8): the slices of a (g, kc) share
// one XCD (its x rows are read once from HBM), and the token blocks of a
// (g, item) share one XCD (its lora_b rows are read once).
#include "discover.hpp"

namespace aa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;     // 4
constexpr int kG = kRelayGroup;              // tokens per group (32)
constexpr int kMaxSubs = kG / 8;             // expand work-groups per (group, item), at most
constexpr int kKc = kRelayKc;                // K columns per shrink item (256)
constexpr int kCols = kRelayCols;            // output columns per expand item (512)
constexpr int kColsW = kCols / kWaves;       // 128 per wave
constexpr int kSpin = 1 << 20;
constexpr uint32_t kReady = 0x7fc0deadu;   // stored word = fp32 bits ^ kReady (never 0)
constexpr int kLine = 64;                  // int32 per counter: one 256-byte line each
constexpr int kRelayMaxCpi = 4;            // 512-column chunks per expand item, at most (1, 2 or 4)
constexpr int kRelayMinItems = 1024;       // expand work-groups to keep (four per CU)

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

struct RelayArgs {
    const uint16_t *x;
    int64_t ldx;
    uint16_t *y;
    int64_t ldy;
    int32_t T, K, S, L, R;
    int32_t n_kc;        // K / kKc
    int32_t n_items;     // expand items per (group, token block) over all slices
    int32_t max_groups;
    int32_t n_first;     // groups in the first part of the grid
    int32_t pstart[4];   // first block of: part 1 expand, part 2 shrink, part 2 expand, the end
    int32_t S_shrink;    // slices with a shrink of their own: S, or 1 when every slice
                         // shares one lora_a (the expands of all slices read slice 0's)
    const int32_t *idx;
    const int32_t *slot_rank;
    const float *scale;
    Slices sl;
    int32_t chunk_start[kMaxSlices + 1];   // first 512-column chunk of each slice
    int32_t item_start[kMaxSlices + 1];    // first expand item of each slice
    float *part;         // fp32 [S][n_kc][T][R]
    int32_t *sync;       // per (group, slice, token block) reader count, kLine int32 apart
    int32_t *err;        // error word: set when a wait gives up
    int32_t give_up;     // test hook: every wait gives up after its first poll
};

struct RelayDisc {
    int32_t cnt[kWave];
    int32_t tok[kG];
    int32_t info[6];
};

// The work item's slice parameters (kernel arguments indexed at run time),
// resolved by an otherwise idle wave during the group discovery.
struct RelaySlice {
    const uint16_t *a;
    const uint16_t *b;
    int64_t n, off;
    int32_t sg, c0, c1, i0, i1;
};

__device__ __forceinline__ bf16x8_t frag8(const uint4 &u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ short4_t frag4(const uint2 &u) { return __builtin_bit_cast(short4_t, u); }

// D += A . B over one 16-rank block (4 ranks per lane) or two (8 per lane)
__device__ __forceinline__ floatx4_t mfma_rank(const uint2 &a, const uint2 &b, floatx4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(a), frag4(b), acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma_rank(const uint4 &a, const uint4 &b, floatx4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag8(a), frag8(b), acc, 0, 0, 0);
}

// Byte offset of 16-byte unit u of row r in a staging area of 128-byte rows,
// the unit XOR-swizzled with the row (fragment reads of 8 rows hit 8 bank groups).
__device__ __forceinline__ int stage_off(int r, int u) { return r * 128 + ((u ^ (r & 7)) << 4); }

// A pointer that every lane of the wave holds, moved into scalar registers.
template <typename P>
__device__ __forceinline__ P *uniform_ptr(P *p) {
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<P *>(((uint64_t)hi << 32) | lo);
}

// A load through a pointer read from LDS: the compiler cannot see that it is
// a global address and would emit a flat load, which also counts against
// lgkmcnt (every later LDS or scalar wait would then wait for it).
__device__ __forceinline__ uint4 ldg_as1(const void *p) {
    const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t *>(
        reinterpret_cast<uintptr_t>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void ldg_as1(const void *p, uint2 &out) {
    const u32x2_t v = *reinterpret_cast<const __attribute__((address_space(1))) u32x2_t *>(
        reinterpret_cast<uintptr_t>(p));
    out = make_uint2(v.x, v.y);
}
__device__ __forceinline__ void ldg_as1(const void *p, uint4 &out) { out = ldg_as1(p); }

__device__ __forceinline__ void st_coherent(float *p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t encode2(float a, float b) {
    return (uint64_t)(__float_as_uint(a) ^ kReady) | ((uint64_t)(__float_as_uint(b) ^ kReady) << 32);
}
__device__ __forceinline__ uint64_t ld_coherent(const float *p) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

template <int NRB, int kSubTok>
struct RelaySmem {
    static constexpr int RP = 16 * NRB;                        // padded rank
    static constexpr int RR = kG + RP;                         // staged rows per wave: x then lora_a
    static constexpr int kStage = kWaves * RR * 128;
    static constexpr int kPart = kWaves * kG * (RP + 4) * 4;   // aliases the staging
    static constexpr int kProd = kStage > kPart ? kStage : kPart;
    static constexpr int kDelta = kSubTok * (kCols + 4) * 4;   // expand: fp32 deltas
    static constexpr int kUnion = kProd > kDelta ? kProd : kDelta;
    static constexpr int PP = kSubTok * RP / 2;                // partial pairs per K chunk
    static_assert(PP % kWave == 0 && PP <= kThreads, "pairs of a block fill whole waves");
};

// NRB: 16-rank blocks of R (1 or 2); MKC: bound on the K chunks (16 or 32);
// SUB: tokens per expand item (8, or 16 for wide outputs, where fewer expand
// work-groups re-read each lora_b block); CPI: 512-column chunks per expand
// item (several for wide outputs, so that the group discovery and the wait
// for the partials are paid once for them).  At rank 16 and K <= 4096 an
// occupancy bound keeps four work-groups per CU without spills.
template <int NRB, int MKC, int SUB, int CPI>
__global__ __launch_bounds__(kThreads, (NRB == 1 && MKC == 16) ? 4 : 1) void k_dec_relay(RelayArgs a) {
    constexpr int kSubTok = SUB;
    constexpr int kSubs = kG / SUB;
    using SM = RelaySmem<NRB, SUB>;
    constexpr int RP = SM::RP, RR = SM::RR;
    constexpr int LPS = RR / 8;                    // load instructions per wave (8 rows x 128 B)
    constexpr int BROW = RP * 2;                   // bytes of one lora_b row
    constexpr int kNB = kColsW / 16;               // 16-column MFMA blocks per wave
    using BFrag = typename std::conditional<NRB == 1, uint2, uint4>::type;   // a lane's ranks of one row
    constexpr int PP = SM::PP;
    constexpr int TW = kSubTok / kWaves;             // y rows per wave

    __shared__ __attribute__((aligned(16))) char s_union[SM::kUnion];
    __shared__ __attribute__((aligned(16))) uint16_t s_buf[16][RP + 8];   // MFMA tile: 16 tokens
    __shared__ RelayDisc d;
    __shared__ int s_last[1];
    __shared__ float s_scale[kWave];
    __shared__ RelaySlice s_sl;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = lane & 15, quad = lane >> 4;
    // Two parts, each its shrink items then its expand items: the groups a
    // batch usually fills, then the rest (known only after the discovery),
    // so that idle work-groups do not hold slots ahead of working ones.
    const int b = blockIdx.x;
    const bool second = b >= a.pstart[1];
    const int g0 = second ? a.n_first : 0, gn = second ? a.max_groups : a.n_first;
    const bool shrink = b < a.pstart[0] || (second && b < a.pstart[2]);
    const int rel = b - (shrink ? (second ? a.pstart[1] : 0) : (second ? a.pstart[2] : a.pstart[0]));
    const int xcd = rel % 8, j = rel / 8;
    int g, kc = 0, item = 0, sub = 0;
    if (shrink) {
        const int u = (j / a.S_shrink) * 8 + xcd;
        g = g0 + u / a.n_kc;
        kc = u % a.n_kc;
    } else {
        const int v = (j / kSubs) * 8 + xcd;
        sub = j % kSubs;
        g = g0 + v / a.n_items;
        item = v % a.n_items;
    }
    if (g >= gn) g = -1;
    {
        const auto pick = [=](int n) { return g < n ? g : -1; };
        // wave 1 fetches the slot scales (L <= 64) and the item's slice
        // parameters while wave 0 finds the group
        if (w == 1) {
            s_scale[lane] = a.scale[min(lane, a.L - 1)];
            if (lane == 0) {
                int sg = 0;
                if (shrink) sg = j % a.S_shrink;
                else
                    while (sg + 1 < a.S && item >= a.item_start[sg + 1]) ++sg;
                s_sl.sg = sg;
                s_sl.a = static_cast<const uint16_t *>(a.sl.a[sg]);
                s_sl.b = static_cast<const uint16_t *>(a.sl.b[sg]);
                s_sl.n = a.sl.n[sg];
                s_sl.off = a.sl.off[sg];
                s_sl.c0 = a.chunk_start[sg];
                s_sl.c1 = a.chunk_start[sg + 1];
                s_sl.i0 = a.item_start[sg];
                s_sl.i1 = a.item_start[sg + 1];
            }
        }
        if (w == 0) {
            if (a.T <= 4 * kWave) one_wave_group<kG, 4>(a.idx, a.slot_rank, a.T, a.L, a.R, d, pick);
            else if (a.T <= 8 * kWave) one_wave_group<kG, 8>(a.idx, a.slot_rank, a.T, a.L, a.R, d, pick);
            else one_wave_group<kG, kOneWaveChunks>(a.idx, a.slot_rank, a.T, a.L, a.R, d, pick);
        }
        // every wave has the plain arguments in registers before the barrier
        // (their loads would otherwise sink past it, into the critical chain)
        asm volatile("" ::"s"(a.x), "s"(a.y), "s"(a.ldx), "s"(a.ldy), "s"(a.part), "s"(a.sync));
        asm volatile("" ::"s"(a.T), "s"(a.K), "s"(a.S), "s"(a.R), "s"(a.n_kc), "s"(a.max_groups));
        __syncthreads();
    }
    const int s = d.info[0];
    if (s < 0) return;
    const int ntok = d.info[2], pos0 = d.info[3], r = d.info[5];
    const int sg = s_sl.sg;

    if (shrink) {
        // ---- shrink item (g, kc, sg) ----------------------------------------
        char *stage = s_union + w * (RR * 128);
        const uint16_t *abase = uniform_ptr(s_sl.a) + (int64_t)s * a.R * a.K;
        const int k0 = kc * kKc + w * 64 + 8 * (lane & 7);
        uint4 v[LPS];
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            // staged row p: x row of token p (p < 32) or lora_a rank row p - 32;
            // rows past the group or the rank re-read valid rows, dropped below
            const int p = 8 * i + (lane >> 3);
            const uint16_t *src = p < kG ? a.x + (int64_t)d.tok[p < ntok ? p : 0] * a.ldx
                                         : abase + (int64_t)min(p - kG, r - 1) * a.K;
            v[i] = ldg_as1(src + k0);
        }
#pragma unroll
        for (int i = 0; i < LPS; ++i)
            *reinterpret_cast<uint4 *>(stage + stage_off(8 * i + (lane >> 3), lane & 7)) = v[i];
        floatx4_t acc[2][NRB];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int b = 0; b < NRB; ++b) acc[t][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint4 xf = *reinterpret_cast<const uint4 *>(stage + stage_off(16 * t + row, 4 * ks + quad));
#pragma unroll
                for (int b = 0; b < NRB; ++b) {
                    const uint4 af = *reinterpret_cast<const uint4 *>(stage + stage_off(kG + 16 * b + row, 4 * ks + quad));
                    acc[t][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag8(xf), frag8(af), acc[t][b], 0, 0, 0);
                }
            }
        __syncthreads();   // every wave is done with the staging (the partials alias it)
        // acc[t][b][i]: token 16t + 4 quad + i, rank 16b + row
        float *s_part = reinterpret_cast<float *>(s_union);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int b = 0; b < NRB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_part[(w * kG + 16 * t + 4 * quad + i) * (RP + 4) + 16 * b + row] = acc[t][b][i];
        __syncthreads();
        // the 4 waves' K slices summed in order; ranks past r written as zero
        float *dst = a.part + ((int64_t)(sg * a.n_kc + kc) * a.T + pos0) * RP;
#pragma unroll
        for (int q = 0; q < kG * RP / 2 / kThreads; ++q) {
            const int e = tid + kThreads * q;
            const int tk = e / (RP / 2), jp = 2 * (e % (RP / 2));
            float v0 = 0.f, v1 = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                v0 += s_part[(ww * kG + tk) * (RP + 4) + jp];
                v1 += s_part[(ww * kG + tk) * (RP + 4) + jp + 1];
            }
            if (jp >= r) v0 = 0.f;
            if (jp + 1 >= r) v1 = 0.f;
            if (tk < ntok) st_coherent(dst + tk * RP + jp, encode2(v0, v1));
        }
        return;
    }

    // ---- expand item (g, item, sub) -----------------------------------------
    const int t0 = sub * kSubTok;
    if (t0 >= ntok) return;
    const int ct = min(kSubTok, ntok - t0);
    const int Ns = (int)s_sl.n;
    // the item's chunks: cfirst .. cfirst + nc - 1 of its slice
    const int cfirst = s_sl.c0 + (item - s_sl.i0) * CPI;
    const int nc = min(CPI, s_sl.c1 - cfirst);
    const int n_base = (cfirst - s_sl.c0) * kCols;
    // readers of a block of partials: one per item of the slice, or of every
    // slice when they share the shrink
    const int n_readers = a.S_shrink == 1 && a.S > 1 ? a.n_items : s_sl.i1 - s_sl.i0;
    const int sp = a.S_shrink == 1 ? 0 : sg;   // the slice whose partials this item adds
    const float sc = s_scale[s];

    // lora_b in MFMA fragment order, straight from memory: for column block
    // nb the lane reads row 16 nb + row of the wave's 128 columns, ranks
    // 4 quad .. 4 quad + 3 (8 bytes; at rank 32, 8 quad .. 8 quad + 7), so one
    // wave instruction reads 16 whole rows.  The buffer fragment below takes
    // the same ranks of its token.
    const char *bblk = reinterpret_cast<const char *>(uniform_ptr(s_sl.b) + (int64_t)s * Ns * a.R);
    const auto load_b = [&](BFrag(&bq)[kNB], int nb0) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const int nr = min(nb0 + w * kColsW + 16 * nb + row, Ns - 1);
            ldg_as1(bblk + (int64_t)nr * BROW + (int)sizeof(BFrag) * quad, bq[nb]);
        }
    };
    // y rows of tokens TW w .. TW w + TW - 1, 8 columns per lane
    uint16_t *yrow[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int tk = TW * w + i;
        yrow[i] = a.y + (int64_t)d.tok[t0 + (tk < ct ? tk : 0)] * a.ldy + s_sl.off;
    }
    const auto load_y = [&](uint4(&yv)[TW], int nb0) {
#pragma unroll
        for (int i = 0; i < TW; ++i) yv[i] = ldg_nt(yrow[i] + min(nb0 + 8 * lane, Ns - 8));
    };
    // the first chunk's loads do not depend on the shrink: issued before the wait
    BFrag bq[CPI][kNB];
    uint4 yv[CPI][TW];
    load_b(bq[0], n_base);
    load_y(yv[0], n_base);

    int32_t *readers = a.sync + kLine * ((g * a.S + sp) * kSubs + sub);
    const float *blk = a.part + ((int64_t)sp * a.n_kc * a.T + pos0 + t0) * RP;   // chunk k: + k * T * RP

    // The buffer's padding token rows are zeroed before the wait, so that
    // after it only the buffer itself stands between the partials and the MFMA.
    for (int i = tid; i < (16 - kSubTok) * RP; i += kThreads)
        s_buf[kSubTok + i / RP][i % RP] = 0;

    // K-chunk partials of the block's tokens: the first PP threads (whole
    // waves) each own one pair of rank entries of one token and add its
    // n_kc chunks in order.  The loads are the wait: a wave repeats them while
    // any of its words is still unwritten; the other waves go on to the
    // barrier.  (By the time the expand-side loads above have landed, the
    // shrink items have mostly stored, so one round trip usually suffices.)
    if (tid < PP) {
        const int tk = tid / (RP / 2), jp = 2 * (tid % (RP / 2));
        const float *src = blk + (tk < ct ? tk : 0) * RP + jp;
        uint64_t pv[MKC];
        for (int n = 0;; ++n) {
            bool ok = true;
#pragma unroll
            for (int c = 0; c < MKC; ++c)
                pv[c] = ld_coherent(src + (int64_t)min(c, a.n_kc - 1) * a.T * RP);
#pragma unroll
            for (int c = 0; c < MKC; ++c)
                ok = ok && (uint32_t)pv[c] != 0u && (uint32_t)(pv[c] >> 32) != 0u;
            if (__all(ok) && !a.give_up) break;
            if (n >= (a.give_up ? 0 : kSpin)) {
                if (lane == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int c = 0; c < MKC; ++c)
            if (c < a.n_kc) {
                v0 += __uint_as_float((uint32_t)pv[c] ^ kReady);
                v1 += __uint_as_float((uint32_t)(pv[c] >> 32) ^ kReady);
            }
        if (jp >= r || tk >= ct) v0 = 0.f;
        if (jp + 1 >= r || tk >= ct) v1 = 0.f;
        *reinterpret_cast<uint32_t *>(&s_buf[tk][jp]) = pack_bf16x2(v0, v1);
    }
    // The block is read: count it, one count per work-group (a block has as
    // many readers as its slice has column chunks, all adding to one counter).
    // With one polling wave it counts right after its poll, so the round trip
    // overlaps the barrier and the expand; with several, after the barrier
    // that follows all their reads.  The work-group that makes the last count
    // clears the block.
    int nread = -1;
    if (PP == kWave && tid == 0)
        nread = __hip_atomic_fetch_add(readers, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();   // the buffer is complete
    if (PP > kWave && tid == 0)
        nread = __hip_atomic_fetch_add(readers, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // D[n][t] = B[n][:] . buf[t][:] per chunk (MFMA; tokens past the block are
    // zero).  Chunk c + 1's lora_b and y rows are loaded while chunk c is
    // multiplied and written; items with fewer than CPI chunks repeat their
    // last chunk's loads and skip its stores.
    const BFrag bfr = *reinterpret_cast<const BFrag *>(&s_buf[row][(int)sizeof(BFrag) / 2 * quad]);
    float *s_delta = reinterpret_cast<float *>(s_union);
#pragma unroll
    for (int c = 0; c < CPI; ++c) {
        const int nb0 = n_base + min(c, nc - 1) * kCols;
        floatx4_t out[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) out[nb] = mfma_rank(bq[c][nb], bfr, floatx4_t{0.f, 0.f, 0.f, 0.f});
        if (c + 1 < CPI) {
            const int nb1 = n_base + min(c + 1, nc - 1) * kCols;
            load_b(bq[c + 1], nb1);
            load_y(yv[c + 1], nb1);
        }
        if (c > 0) lds_barrier();   // every wave has read the previous chunk's deltas
        // lane: token `row`, columns 128 w + 16 nb + 4 quad .. + 3 of the chunk
        if (row < kSubTok) {
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
                *reinterpret_cast<float4 *>(s_delta + row * (kCols + 4) + w * kColsW + 16 * nb + 4 * quad) =
                    make_float4(sc * out[nb][0], sc * out[nb][1], sc * out[nb][2], sc * out[nb][3]);
        }
        // the count is needed before the y stores: a wait on it after them would
        // also wait for the stores (vmcnt counts both)
        if (c == 0 && tid == 0) s_last[0] = nread == n_readers - 1;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int tk = TW * w + i;
            const int cl = 8 * lane;
            if (c < nc && tk < ct && nb0 + cl < Ns) {
                const float4 d0 = *reinterpret_cast<const float4 *>(s_delta + tk * (kCols + 4) + cl);
                const float4 d1 = *reinterpret_cast<const float4 *>(s_delta + tk * (kCols + 4) + cl + 4);
                const uint4 y0 = yv[c][i];
                uint4 o;
                o.x = pack_bf16x2(bf16_lo(y0.x) + d0.x, bf16_hi(y0.x) + d0.y);
                o.y = pack_bf16x2(bf16_lo(y0.y) + d0.z, bf16_hi(y0.y) + d0.w);
                o.z = pack_bf16x2(bf16_lo(y0.z) + d1.x, bf16_hi(y0.z) + d1.y);
                o.w = pack_bf16x2(bf16_lo(y0.w) + d1.z, bf16_hi(y0.w) + d1.w);
                stg_nt(yrow[i] + nb0 + cl, o);
            }
        }
    }
    // the last reader of the block writes it back to zero for the next call
    if (s_last[0]) {
        for (int e = tid; e < a.n_kc * ct * (RP / 2); e += kThreads) {
            const int k = e / (ct * (RP / 2)), rem = e - k * (ct * (RP / 2));
            st_coherent(const_cast<float *>(blk) + (int64_t)k * a.T * RP + 2 * rem, 0ull);
        }
        if (tid == 0) __hip_atomic_store(readers, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

int32_t relay_max_groups(int32_t T, int32_t L) {
    return (T + kRelayGroup - 1) / kRelayGroup + (T < L ? T : L);
}

int32_t relay_sync_ints(int32_t T, int32_t L, int32_t S) {
    return kLine * (relay_max_groups(T, L) * S * kMaxSubs);
}

hipError_t launch_dec_relay(void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T,
                            int32_t K, const Slices &sl, int32_t S, int32_t L, int32_t R,
                            const int32_t *idx, const int32_t *slot_rank, const float *scale,
                            float *part, int32_t *sync, int32_t *err, bool give_up,
                            hipStream_t st) {
    RelayArgs a;
    a.x = static_cast<const uint16_t *>(x); a.ldx = ldx;
    a.y = static_cast<uint16_t *>(y); a.ldy = ldy;
    a.T = T; a.K = K; a.S = S; a.L = L; a.R = R;
    a.idx = idx; a.slot_rank = slot_rank; a.scale = scale; a.sl = sl;
    a.part = part; a.sync = sync; a.err = err; a.give_up = give_up ? 1 : 0;
    a.n_kc = K / kKc;
    a.max_groups = relay_max_groups(T, L);
    // one lora_a for every slice (the same pointer): one shrink for all
    bool shared_a = S > 1;
    for (int s = 1; s < S && shared_a; ++s) shared_a = sl.a[s] == sl.a[0];
    a.S_shrink = shared_a ? 1 : S;
    // The first part holds the groups a batch usually fills: the larger of
    // T/32 plus half the slots, and the expected number of slots with tokens
    // (slots drawn uniformly) plus two.
    {
        const int tl = T < L ? T : L;
        const int dense = (T + kG - 1) / kG + (tl + 1) / 2;
        const int sparse = (int)ceil(L * (1.0 - exp(-(double)T / L))) + 2;
        a.n_first = min(a.max_groups, dense > sparse ? dense : sparse);
    }
    // wide outputs: 16-token expand items (half the lora_b block reads)
    int64_t ntot = 0;
    for (int s = 0; s < S; ++s) ntot += sl.n[s];
    const bool wide = ntot > kAutoMaxDecodeCols;
    const int subs = wide ? kG / 16 : kG / 8;
    int n_chunks = 0;
    for (int s = 0; s < S; ++s) n_chunks += (int)((sl.n[s] + kCols - 1) / kCols);
    // chunks per expand item: as many as keep the expected expand items at
    // four work-groups per CU or more
    int cpi = 1;
    if (wide)
        while (cpi < kRelayMaxCpi && a.n_first * ((n_chunks + 2 * cpi - 1) / (2 * cpi)) * subs >= kRelayMinItems)
            cpi *= 2;
    int c = 0, it = 0;
    for (int s = 0; s < S; ++s) {
        a.chunk_start[s] = c;
        a.item_start[s] = it;
        const int ch = (int)((sl.n[s] + kCols - 1) / kCols);
        c += ch;
        it += (ch + cpi - 1) / cpi;
    }
    for (int s = S; s <= kMaxSlices; ++s) {
        a.chunk_start[s] = c;
        a.item_start[s] = it;
    }
    a.n_items = it;
    const auto sblocks = [&](int groups) { return 8 * ((groups * a.n_kc + 7) / 8 * a.S_shrink); };
    const auto eblocks = [&](int groups) { return 8 * ((groups * it + 7) / 8 * subs); };
    a.pstart[0] = sblocks(a.n_first);
    a.pstart[1] = a.pstart[0] + eblocks(a.n_first);
    a.pstart[2] = a.pstart[1] + sblocks(a.max_groups - a.n_first);
    a.pstart[3] = a.pstart[2] + eblocks(a.max_groups - a.n_first);
    dim3 grid((unsigned)a.pstart[3]);
    const bool few = a.n_kc <= 16;
#define AA_RELAY(NRB, MKC, SUB, CPI) hipLaunchKernelGGL((k_dec_relay<NRB, MKC, SUB, CPI>), grid, dim3(kThreads), 0, st, a)
#define AA_RELAY_SUB(NRB, MKC)                                                       \
    do {                                                                             \
        if (!wide) AA_RELAY(NRB, MKC, 8, 1);                                         \
        else if (cpi == 1) AA_RELAY(NRB, MKC, 16, 1);                                \
        else if (cpi == 2) AA_RELAY(NRB, MKC, 16, 2);                                \
        else AA_RELAY(NRB, MKC, 16, 4);                                              \
    } while (0)
    if (R == 16) {
        if (few) AA_RELAY_SUB(1, 16);
        else AA_RELAY_SUB(1, kRelayMaxKc);
    } else {
        if (few) AA_RELAY_SUB(2, 16);
        else AA_RELAY_SUB(2, kRelayMaxKc);
    }
#undef AA_RELAY_SUB
#undef AA_RELAY
    return hipGetLastError();
}

}  // namespace aa
