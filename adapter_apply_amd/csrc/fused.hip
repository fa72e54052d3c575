// Single-launch decode: shrink and expand of a small batch in one kernel.
//
// At decode sizes (a few hundred tokens) the delta moves ~10 MB and every
// extra kernel or dependent global load costs more than the data itself, so
// this path has no segment build, no workspace and no second launch.
//
// Work-group (16 waves) = (token group g, output chunk c of 1024 columns of
// one slice).  The groups are the slot-major runs of at most 8 tokens that a
// stable sort by slot would give; every work-group derives them itself from
// idx (discover.hpp), so its only dependent global loads are
// idx -> {x, lora_a, lora_b, y}.  Work-group i runs on XCD i % 8 (round-robin
// dispatch); XCD x takes a contiguous range of groups with all their chunks,
// so the chunks of a group, and mostly the groups of a slot, share one L2.
// Each work-group then
//   1. shrinks its group for that slice with v_mfma_f32_16x16x32_bf16
//      (16-row token tiles, 8 of them real; the 16 waves split K and add in
//      LDS),
//   2. expands its columns with v_mfma_f32_16x16x16_bf16 formed as
//      D[n][t] = B[n][:] . buf[t][:].
// Group size: a work-group streams its group's x rows and the slot's lora_a
// slice through one CU (8 tokens: 64 KB + 128 KB at K = 4096); 8 rather than
// 16 tokens per group cut that volume by a quarter and spread the work over
// twice as many CUs.
// The shrink of a (group, slice) is recomputed by each chunk of that slice:
// the price of one launch, paid in reads of the XCD's L2 (x rows, lora_a rows).
// Every global access is row-contiguous (a wave instruction covers whole
// 128-byte lines): on this part a load that spreads a wave over 16 rows at
// 64 bytes each runs ~3.5x slower per CU than one covering 8 full lines.
// Each wave therefore loads its K slice of the x and lora_a rows line by line,
// all before the first use, and turns them into MFMA fragments through its
// own swizzled LDS staging area; the output goes through an LDS buffer so y
// is read and written 16 bytes per lane along rows.
#include "discover.hpp"

namespace aa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;   // 16
constexpr int kG = kFusedGroup;            // tokens per group (8)
constexpr int kM = 16;                     // MFMA tile rows: tokens kG..15 are padding
constexpr int kCols = kFusedCols;          // output columns per work-group (1024)
constexpr int kColsW = kCols / kWaves;     // 64 per wave = 4 blocks of 16
constexpr int kSub = 64;                   // K elements per sub-chunk: one 128-byte line per row

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

struct FusedArgs {
    const uint16_t *x;
    int64_t ldx;
    uint16_t *y;
    int64_t ldy;
    int32_t T, K, S, L, R, n_chunks;
    const int32_t *idx;
    const int32_t *slot_rank;
    const float *scale;
    Slices sl;
    int32_t chunk_start[kMaxSlices + 1];
};

__device__ __forceinline__ bf16x8_t frag8(const uint4 &u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ short4_t frag4(const uint2 &u) { return __builtin_bit_cast(short4_t, u); }

// Byte offset of 16-byte unit u of row r in a staging area of 128-byte rows;
// the unit index is XOR-swizzled with the row so fragment reads of 8
// consecutive rows hit 8 different bank groups.
__device__ __forceinline__ int stage_off(int r, int u) { return r * 128 + ((u ^ (r & 7)) << 4); }

// NRB: 16-rank blocks of the padded rank R (1 or 2); the slot's own rank may be lower.
template <int NRB>
struct FusedSmem {
    static constexpr int RR = kG + 16 * NRB;                   // staged rows per sub-chunk: x then lora_a
    static constexpr int kStage = kWaves * RR * 128;           // per-wave staging areas
    static constexpr int kDelta = kM * (kCols + 4) * 4;        // fp32 deltas, aliases the staging
    static constexpr int kUnion = kStage > kDelta ? kStage : kDelta;
    static constexpr int kPart = kWaves * kM * (NRB * 16 + 4) * 4;
};

template <int NRB>
__global__ __launch_bounds__(kThreads) void k_dec_fused(FusedArgs a) {
    using SM = FusedSmem<NRB>;
    constexpr int RR = SM::RR;
    constexpr int SUBB = 4 / NRB;                  // sub-chunks per load batch (register budget)
    constexpr int LPS = RR / 8;                    // load instructions per sub-chunk (8 rows x 128 B each)
    constexpr int BROW = NRB * 32;                 // bytes of one lora_b row (R = 16 * NRB)
    constexpr int BLD = kColsW * BROW / 1024;      // load instructions for a wave's lora_b rows

    __shared__ __attribute__((aligned(16))) char s_union[SM::kUnion];
    __shared__ __attribute__((aligned(16))) float s_part[kWaves][kM][NRB * 16 + 4];
    __shared__ DiscLds<kG, kFusedMaxTokens, kWaves> g;
    __shared__ __attribute__((aligned(16))) uint16_t s_buf[kM][NRB * 16 + 8];   // bf16 buffer

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int xcd = blockIdx.x % kFusedXcds;
    const int j = blockIdx.x / kFusedXcds;
    const int chunk = j % a.n_chunks;
    const int lg = j / a.n_chunks;
    const auto pick = [=](int n) {
        const int per = (n + kFusedXcds - 1) / kFusedXcds;
        return lg < per ? xcd * per + lg : -1;
    };
    const GroupSel gsel = find_group(a.idx, a.slot_rank, a.T, a.L, a.R, g, pick);
    const int32_t *s_tok = g.tok;
    const int s = gsel.slot;
    if (s < 0) return;
    const int ntok = gsel.ntok;
    const int r = gsel.rank;
    int sg = 0;
    while (sg + 1 < a.S && chunk >= a.chunk_start[sg + 1]) ++sg;
    const int Ns = (int)a.sl.n[sg];
    const int n_base = (chunk - a.chunk_start[sg]) * kCols;

    const int row = lane & 15, quad = lane >> 4;
    const float sc = a.scale[s];
    char *stage = s_union + w * (RR * 128);

    // ---- 2. shrink of the group for slice sg (MFMA 16x16x32) ----------------
    // The first batch of shrink loads goes out first, then the expand-side
    // loads (lora_b rows, y rows), which land while the shrink computes.
    const char *bblk = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.sl.b[sg]) +
                                                      (int64_t)s * Ns * a.R);
    const bool ytok = w < ntok;
    uint16_t *yrow = a.y + (int64_t)s_tok[ytok ? w : 0] * a.ldy + a.sl.off[sg];
    uint4 bq[BLD];
    uint4 yv[2];
    floatx4_t acc[NRB];
    {
        // staged row p: x row of token p (p < kG) or lora_a rank row p - kG; rows
        // past the group or the rank are clamped to valid ones and dropped later.
        // MFMA rows kG..15 read staged lora_a rows: finite values whose
        // outputs belong to padding tokens, zeroed with the buffer.
        const uint16_t *srcrow[LPS];
        const uint16_t *abase = static_cast<const uint16_t *>(a.sl.a[sg]) + (int64_t)s * a.R * a.K;
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int p = 8 * i + (lane >> 3);
            srcrow[i] = p < kG ? a.x + (int64_t)s_tok[p < ntok ? p : 0] * a.ldx
                               : abase + (int64_t)min(p - kG, r - 1) * a.K;
        }
        const int ucol = 8 * (lane & 7);                       // element offset of this lane's unit
        const int kw = a.K / kWaves;                           // K % 1024 == 0
        const int nsub = kw / kSub;
#pragma unroll
        for (int b = 0; b < NRB; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        uint4 v[SUBB][LPS];
        // batch c0: SUBB sub-chunks of 64 K columns; one past the end re-reads the
        // last one and contributes zero (a select, not a branch, keeps loads in flight)
        auto issue = [&](int c0) {
#pragma unroll
            for (int c = 0; c < SUBB; ++c)
#pragma unroll
                for (int i = 0; i < LPS; ++i) {
                    const int k = w * kw + (c0 + min(c, nsub - 1 - c0)) * kSub + ucol;
                    v[c][i] = ldg<uint4>(srcrow[i] + k);
                }
        };
        auto consume = [&](int c0) {
#pragma unroll
            for (int c = 0; c < SUBB; ++c) {
                const bool cv = c0 + c < nsub;
#pragma unroll
                for (int i = 0; i < LPS; ++i)
                    *reinterpret_cast<uint4 *>(stage + stage_off(8 * i + (lane >> 3), lane & 7)) = v[c][i];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint4 xf = *reinterpret_cast<const uint4 *>(stage + stage_off(row, 4 * ks + quad));
                    if (!cv) xf = make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int b = 0; b < NRB; ++b) {
                        const uint4 af = *reinterpret_cast<const uint4 *>(stage + stage_off(kG + 16 * b + row, 4 * ks + quad));
                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag8(xf), frag8(af), acc[b], 0, 0, 0);
                    }
                }
            }
        };
        issue(0);
        // lora_b rows of this wave's 64 columns: one contiguous block of 64 * BROW bytes
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int byte = 1024 * i + 16 * lane;
            const int nr = min(n_base + w * kColsW + byte / BROW, Ns - 1);
            bq[i] = ldg<uint4>(reinterpret_cast<const uint4 *>(bblk + (int64_t)nr * BROW + byte % BROW));
        }
        // y: wave w owns token w of the group, 8 columns per lane, 2 x 512 columns
#pragma unroll
        for (int i = 0; i < 2; ++i) yv[i] = ldg_nt(yrow + min(n_base + 512 * i + 8 * lane, Ns - 8));
        __builtin_amdgcn_sched_barrier(0);
        consume(0);
        for (int c0 = SUBB; c0 < nsub; c0 += SUBB) {
            issue(c0);
            __builtin_amdgcn_sched_barrier(0);
            consume(c0);
        }
        // acc[b][i]: token 4*quad + i, rank 16*b + row
#pragma unroll
        for (int b = 0; b < NRB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_part[w][4 * quad + i][16 * b + row] = acc[b][i];
    }
    __syncthreads();
    // Sum the 16 K slices in order; store bf16 (ranks past r, tokens past ntok: 0).
    for (int i = tid; i < kM * NRB * 16; i += kThreads) {
        const int tk = i / (NRB * 16), j = i - tk * (NRB * 16);
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) v += s_part[q][tk][j];
        if (j >= r || tk >= ntok) v = 0.0f;
        s_buf[tk][j] = (uint16_t)f32_to_bf16_rne(v);
    }
    __syncthreads();

    // ---- 4. expand (MFMA 16x16x16): D[n][t] = B[n][:] . buf[t][:] ----------
    // The wave's lora_b rows go through its own staging area into fragment order.
#pragma unroll
    for (int i = 0; i < BLD; ++i) *reinterpret_cast<uint4 *>(stage + 1024 * i + 16 * lane) = bq[i];
    uint2 bfr[NRB];
#pragma unroll
    for (int ks = 0; ks < NRB; ++ks)
        bfr[ks] = *reinterpret_cast<const uint2 *>(&s_buf[row][16 * ks + 4 * quad]);
    floatx4_t out[kColsW / 16];
#pragma unroll
    for (int nb = 0; nb < kColsW / 16; ++nb) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NRB; ++ks) {
            const uint2 af = *reinterpret_cast<const uint2 *>(stage + (16 * nb + row) * BROW + 32 * ks + 8 * quad);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(af), frag4(bfr[ks]), acc, 0, 0, 0);
        }
        out[nb] = acc;
    }
    __syncthreads();   // every wave is done with its staging area (the delta buffer aliases it)
    // lane: token `row`, columns 64w + 16nb + 4*quad .. +3 of the chunk
    float *s_delta = reinterpret_cast<float *>(s_union);
#pragma unroll
    for (int nb = 0; nb < kColsW / 16; ++nb)
        *reinterpret_cast<float4 *>(s_delta + row * (kCols + 4) + w * kColsW + 16 * nb + 4 * quad) =
            make_float4(sc * out[nb][0], sc * out[nb][1], sc * out[nb][2], sc * out[nb][3]);
    __syncthreads();
    // y: wave w writes token w's row, 16 bytes per lane.
    if (ytok) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int cl = 512 * i + 8 * lane;
            if (n_base + cl < Ns) {
                const float4 d0 = *reinterpret_cast<const float4 *>(s_delta + w * (kCols + 4) + cl);
                const float4 d1 = *reinterpret_cast<const float4 *>(s_delta + w * (kCols + 4) + cl + 4);
                const uint4 y0 = yv[i];
                uint4 o;
                o.x = pack_bf16x2(bf16_lo(y0.x) + d0.x, bf16_hi(y0.x) + d0.y);
                o.y = pack_bf16x2(bf16_lo(y0.y) + d0.z, bf16_hi(y0.y) + d0.w);
                o.z = pack_bf16x2(bf16_lo(y0.z) + d1.x, bf16_hi(y0.z) + d1.y);
                o.w = pack_bf16x2(bf16_lo(y0.w) + d1.z, bf16_hi(y0.w) + d1.w);
                stg_nt(yrow + n_base + cl, o);
            }
        }
    }
}

}  // namespace

int32_t fused_max_groups(int32_t T, int32_t L) {
    return (T + kFusedGroup - 1) / kFusedGroup + (T < L ? T : L);
}

hipError_t launch_dec_fused(void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T,
                            int32_t K, const Slices &sl, int32_t S, int32_t L, int32_t R,
                            const int32_t *idx, const int32_t *slot_rank, const float *scale,
                            hipStream_t st) {
    FusedArgs a;
    a.x = static_cast<const uint16_t *>(x); a.ldx = ldx;
    a.y = static_cast<uint16_t *>(y); a.ldy = ldy;
    a.T = T; a.K = K; a.S = S; a.L = L; a.R = R;
    a.idx = idx; a.slot_rank = slot_rank; a.scale = scale; a.sl = sl;
    int c = 0;
    for (int s = 0; s < S; ++s) {
        a.chunk_start[s] = c;
        c += (int)((sl.n[s] + kCols - 1) / kCols);
    }
    for (int s = S; s <= kMaxSlices; ++s) a.chunk_start[s] = c;
    a.n_chunks = c;
    const int per_xcd = (fused_max_groups(T, L) + kFusedXcds - 1) / kFusedXcds;
    dim3 grid((unsigned)(kFusedXcds * per_xcd * c));
    if (R <= 16)
        hipLaunchKernelGGL(k_dec_fused<1>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_dec_fused<2>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace aa
