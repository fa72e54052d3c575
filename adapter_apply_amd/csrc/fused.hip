// Single-launch decode: shrink and expand of a small batch in one kernel.
//
// At decode sizes (a few hundred tokens) the delta moves ~10 MB and every
// extra kernel or dependent global load costs more than the data itself, so
// this path has no segment build, no workspace and no second launch.
//
// Work-group (16 waves) = (token group g, output chunk c of 1024 columns).  The groups are the slot-major
// runs of at most 16 tokens that a stable sort by slot would give; every
// work-group derives them itself from idx (staged in LDS: histogram, scan over
// slots, ballot compaction), so its only dependent global loads are
// idx -> {x, lora_a, lora_b, y}.  The chunk is 512 output columns of one
// slice.  Each work-group then
//   1. shrinks its group for that slice with v_mfma_f32_16x16x32_bf16
//      (16 tokens x 16 ranks blocks; the 16 waves split K and add in LDS),
//   2. expands its columns with v_mfma_f32_16x16x16_bf16 formed as
//      D[n][t] = B[n][:] . buf[t][:].
// The shrink of a (group, slice) is recomputed by each chunk of that slice:
// the price of one launch, paid in L2 reads (x rows and lora_a rows).
// Every global access is row-contiguous (a wave instruction covers whole
// 128-byte lines): on this part a load that spreads a wave over 16 rows at
// 64 bytes each runs ~3.5x slower per CU than one covering 8 full lines.
// Each wave therefore loads its K slice of the x and lora_a rows line by line,
// all before the first use, and turns them into MFMA fragments through its
// own swizzled LDS staging area; the output goes through an LDS buffer so y
// is read and written 16 bytes per lane along rows.
#include "common.hpp"

namespace aa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;   // 16
constexpr int kG = kFusedGroup;            // tokens per group (16)
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
    int32_t T, K, S, L, R, n_chunks, max_groups;
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
    static constexpr int RR = kG * (1 + NRB);                  // staged rows per sub-chunk: x then lora_a
    static constexpr int kStage = kWaves * RR * 128;           // per-wave staging areas
    static constexpr int kDelta = kG * (kCols + 4) * 4;        // fp32 deltas, aliases the staging
    static constexpr int kUnion = kStage > kDelta ? kStage : kDelta;
    static constexpr int kPart = kWaves * kG * (NRB * 16 + 4) * 4;
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
    __shared__ __attribute__((aligned(16))) float s_part[kWaves][kG][NRB * 16 + 4];
    __shared__ int32_t s_slot[kFusedMaxTokens];   // active slot of each token, -1 if none
    __shared__ int32_t s_rank[kMaxSlots];
    __shared__ int32_t s_cnt[kMaxSlots];          // tokens per slot
    __shared__ int32_t s_tok[kG];
    __shared__ int32_t s_info[4];                 // slot, rank within slot of the first token, count
    __shared__ __attribute__((aligned(16))) uint16_t s_buf[kG][NRB * 16 + 8];   // bf16 buffer

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // Live work-groups are the first ones, so they spread evenly over the XCDs.
    const int chunk = blockIdx.x % a.n_chunks;
    const int group = blockIdx.x / a.n_chunks;
    const int T = a.T, L = a.L;

    // ---- 1. who am I: stage idx and ranks, count per slot -------------------
    for (int i = tid; i < L; i += kThreads) {
        s_rank[i] = a.slot_rank ? min(a.slot_rank[i], a.R) : a.R;
        s_cnt[i] = 0;
    }
    for (int i = tid; i < T; i += kThreads) s_slot[i] = a.idx[i];
    __syncthreads();
    for (int base = w * kWave; base < T; base += kThreads) {
        // one LDS atomic per (wave, slot): lanes of a slot are counted by ballot
        const int i = base + lane;
        int v = i < T ? s_slot[i] : -1;
        v = (v >= 0 && v < L && s_rank[v] > 0) ? v : -1;
        if (i < T) s_slot[i] = v;
        uint64_t rem = __ballot(v >= 0);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int ls = __shfl(v, leader);
            const uint64_t peers = __ballot(v == ls);
            if (lane == leader) atomicAdd(&s_cnt[ls], __popcll(peers));
            rem &= ~peers;
        }
    }
    __syncthreads();
    // Wave 0: exclusive scan of groups per slot, find this group's slot.
    if (w == 0) {
        const int per = (L + kWave - 1) / kWave;
        const int lo = lane * per, hi = min(L, lo + per);
        int tot = 0;
        for (int s = lo; s < hi; ++s) tot += (s_cnt[s] + kG - 1) / kG;
        int incl = tot;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int run = incl - tot;
        for (int s = lo; s < hi; ++s) {
            const int c = s_cnt[s];
            const int ng = (c + kG - 1) / kG;
            if (group >= run && group < run + ng) {
                s_info[0] = s;
                s_info[1] = (group - run) * kG;
                s_info[2] = min(kG, c - (group - run) * kG);
            }
            run += ng;
        }
        if (lane == kWave - 1 && group >= incl) s_info[0] = -1;   // past the last group
    }
    __syncthreads();
    const int s = s_info[0];
    if (s < 0) return;
    const int first = s_info[1], ntok = s_info[2];
    const int r = s_rank[s];
    // Wave 0: the tokens of slot s with rank first .. first+ntok-1, ascending.
    if (w == 0) {
        int seen = 0;
        for (int base = 0; base < T && seen < first + ntok; base += kWave) {
            const int t = base + lane;
            const bool m = t < T && s_slot[t] == s;
            const uint64_t bal = __ballot(m);
            const int rk = seen + __popcll(bal & ((1ull << lane) - 1ull));
            if (m && rk >= first && rk < first + ntok) s_tok[rk - first] = t;
            seen += __popcll(bal);
        }
    }
    int sg = 0;
    while (sg + 1 < a.S && chunk >= a.chunk_start[sg + 1]) ++sg;
    const int Ns = (int)a.sl.n[sg];
    const int n_base = (chunk - a.chunk_start[sg]) * kCols;
    __syncthreads();

    const int row = lane & 15, quad = lane >> 4;
    const float sc = a.scale[s];
    char *stage = s_union + w * (RR * 128);

    // ---- 2. expand-side loads, row-contiguous, issued first ----------------
    // lora_b rows of this wave's 64 columns: one contiguous block of 64 * BROW bytes.
    const char *bblk = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.sl.b[sg]) +
                                                      (int64_t)s * Ns * a.R);
    uint4 bq[BLD];
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
        const int byte = 1024 * i + 16 * lane;                 // within the wave's block
        const int nr = min(n_base + w * kColsW + byte / BROW, Ns - 1);
        bq[i] = ldg<uint4>(reinterpret_cast<const uint4 *>(bblk + (int64_t)nr * BROW + byte % BROW));
    }
    // y: wave w owns token w of the group, 8 columns per lane, 2 x 512 columns.
    const bool ytok = w < ntok;
    uint16_t *yrow = a.y + (int64_t)s_tok[ytok ? w : 0] * a.ldy + a.sl.off[sg];
    uint4 yv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) yv[i] = ldg<uint4>(yrow + min(n_base + 512 * i + 8 * lane, Ns - 8));

    // ---- 3. shrink of the group for slice sg (MFMA 16x16x32) ----------------
    {
        // staged row p: x row of token p (p < 16) or lora_a rank row p - 16; rows
        // past the group or the rank are clamped to valid ones and dropped later.
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
        floatx4_t acc[NRB];
#pragma unroll
        for (int b = 0; b < NRB; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nsub; c0 += SUBB) {
            uint4 v[SUBB][LPS];
#pragma unroll
            for (int c = 0; c < SUBB; ++c)
#pragma unroll
                for (int i = 0; i < LPS; ++i) {
                    const int k = w * kw + (c0 + min(c, nsub - 1 - c0)) * kSub + ucol;
                    v[c][i] = ldg<uint4>(srcrow[i] + k);
                }
            // all of the batch's loads stay ahead of the first use
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < SUBB; ++c) {
                // a sub-chunk past the end (batch padding) re-reads the last one and
                // contributes zero: a select, not a branch, keeps the loads in flight
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
        }
        // acc[b][i]: token 4*quad + i, rank 16*b + row
#pragma unroll
        for (int b = 0; b < NRB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_part[w][4 * quad + i][16 * b + row] = acc[b][i];
    }
    __syncthreads();
    // Sum the 16 K slices in order; store bf16 (ranks past r, tokens past ntok: 0).
    for (int i = tid; i < kG * NRB * 16; i += kThreads) {
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
                *reinterpret_cast<uint4 *>(yrow + n_base + cl) = o;
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
    a.max_groups = fused_max_groups(T, L);
    dim3 grid((unsigned)(a.max_groups * c));
    if (R <= 16)
        hipLaunchKernelGGL(k_dec_fused<1>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_dec_fused<2>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace aa
