// Single-launch decode: shrink and expand of a small batch in one kernel.
//
// At decode sizes (a few hundred tokens) the delta moves ~10 MB and every
// extra kernel or dependent global load costs more than the data itself, so
// this path has no segment build, no workspace and no second launch.
//
// Work-group (16 waves) = (token group g, output chunk c).  The groups are the slot-major
// runs of at most 16 tokens that a stable sort by slot would give; every
// work-group derives them itself from idx (staged in LDS: histogram, scan over
// slots, ballot compaction), so its only dependent global loads are
// idx -> {x, lora_a, lora_b, y}.  The chunk is 512 output columns of one
// slice.  Each work-group then
//   1. shrinks its group for that slice with v_mfma_f32_16x16x32_bf16
//      (16 tokens x 16 ranks blocks; the 16 waves split K and add in LDS),
//   2. expands its 512 columns with v_mfma_f32_16x16x16_bf16 formed as
//      D[n][t] = B[n][:] . buf[t][:], so a lane holds 4 consecutive columns of
//      one token and y moves 8 bytes per lane.
// The shrink of a (group, slice) is recomputed by each chunk of that slice:
// the price of one launch, paid in L2 reads (x rows and lora_a rows).
// The kernel is bound by memory latency, so every global load a wave needs
// (its K slice of x and lora_a, its lora_b rows and y values) is issued
// before the first of them is consumed.
#include "common.hpp"

namespace aa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;   // 16: each owns 1/16 of K and 2 of the 32 column blocks
constexpr int kG = kFusedGroup;            // tokens per group
constexpr int kCols = kFusedCols;          // output columns per work-group
constexpr int kRmax = kFusedMaxRank;       // ranks held in LDS
constexpr int kNbPerWave = kCols / 16 / kWaves;

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

// NRB: 16-rank blocks of the padded rank R (1..4); the per-slot rank may be lower.
template <int NRB>
__global__ __launch_bounds__(kThreads) void k_dec_fused(FusedArgs a) {
    constexpr int KB = 8 / NRB;   // k-steps of 32 per load batch (register budget)
    __shared__ int32_t s_slot[kFusedMaxTokens];   // active slot of each token, -1 if none
    __shared__ int32_t s_rank[kMaxSlots];
    __shared__ int32_t s_cnt[kMaxSlots];          // tokens per slot
    __shared__ int32_t s_tok[kG];
    __shared__ int32_t s_info[4];                 // slot, rank within slot of the first token, count
    __shared__ float s_part[kWaves][kG][NRB * 16 + 4];
    __shared__ __attribute__((aligned(16))) uint16_t s_buf[kG][NRB * 16 + 8];   // bf16 buffer

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // All chunks of a group go to one XCD (work-groups are dealt to the 8 XCDs
    // round-robin), so the group's x rows and lora_a rows are fetched into one L2.
    const int xcd = blockIdx.x % kFusedXcds;
    const int local = blockIdx.x / kFusedXcds;
    const int chunk = local % a.n_chunks;
    const int group = xcd + kFusedXcds * (local / a.n_chunks);
    if (group >= a.max_groups) return;
    const int T = a.T, L = a.L;

    // ---- 1. who am I: stage idx and ranks, count per slot -------------------
    for (int i = tid; i < L; i += kThreads) {
        s_rank[i] = a.slot_rank ? min(a.slot_rank[i], a.R) : a.R;
        s_cnt[i] = 0;
    }
    for (int i = tid; i < T; i += kThreads) s_slot[i] = a.idx[i];
    __syncthreads();
    for (int i = tid; i < T; i += kThreads) {
        const int v = s_slot[i];
        const bool ok = v >= 0 && v < L && s_rank[v] > 0;
        s_slot[i] = ok ? v : -1;
        if (ok) atomicAdd(&s_cnt[v], 1);
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
    const int64_t Ns = a.sl.n[sg];
    const int n_base = (chunk - a.chunk_start[sg]) * kCols;
    __syncthreads();

    const int nrb = (r + 15) >> 4;                       // 16-rank blocks of this slot
    const int row = lane & 15, quad = lane >> 4;
    const float sc = a.scale[s];

    // ---- 2. expand-side loads first: they do not depend on the shrink -------
    // A operand: lora_b rows (output columns); y: token `row`, 4 columns.
    const uint16_t *bbase = static_cast<const uint16_t *>(a.sl.b[sg]) + (int64_t)s * Ns * a.R;
    // Unconditional loads from clamped rows (the group's first token, the last
    // output column; R >= 16 * NRB); padding results are never stored.
    const bool tcol_ok = row < ntok;
    uint16_t *yrow = a.y + (int64_t)s_tok[tcol_ok ? row : 0] * a.ldy + a.sl.off[sg];
    uint2 bq[kNbPerWave][NRB], yv[kNbPerWave];
    bool y_ok[kNbPerWave];
#pragma unroll
    for (int e = 0; e < kNbPerWave; ++e) {
        const int n0 = n_base + (w + kWaves * e) * 16;
        const uint16_t *brow = bbase + (int64_t)min(n0 + row, (int)Ns - 1) * a.R;
#pragma unroll
        for (int ks = 0; ks < NRB; ++ks) bq[e][ks] = ldg<uint2>(brow + 16 * ks + 4 * quad);
        const int n = n0 + 4 * quad;
        y_ok[e] = tcol_ok && n < Ns;                     // N_s % 4 == 0
        yv[e] = ldg<uint2>(yrow + min(n, (int)Ns - 4));
    }

    // ---- 3. shrink of the group for slice sg (MFMA 16x16x32) ----------------
    {
        // x rows past the group and lora_a rows past the rank are clamped to valid
        // rows; the garbage they make is dropped when the buffer is formed.
        const uint16_t *xr = a.x + (int64_t)s_tok[row < ntok ? row : 0] * a.ldx;
        const uint16_t *abase = static_cast<const uint16_t *>(a.sl.a[sg]) + (int64_t)s * a.R * a.K;
        const uint16_t *arow[NRB];
#pragma unroll
        for (int b = 0; b < NRB; ++b) arow[b] = abase + (int64_t)min(16 * b + row, r - 1) * a.K;
        const int ksteps = (a.K + 31) >> 5;
        const int kper = (ksteps + kWaves - 1) / kWaves;
        const int k_lo = w * kper * 32, k_hi = min(a.K, (w + 1) * kper * 32);
        floatx4_t acc[NRB];
#pragma unroll
        for (int b = 0; b < NRB; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        int k0 = k_lo;
        for (; k0 + KB * 32 <= k_hi; k0 += KB * 32) {   // whole batches, no guards
            uint4 xf[KB], af[KB][NRB];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const int k = k0 + 32 * u + 8 * quad;
                xf[u] = ldg<uint4>(xr + k);
#pragma unroll
                for (int b = 0; b < NRB; ++b) af[u][b] = ldg<uint4>(arow[b] + k);
            }
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
                for (int b = 0; b < NRB; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag8(xf[u]), frag8(af[u][b]), acc[b], 0, 0, 0);
        }
        for (; k0 < k_hi; k0 += 32) {                     // K tail, guarded (K % 8 == 0)
            const int k = k0 + 8 * quad;
            uint4 xf = make_uint4(0, 0, 0, 0), af[NRB];
            if (k < k_hi) xf = ldg<uint4>(xr + k);
#pragma unroll
            for (int b = 0; b < NRB; ++b) {
                af[b] = make_uint4(0, 0, 0, 0);
                if (k < k_hi) af[b] = ldg<uint4>(arow[b] + k);
            }
#pragma unroll
            for (int b = 0; b < NRB; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag8(xf), frag8(af[b]), acc[b], 0, 0, 0);
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
    uint2 bfr[NRB];
#pragma unroll
    for (int ks = 0; ks < NRB; ++ks)
        bfr[ks] = *reinterpret_cast<const uint2 *>(&s_buf[row][16 * ks + 4 * quad]);
#pragma unroll
    for (int e = 0; e < kNbPerWave; ++e) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NRB; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(bq[e][ks]), frag4(bfr[ks]), acc, 0, 0, 0);
        // lane: token `row`, columns n0 + 4*quad .. +3
        if (y_ok[e]) {
            const int n = n_base + (w + kWaves * e) * 16 + 4 * quad;
            uint2 o;
            o.x = pack_bf16x2(bf16_lo(yv[e].x) + sc * acc[0], bf16_hi(yv[e].x) + sc * acc[1]);
            o.y = pack_bf16x2(bf16_lo(yv[e].y) + sc * acc[2], bf16_hi(yv[e].y) + sc * acc[3]);
            *reinterpret_cast<uint2 *>(yrow + n) = o;
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
    const int per_xcd = (a.max_groups + kFusedXcds - 1) / kFusedXcds;
    dim3 grid((unsigned)(kFusedXcds * per_xcd * c));
    switch ((R + 15) / 16) {
        case 1: hipLaunchKernelGGL(k_dec_fused<1>, grid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_dec_fused<2>, grid, dim3(kThreads), 0, st, a); break;
        case 3: hipLaunchKernelGGL(k_dec_fused<3>, grid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL(k_dec_fused<4>, grid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace aa
