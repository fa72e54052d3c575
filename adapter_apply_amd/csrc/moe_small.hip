// Fused-MoE LoRA delta of a small batch without the alignment.
//
// [vLLM] FusedMoEWithLoRA switches to a naive, unsorted regime when the batch
// holds few (token, k) pairs for its experts and adapters: sorting them by
// (slot, expert) then costs more than it saves.  Here a batch of at most
// kMoeSmallPairs pairs skips the segment build: work-group = (pair, 1024
// output columns of one slice).  Each work-group computes its pair's shrink
// x[row] . A[slot][ea]^T (1024 threads over K, 8 elements per thread and
// step, fp32, then a wave butterfly and an ordered sum over the 16 waves),
// and expands its columns from that fp32 buffer, one column per thread:
// y[p][off + n] = RNE(y + scale[slot] * coef[p] * sum_j buf[j] * B[n][j]).
// The shrink is recomputed by each column chunk of a pair; at this size the
// bytes are lora_a and lora_b, read once per pair and chunk through the L2.
#include "common.hpp"

namespace aa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCols = 1024;                // output columns per work-group
constexpr int kRank = 16;                  // the padded rank this kernel takes

struct SmallArgs {
    uint16_t *y;
    int64_t ldy;
    const uint16_t *x;
    int64_t ldx;
    int32_t K, E, L, R, S, Ea, Eb, top_k, x_div, n_chunks;
    const int32_t *idx;
    const int32_t *topk;
    const int32_t *slot_rank;
    const float *scale;
    const float *coef;         // per pair, or null
    Slices sl;
    int32_t chunk_start[kMaxSlices + 1];
};

// sum_i x[i] * a[i] over 8 bf16 pairs, in order, fp32
__device__ __forceinline__ float dot8(const uint4 &x, const uint4 &a, float acc) {
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, as[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = fmaf(bf16_lo(xs[q]), bf16_lo(as[q]), acc);
        acc = fmaf(bf16_hi(xs[q]), bf16_hi(as[q]), acc);
    }
    return acc;
}

__global__ __launch_bounds__(kThreads) void k_moe_small(SmallArgs a) {
    __shared__ float s_part[kWaves][kRank];
    __shared__ float s_buf[kRank];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int p = blockIdx.x / a.n_chunks;
    const int chunk = blockIdx.x - p * a.n_chunks;
    const int t = p / a.top_k;
    const int s = a.idx[t];
    const int e = a.topk[p];
    if (s < 0 || s >= a.L || e < 0 || e >= a.E) return;       // uniform: no delta
    const int r = a.slot_rank ? min(a.slot_rank[s], kRank) : kRank;
    if (r <= 0) return;
    int sg = 0;
    while (sg + 1 < a.S && chunk >= a.chunk_start[sg + 1]) ++sg;
    const int Ns = (int)a.sl.n[sg];
    const int n_base = (chunk - a.chunk_start[sg]) * kCols;

    // ---- shrink: thread tid takes elements 8 tid + 8192 i of K ------------
    const uint16_t *xr = a.x + (int64_t)(p / a.x_div) * a.ldx;
    const uint16_t *ar = static_cast<const uint16_t *>(a.sl.a[sg]) +
                         (int64_t)(s * a.Ea + (a.Ea == 1 ? 0 : e)) * kRank * a.K;
    float acc[kRank];
#pragma unroll
    for (int j = 0; j < kRank; ++j) acc[j] = 0.0f;
    for (int k0 = 8 * tid; k0 < a.K; k0 += 8 * kThreads) {
        const uint4 xv = ldg<uint4>(xr + k0);
        uint4 av[kRank];
#pragma unroll
        for (int j = 0; j < kRank; ++j) av[j] = ldg<uint4>(ar + (int64_t)min(j, r - 1) * a.K + k0);
#pragma unroll
        for (int j = 0; j < kRank; ++j) acc[j] = dot8(xv, av[j], acc[j]);
    }
    // wave butterfly (the same order on every lane), then the waves in order
#pragma unroll
    for (int j = 0; j < kRank; ++j) {
        float v = acc[j];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
        acc[j] = v;
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kRank; ++j) s_part[w][j] = acc[j];
    }
    __syncthreads();
    if (tid < kRank) {
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) v += s_part[q][tid];
        s_buf[tid] = tid < r ? v : 0.0f;
    }
    __syncthreads();

    // ---- expand: thread tid takes column n_base + tid ---------------------
    const int n = n_base + tid;
    if (n >= Ns) return;
    const uint16_t *br = static_cast<const uint16_t *>(a.sl.b[sg]) +
                         ((int64_t)(s * a.Eb + (a.Eb == 1 ? 0 : e)) * Ns + n) * kRank;
    const uint4 b0 = ldg<uint4>(br), b1 = ldg<uint4>(br + 8);
    const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    float d = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        d = fmaf(s_buf[2 * q], bf16_lo(bw[q]), d);
        d = fmaf(s_buf[2 * q + 1], bf16_hi(bw[q]), d);
    }
    const float c = a.scale[s] * (a.coef ? a.coef[p] : 1.0f);
    uint16_t *yp = a.y + (int64_t)p * a.ldy + a.sl.off[sg] + n;
    const float yv = __builtin_bit_cast(float, (uint32_t)*yp << 16);
    *yp = (uint16_t)f32_to_bf16_rne(yv + c * d);
}

}  // namespace

bool moe_small_takes(int32_t pairs, int32_t R, int32_t reduce_k) {
    return pairs <= kMoeSmallPairs && R == kRank && !reduce_k;
}

hipError_t launch_moe_small(void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T, int32_t top_k,
                            int32_t K, const Slices &sl, int32_t S, int32_t E, int32_t L, int32_t R,
                            int32_t Ea, int32_t Eb, int32_t x_div, const int32_t *topk_ids,
                            const float *coef, const int32_t *idx, const int32_t *slot_rank,
                            const float *scale, hipStream_t st) {
    SmallArgs a{};
    a.y = static_cast<uint16_t *>(y); a.ldy = ldy;
    a.x = static_cast<const uint16_t *>(x); a.ldx = ldx;
    a.K = K; a.E = E; a.L = L; a.R = R; a.S = S; a.Ea = Ea; a.Eb = Eb; a.top_k = top_k;
    a.x_div = x_div;
    a.idx = idx; a.topk = topk_ids; a.slot_rank = slot_rank; a.scale = scale; a.coef = coef;
    a.sl = sl;
    int c = 0;
    for (int s = 0; s < S; ++s) {
        a.chunk_start[s] = c;
        c += (int)((sl.n[s] + kCols - 1) / kCols);
    }
    for (int s = S; s <= kMaxSlices; ++s) a.chunk_start[s] = c;
    a.n_chunks = c;
    const int64_t grid = (int64_t)T * top_k * c;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_moe_small, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace aa
