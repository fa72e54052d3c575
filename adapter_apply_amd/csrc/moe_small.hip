// Fused-MoE LoRA delta of a small batch without the alignment.
//
// [vLLM] FusedMoEWithLoRA switches to a naive, unsorted regime when the batch
// holds few (token, k) pairs for its experts and adapters: sorting them by
// (slot, expert) then costs more than it saves.  Here a batch of at most
// kMoeSmallPairs pairs skips the segment build: work-group = (pair, chunk of
// 512 * CPT output columns of one slice), 512 threads.  Each thread first
// loads the y values and (up to 2 columns per thread) the lora_b rows of its
// CPT adjacent columns, which do not depend on the shrink, then computes its
// part of the pair's shrink x[row] . A[slot][ea]^T (8 elements of K per
// thread and step, every rank row, fp32), which a wave sum and an ordered
// sum over the 8 waves complete;
// then y[p][off + n] = RNE(y + scale[slot] * coef[p] * sum_j buf[j] * B[n][j]).
// The shrink is recomputed by each column chunk of a pair; the host picks the
// smallest CPT (1, 2 or 4) whose grid holds at most one work-group per CU,
// so few pairs get many short chunks and more pairs fewer, wider ones (two
// work-groups on one CU share its load bandwidth and read lora_a twice).
#include "common.hpp"

namespace aa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kRank = 16;                  // the padded rank this kernel takes
constexpr int kResident = 256;         // work-groups of one round, one per CU

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

// CPT adjacent bf16 values of a y row (CPT * 2 bytes, aligned to that size)
template <int CPT> struct YVec;
template <> struct YVec<1> {
    uint16_t v;
    __device__ void load(const uint16_t *p) { v = *p; }
    __device__ float get(int) const { return bf16_to_f32(v); }
    __device__ void store(uint16_t *p, const float *d) { *p = (uint16_t)f32_to_bf16_rne(d[0]); }
};
template <> struct YVec<2> {
    uint32_t v;
    __device__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint32_t *>(p); }
    __device__ float get(int i) const { return i ? bf16_hi(v) : bf16_lo(v); }
    __device__ void store(uint16_t *p, const float *d) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(d[0], d[1]);
    }
};
template <> struct YVec<4> {
    uint2 v;
    __device__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint2 *>(p); }
    __device__ float get(int i) const {
        const uint32_t w = i < 2 ? v.x : v.y;
        return (i & 1) ? bf16_hi(w) : bf16_lo(w);
    }
    __device__ void store(uint16_t *p, const float *d) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
    }
};

template <int CPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_moe_small(SmallArgs a) {
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
    // N % 4 == 0 and CPT divides 4: a thread's columns are all in or all out
    const int n = (chunk - a.chunk_start[sg]) * (kThreads * CPT) + CPT * tid;
    const bool live = n < Ns;

    // ---- expand operands: lora_b rows n .. n+CPT-1 (contiguous) and y -----
    const uint16_t *br = static_cast<const uint16_t *>(a.sl.b[sg]) +
                         ((int64_t)(s * a.Eb + (a.Eb == 1 ? 0 : e)) * Ns + (live ? n : 0)) * kRank;
    uint16_t *yp = a.y + (int64_t)p * a.ldy + a.sl.off[sg] + (live ? n : 0);
    // (at 4 columns per thread the lora_b rows are loaded after the shrink's
    // loads: all of them in flight at once would not fit 128 registers)
    constexpr bool kEarlyB = CPT <= 2;
    uint4 bv[2 * CPT];
    if (kEarlyB) {
#pragma unroll
        for (int q = 0; q < 2 * CPT; ++q) bv[q] = ldg<uint4>(br + 8 * q);
    }
    YVec<CPT> yv;
    yv.load(yp);

    // ---- shrink: thread tid takes elements 8 tid + 4096 i of K ------------
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
    if (!kEarlyB) {
#pragma unroll
        for (int q = 0; q < 2 * CPT; ++q) bv[q] = ldg<uint4>(br + 8 * q);
    }
    // wave sums (a fixed order), then the waves in order
#pragma unroll
    for (int j = 0; j < kRank; ++j) acc[j] = wave_sum_f32(acc[j]);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kRank; ++j) s_part[w][j] = acc[j];
    }
    lds_barrier();
    if (tid < kRank) {
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) v += s_part[q][tid];
        s_buf[tid] = tid < r ? v : 0.0f;
    }
    lds_barrier();

    // ---- expand: CPT columns per thread -----------------------------------
    if (!live) return;
    float bj[kRank];
#pragma unroll
    for (int j = 0; j < kRank; ++j) bj[j] = s_buf[j];
    const float c = a.scale[s] * (a.coef ? a.coef[p] : 1.0f);
    float out[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const uint32_t bw[8] = {bv[2 * i].x, bv[2 * i].y, bv[2 * i].z, bv[2 * i].w,
                                bv[2 * i + 1].x, bv[2 * i + 1].y, bv[2 * i + 1].z, bv[2 * i + 1].w};
        float d = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            d = fmaf(bj[2 * q], bf16_lo(bw[q]), d);
            d = fmaf(bj[2 * q + 1], bf16_hi(bw[q]), d);
        }
        out[i] = yv.get(i) + c * d;
    }
    yv.store(yp, out);
}

int chunks_for(const Slices &sl, int S, int cpt, int32_t *start) {
    int c = 0;
    for (int s = 0; s < S; ++s) {
        if (start) start[s] = c;
        c += (int)((sl.n[s] + (int64_t)kThreads * cpt - 1) / ((int64_t)kThreads * cpt));
    }
    return c;
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
    const int64_t pairs = (int64_t)T * top_k;
    if (pairs <= 0) return hipSuccess;
    // the narrowest chunks whose grid holds at most one work-group per CU
    int cpt = 1;
    while (cpt < 4 && pairs * chunks_for(sl, S, cpt, nullptr) > kResident) cpt *= 2;
    const int c = chunks_for(sl, S, cpt, a.chunk_start);
    for (int s = S; s <= kMaxSlices; ++s) a.chunk_start[s] = c;
    a.n_chunks = c;
    const dim3 grid((unsigned)(pairs * c));
    if (cpt == 1) hipLaunchKernelGGL(k_moe_small<1>, grid, dim3(kThreads), 0, st, a);
    else if (cpt == 2) hipLaunchKernelGGL(k_moe_small<2>, grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(k_moe_small<4>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace aa
