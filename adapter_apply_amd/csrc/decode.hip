// Decode path: VALU kernels for short per-slot token runs (BGMV regime).
//
// Tokens are grouped by slot into tiles of at most 32 (the segment build), so
// a slot's lora_a / lora_b rows are streamed from HBM once per tile instead of
// once per token.  No MFMA: dot products use packed bf16 dot instructions
// (fp32 accumulate) and one cross-lane add.
//
// Shrink (buf = x . A^T): work-group = (tile, 256-column K chunk, 16 rows of
// the slot's (slice, rank) rows).  Lane = (token, column half); each wave owns
// 64 columns, so every lane holds 32 x values in registers and streams the
// rank rows from LDS (broadcast reads).  Partial sums of the K chunks go to
// the workspace and are added, in ascending chunk order (deterministic), by a
// later kernel: the reduce kernel, or the expand itself when the partials of
// a tile are few.  The kernel boundary is the only synchronisation: an
// agent-scope release per work-group writes back the whole L2 on this part
// and costs about a microsecond each.
//
// Expand (y += scale * buf . B^T): work-group = (tile, 128 output columns of
// one slice).  Lane = 2 adjacent columns, waves split the tile's tokens; the
// lane's B rows live in registers (rank in chunks of 32), buf rows in LDS.
#include "common.hpp"

namespace aa {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWg = kThreads / kWave;
constexpr int kColsPerWave = kDecKc / kWavesPerWg;     // 64
constexpr int kColsPerLane = kColsPerWave / 2;         // 32
constexpr int kExpCols = 128;                          // columns per expand work-group
constexpr int kRankChunk = 32;

struct ShrinkArgs {
    const void *x;
    int64_t ldx;
    int32_t T, K, S, L, R, n_kchunks, n_rg;
    const int32_t *slot_rank;
    SegPtrs seg;
    Slices sl;
    float *partial;   // [n_kchunks][T][S][R]
    float *buf;       // [S][T][R]
};

struct ExpandArgs {
    void *y;
    int64_t ldy;
    const float *buf;       // [S][T][R], or
    const float *partial;   // [n_kchunks][T][S][R] K-chunk partials summed here when non-null
    int32_t n_kchunks;      // upper bound on the chunk count (the shrink records the real one)
    int32_t T, S, L, R;
    const int32_t *slot_rank;
    const float *scale;
    SegPtrs seg;
    Slices sl;
    int32_t chunk_start[kMaxSlices + 1];
};

template <bool BF16> struct Elt;
template <> struct Elt<true> {
    typedef uint16_t T;
    static constexpr int kPerVec = 8;   // elements per 16-byte vector
};
template <> struct Elt<false> {
    typedef float T;
    static constexpr int kPerVec = 4;
};

__device__ __forceinline__ float dot_vec(const uint4 &x, const uint4 &a, float acc, bool) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.x),
                                          __builtin_bit_cast(bf16x2_t, a.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.y),
                                          __builtin_bit_cast(bf16x2_t, a.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.z),
                                          __builtin_bit_cast(bf16x2_t, a.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.w),
                                          __builtin_bit_cast(bf16x2_t, a.w), acc, false);
    return acc;
}

__device__ __forceinline__ float dot_vec(const float4 &x, const float4 &a, float acc, int) {
    acc = fmaf(x.x, a.x, acc);
    acc = fmaf(x.y, a.y, acc);
    acc = fmaf(x.z, a.z, acc);
    acc = fmaf(x.w, a.w, acc);
    return acc;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dec_shrink(ShrinkArgs a) {
    typedef typename Elt<BF16>::T E;
    typedef typename std::conditional<BF16, uint4, float4>::type V;
    constexpr int EPV = Elt<BF16>::kPerVec;
    constexpr int VPL = kColsPerLane / EPV;     // vectors per lane (4 bf16, 8 fp32)
    constexpr int VPR = kDecKc / EPV;           // vectors per A row chunk

    const int kc = blockIdx.x;
    const int g = blockIdx.y;
    const int tile = blockIdx.z;
    if ((kc | g | tile) == 0 && threadIdx.x == 0) a.seg.header[4] = a.n_kchunks;
    if (tile >= a.seg.header[2]) return;
    const int4 tl = a.seg.tiles_dec[tile];
    const int s = tl.x, p0 = tl.y, ntok = tl.z - tl.y;
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    const int SR = a.S * r;
    const int q0 = g * kDecRows;
    if (q0 >= SR) return;
    const int nrows = min(kDecRows, SR - q0);
    const int k0 = kc * kDecKc;

    __shared__ __attribute__((aligned(16))) E sA[kDecRows][kDecKc];
    __shared__ float sRed[kWavesPerWg][kDecRows][32];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    // Stage the rank rows of this chunk (rows past nrows or columns past K are zero).
    for (int v = tid; v < kDecRows * VPR; v += kThreads) {
        const int row = v / VPR, cv = v - row * VPR;
        const int col = k0 + cv * EPV;
        V val = {};
        if (row < nrows && col < a.K) {
            const int q = q0 + row;
            const int sg = q / r, j = q - sg * r;
            const E *src = static_cast<const E *>(a.sl.a[sg]) +
                           (((int64_t)s * a.R + j) * a.K + col);
            val = *reinterpret_cast<const V *>(src);
        }
        *reinterpret_cast<V *>(&sA[row][cv * EPV]) = val;
    }

    // This lane's 32 columns of its token's x row.
    const int tok = lane & 31, h = lane >> 5;
    const int cbase = w * kColsPerWave + h * kColsPerLane;
    V xv[VPL];
    {
        const bool live = tok < ntok;
        const int t = live ? a.seg.perm[p0 + tok] : 0;
        const E *xr = static_cast<const E *>(a.x) + (int64_t)t * a.ldx;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int col = k0 + cbase + v * EPV;
            V val = {};
            if (live && col < a.K) val = *reinterpret_cast<const V *>(xr + col);
            xv[v] = val;
        }
    }
    __syncthreads();

#pragma unroll
    for (int row = 0; row < kDecRows; ++row) {
        if (row < nrows) {
            const V *ar = reinterpret_cast<const V *>(&sA[row][cbase]);
            float acc = 0.0f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) acc = dot_vec(xv[v], ar[v], acc, 0);
            acc += __shfl_xor(acc, 32);
            if (h == 0) sRed[w][row][tok] = acc;
        }
    }
    __syncthreads();

    // Combine the four waves' column ranges and store this chunk's partial sums.
    const int64_t pstride = (int64_t)a.S * a.R;
    float *part = a.partial + ((int64_t)kc * a.T + p0) * pstride;
    for (int i = tid; i < ntok * nrows; i += kThreads) {
        const int tk = i / nrows, row = i - tk * nrows;
        const float v = ((sRed[0][row][tk] + sRed[1][row][tk]) + sRed[2][row][tk]) + sRed[3][row][tk];
        const int q = q0 + row;
        const int sg = q / r, j = q - sg * r;
        part[(int64_t)tk * pstride + (int64_t)sg * a.R + j] = v;
    }

}

// Sum of the K-chunk partials of one (tile, row group) into buf, chunks in
// ascending order (deterministic).
__global__ __launch_bounds__(kThreads) void k_dec_reduce(ShrinkArgs a) {
    const int g = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= a.seg.header[2]) return;
    const int4 tl = a.seg.tiles_dec[tile];
    const int s = tl.x, p0 = tl.y, ntok = tl.z - tl.y;
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    const int q0 = g * kDecRows;
    if (q0 >= a.S * r) return;
    const int nrows = min(kDecRows, a.S * r - q0);
    const int64_t pstride = (int64_t)a.S * a.R;
    const int64_t cstride = (int64_t)a.T * pstride;
    for (int i = threadIdx.x; i < ntok * nrows; i += kThreads) {
        const int tk = i / nrows, row = i - tk * nrows;
        const int q = q0 + row;
        const int sg = q / r, j = q - sg * r;
        const float *pp = a.partial + (int64_t)(p0 + tk) * pstride + (int64_t)sg * a.R + j;
        float acc = 0.0f;
        int c = 0;
        for (; c + 8 <= a.n_kchunks; c += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = pp[(int64_t)(c + u) * cstride];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
        for (; c < a.n_kchunks; ++c) acc += pp[(int64_t)c * cstride];
        const int t = a.seg.perm[p0 + tk];
        a.buf[((int64_t)sg * a.T + t) * a.R + j] = acc;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dec_expand(ExpandArgs a) {
    typedef typename Elt<BF16>::T E;
    constexpr int EPV = Elt<BF16>::kPerVec;
    constexpr int VPC = kRankChunk / EPV;       // vectors per rank chunk per column
    constexpr int TOK_PER_WAVE = kDecTile / kWavesPerWg;   // 8

    const int chunk = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= a.seg.header[2]) return;
    const int4 tl = a.seg.tiles_dec[tile];
    const int s = tl.x, p0 = tl.y, ntok = tl.z - tl.y;
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    // K chunks written by the shrink, bounded by what the workspace holds
    const int nkc = a.partial ? min(a.seg.header[4], a.n_kchunks) : 0;
    int sg = 0;
    while (sg + 1 < a.S && chunk >= a.chunk_start[sg + 1]) ++sg;
    const int64_t Ns = a.sl.n[sg];
    const int n0 = (chunk - a.chunk_start[sg]) * kExpCols;
    const float sc = a.scale[s];

    extern __shared__ float sBuf[];   // [kDecTile][rpad]
    const int rpad = (r + kRankChunk - 1) / kRankChunk * kRankChunk;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kDecTile * rpad; i += kThreads) {
        const int tk = i / rpad, j = i - tk * rpad;
        float v = 0.0f;
        if (tk < ntok && j < r) {
            if (a.partial) {
                const int64_t pstride = (int64_t)a.S * a.R;
                const int64_t cstride = (int64_t)a.T * pstride;
                const float *pp = a.partial + (int64_t)(p0 + tk) * pstride + (int64_t)sg * a.R + j;
                for (int c = 0; c < nkc; ++c) v += pp[(int64_t)c * cstride];
            } else {
                const int t = a.seg.perm[p0 + tk];
                v = a.buf[((int64_t)sg * a.T + t) * a.R + j];
            }
        }
        sBuf[i] = v;
    }
    __syncthreads();

    const int n = n0 + 2 * lane;
    const bool col_ok = n < Ns;
    const E *brow0 = static_cast<const E *>(a.sl.b[sg]) + ((int64_t)s * Ns + (col_ok ? n : 0)) * a.R;
    const E *brow1 = brow0 + a.R;

    float acc[TOK_PER_WAVE][2];
#pragma unroll
    for (int i = 0; i < TOK_PER_WAVE; ++i) acc[i][0] = acc[i][1] = 0.0f;

    for (int j0 = 0; j0 < r; j0 += kRankChunk) {
        const int nv = min(VPC, (r - j0 + EPV - 1) / EPV);
        float b0[kRankChunk], b1[kRankChunk];
#pragma unroll
        for (int v = 0; v < VPC; ++v) {
            if (v < nv && col_ok) {
                if constexpr (BF16) {
                    const uint4 u0 = *reinterpret_cast<const uint4 *>(brow0 + j0 + v * 8);
                    const uint4 u1 = *reinterpret_cast<const uint4 *>(brow1 + j0 + v * 8);
                    const uint32_t w0[4] = {u0.x, u0.y, u0.z, u0.w};
                    const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b0[v * 8 + 2 * e] = bf16_lo(w0[e]);
                        b0[v * 8 + 2 * e + 1] = bf16_hi(w0[e]);
                        b1[v * 8 + 2 * e] = bf16_lo(w1[e]);
                        b1[v * 8 + 2 * e + 1] = bf16_hi(w1[e]);
                    }
                } else {
                    const float4 f0 = *reinterpret_cast<const float4 *>(brow0 + j0 + v * 4);
                    const float4 f1 = *reinterpret_cast<const float4 *>(brow1 + j0 + v * 4);
                    b0[v * 4 + 0] = f0.x; b0[v * 4 + 1] = f0.y; b0[v * 4 + 2] = f0.z; b0[v * 4 + 3] = f0.w;
                    b1[v * 4 + 0] = f1.x; b1[v * 4 + 1] = f1.y; b1[v * 4 + 2] = f1.z; b1[v * 4 + 3] = f1.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) b0[v * EPV + e] = b1[v * EPV + e] = 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < TOK_PER_WAVE; ++i) {
            const int tk = w * TOK_PER_WAVE + i;
            const float4 *bb = reinterpret_cast<const float4 *>(sBuf + tk * rpad + j0);
#pragma unroll
            for (int v4 = 0; v4 < kRankChunk / 4; ++v4) {
                if (v4 * 4 < nv * EPV) {
                    const float4 q = bb[v4];
                    acc[i][0] = fmaf(q.x, b0[v4 * 4 + 0], acc[i][0]);
                    acc[i][1] = fmaf(q.x, b1[v4 * 4 + 0], acc[i][1]);
                    acc[i][0] = fmaf(q.y, b0[v4 * 4 + 1], acc[i][0]);
                    acc[i][1] = fmaf(q.y, b1[v4 * 4 + 1], acc[i][1]);
                    acc[i][0] = fmaf(q.z, b0[v4 * 4 + 2], acc[i][0]);
                    acc[i][1] = fmaf(q.z, b1[v4 * 4 + 2], acc[i][1]);
                    acc[i][0] = fmaf(q.w, b0[v4 * 4 + 3], acc[i][0]);
                    acc[i][1] = fmaf(q.w, b1[v4 * 4 + 3], acc[i][1]);
                }
            }
        }
    }

    if (!col_ok) return;
    const int64_t col = a.sl.off[sg] + n;
#pragma unroll
    for (int i = 0; i < TOK_PER_WAVE; ++i) {
        const int tk = w * TOK_PER_WAVE + i;
        if (tk < ntok) {
            const int t = a.seg.perm[p0 + tk];
            E *yp = static_cast<E *>(a.y) + (int64_t)t * a.ldy + col;
            if constexpr (BF16) {
                const uint32_t yv = *reinterpret_cast<const uint32_t *>(yp);
                const float lo = bf16_lo(yv) + sc * acc[i][0];
                const float hi = bf16_hi(yv) + sc * acc[i][1];
                *reinterpret_cast<uint32_t *>(yp) = pack_bf16x2(lo, hi);
            } else {
                float2 yv = *reinterpret_cast<const float2 *>(yp);
                yv.x = yv.x + sc * acc[i][0];
                yv.y = yv.y + sc * acc[i][1];
                *reinterpret_cast<float2 *>(yp) = yv;
            }
        }
    }
}

// Single launch for tiny batches: work-group = (token, 256 output columns of
// one slice).  Each work-group computes its token's shrink for its slice,
// x[t] . A[s][j]^T for the slot's r rank rows (wave w takes rows w, w + 4, ...,
// four at a time; lanes over K, 16 bytes each, then a fixed-order wave sum),
// into LDS; then
// each thread adds one column, y[t][n] += scale[s] * sum_j buf[j] * B[s][n][j]
// (j ascending).  The y value and the first lora_b vectors of the column are
// loaded before the shrink.  No segment build, no workspace: the shrink is
// recomputed by every column chunk of a token, which the host allows only
// for a few tokens and a small K * R.
constexpr int kTokCols = kTokenCols;   // output columns per work-group, one per thread
static_assert(kTokCols == kThreads, "one column per thread");
constexpr int kTokPreVecs = 2;         // lora_b vectors per column loaded before the shrink
constexpr int kTokRows = 4;            // rank rows a wave's shrink takes at once

struct TokenArgs {
    void *y;
    int64_t ldy;
    const void *x;
    int64_t ldx;
    int32_t K, L, R, S, n_chunks;
    const int32_t *idx;
    const int32_t *slot_rank;
    const float *scale;
    Slices sl;
    int32_t chunk_start[kMaxSlices + 1];
};

__device__ __forceinline__ float vec_elt(const uint4 &v, int i) {
    const uint32_t w = i < 4 ? (i < 2 ? v.x : v.y) : (i < 6 ? v.z : v.w);
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
}
__device__ __forceinline__ float vec_elt(const float4 &v, int i) {
    return i < 2 ? (i ? v.y : v.x) : (i == 2 ? v.z : v.w);
}
__device__ __forceinline__ float elt_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float elt_f32(float v) { return v; }
__device__ __forceinline__ void elt_store(uint16_t *p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }
__device__ __forceinline__ void elt_store(float *p, float v) { *p = v; }

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dec_token(TokenArgs a) {
    typedef typename Elt<BF16>::T E;
    typedef typename std::conditional<BF16, uint4, float4>::type V;
    constexpr int EPV = Elt<BF16>::kPerVec;
    __shared__ float s_tb[kMaxRank];
    const int t = blockIdx.x / a.n_chunks;
    const int chunk = blockIdx.x - t * a.n_chunks;
    const int s = a.idx[t];
    if (s < 0 || s >= a.L) return;                       // uniform: no adapter
    const int r = a.slot_rank ? min(a.slot_rank[s], a.R) : a.R;
    if (r <= 0) return;
    int sg = 0;
    while (sg + 1 < a.S && chunk >= a.chunk_start[sg + 1]) ++sg;
    const int Ns = (int)a.sl.n[sg];
    const int n = (chunk - a.chunk_start[sg]) * kTokCols + threadIdx.x;
    const bool live = n < Ns;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    // the column's y value and first lora_b vectors (clamped: column 0, and
    // the row's last vector needed)
    E *yp = static_cast<E *>(a.y) + (int64_t)t * a.ldy + a.sl.off[sg] + (live ? n : 0);
    const E y0 = *yp;
    const E *br = static_cast<const E *>(a.sl.b[sg]) + ((int64_t)s * Ns + (live ? n : 0)) * a.R;
    const int nvec = (r + EPV - 1) / EPV;
    V bpre[kTokPreVecs];
#pragma unroll
    for (int q = 0; q < kTokPreVecs; ++q) bpre[q] = ldg<V>(br + EPV * min(q, nvec - 1));

    // ---- shrink --------------------------------------------------------
    const E *xr = static_cast<const E *>(a.x) + (int64_t)t * a.ldx;
    const E *ar = static_cast<const E *>(a.sl.a[sg]) + (int64_t)s * a.R * a.K;
    // wave w takes rank rows w + 4 i, kTokRows at a time (one x load feeds
    // them; rows past r repeat row r - 1 and are not written)
    for (int j0 = w; j0 < r; j0 += kTokRows * kWavesPerWg) {
        const E *arow[kTokRows];
        float acc[kTokRows];
#pragma unroll
        for (int i = 0; i < kTokRows; ++i) {
            arow[i] = ar + (int64_t)min(j0 + i * kWavesPerWg, r - 1) * a.K;
            acc[i] = 0.0f;
        }
#pragma unroll 4
        for (int k0 = EPV * lane; k0 < a.K; k0 += EPV * kWave) {
            const V xv = ldg<V>(xr + k0);
            V av[kTokRows];
#pragma unroll
            for (int i = 0; i < kTokRows; ++i) av[i] = ldg<V>(arow[i] + k0);
#pragma unroll
            for (int i = 0; i < kTokRows; ++i) acc[i] = dot_vec(xv, av[i], acc[i], 0);
        }
#pragma unroll
        for (int i = 0; i < kTokRows; ++i) {
            const int j = j0 + i * kWavesPerWg;
            if (j < r) {                                 // uniform over the wave
                const float v = wave_sum_f32(acc[i]);
                if (lane == 0) s_tb[j] = v;
            }
        }
    }
    __syncthreads();

    // ---- expand: one column per thread ------------------------------------
    if (!live) return;
    float d = 0.0f;
#pragma unroll
    for (int q = 0; q < kTokPreVecs; ++q)
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            const int j = EPV * q + i;
            if (j < r) d = fmaf(s_tb[j], vec_elt(bpre[q], i), d);
        }
    for (int q = kTokPreVecs; q < nvec; ++q) {
        const V bv = ldg<V>(br + EPV * q);
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            const int j = EPV * q + i;
            if (j < r) d = fmaf(s_tb[j], vec_elt(bv, i), d);
        }
    }
    elt_store(yp, elt_f32(y0) + a.scale[s] * d);
}

}  // namespace

hipError_t launch_dec_token(int dtype, void *y, int64_t ldy, const void *x, int64_t ldx, int32_t T,
                            int32_t K, const Slices &sl, int32_t S, int32_t L, int32_t R,
                            const int32_t *idx, const int32_t *slot_rank, const float *scale,
                            hipStream_t st) {
    TokenArgs a{};
    a.y = y; a.ldy = ldy; a.x = x; a.ldx = ldx; a.K = K; a.L = L; a.R = R; a.S = S;
    a.idx = idx; a.slot_rank = slot_rank; a.scale = scale; a.sl = sl;
    int c = 0;
    for (int s = 0; s < S; ++s) {
        a.chunk_start[s] = c;
        c += (int)((sl.n[s] + kTokCols - 1) / kTokCols);
    }
    for (int s = S; s <= kMaxSlices; ++s) a.chunk_start[s] = c;
    a.n_chunks = c;
    const int64_t grid = (int64_t)T * c;
    if (grid <= 0) return hipSuccess;
    if (dtype == 1)
        hipLaunchKernelGGL(k_dec_token<true>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_dec_token<false>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_dec_shrink(int dtype, const void *x, int64_t ldx, int32_t T, int32_t K,
                             const Slices &sl, int32_t S, int32_t L, int32_t R,
                             const int32_t *slot_rank, const SegPtrs &seg, float *partial,
                             int32_t n_kchunks, hipStream_t st) {
    ShrinkArgs a{};
    a.x = x; a.ldx = ldx; a.T = T; a.K = K; a.S = S; a.L = L; a.R = R;
    a.n_kchunks = n_kchunks;
    a.n_rg = row_groups(S, R);
    a.slot_rank = slot_rank; a.seg = seg; a.sl = sl; a.partial = partial; a.buf = nullptr;
    dim3 grid(n_kchunks, a.n_rg, seg.max_tiles_dec);
    if (dtype == 1)
        hipLaunchKernelGGL(k_dec_shrink<true>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_dec_shrink<false>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_dec_reduce(int32_t T, int32_t S, int32_t L, int32_t R,
                             const int32_t *slot_rank, const SegPtrs &seg, const float *partial,
                             int32_t n_kchunks, float *buf, hipStream_t st) {
    ShrinkArgs a{};
    a.T = T; a.S = S; a.L = L; a.R = R; a.n_kchunks = n_kchunks; a.n_rg = row_groups(S, R);
    a.slot_rank = slot_rank; a.seg = seg; a.partial = const_cast<float *>(partial); a.buf = buf;
    hipLaunchKernelGGL(k_dec_reduce, dim3(a.n_rg, seg.max_tiles_dec), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_dec_expand(int dtype, void *y, int64_t ldy, const float *buf,
                             const float *partial, int32_t n_kchunks, int32_t T,
                             const Slices &sl, int32_t S, int32_t L, int32_t R,
                             const int32_t *slot_rank, const float *scale, const SegPtrs &seg,
                             hipStream_t st) {
    ExpandArgs a;
    a.y = y; a.ldy = ldy; a.buf = buf; a.partial = partial; a.n_kchunks = n_kchunks;
    a.T = T; a.S = S; a.L = L; a.R = R;
    a.slot_rank = slot_rank; a.scale = scale; a.seg = seg; a.sl = sl;
    int c = 0;
    for (int s = 0; s < S; ++s) {
        a.chunk_start[s] = c;
        c += (int)((sl.n[s] + kExpCols - 1) / kExpCols);
    }
    for (int s = S; s <= kMaxSlices; ++s) a.chunk_start[s] = c;
    const int rpad = (R + kRankChunk - 1) / kRankChunk * kRankChunk;
    const size_t lds = sizeof(float) * (size_t)kDecTile * rpad;
    dim3 grid(c, seg.max_tiles_dec);
    if (lds > 48 * 1024) {
        const void *fn = dtype == 1 ? reinterpret_cast<const void *>(k_dec_expand<true>)
                                    : reinterpret_cast<const void *>(k_dec_expand<false>);
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (dtype == 1)
        hipLaunchKernelGGL(k_dec_expand<true>, grid, dim3(kThreads), lds, st, a);
    else
        hipLaunchKernelGGL(k_dec_expand<false>, grid, dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace aa
