// Segment build: stable counting sort of the active tokens by adapter slot,
// plus the per-slot work tiles of the decode and prefill paths.
//
// One work-group of 16 waves.  Wave w owns the contiguous token range
// [w*chunk, (w+1)*chunk).  Pass 1 counts tokens per (wave, slot); a scan over
// slots and then over waves turns the counts into write cursors; pass 2 walks
// the same ranges in order and scatters token ids.  Inside a wave, lanes that
// share a key are found with one ballot per key bit and ranked by lane index,
// so the result is the stable order for any schedule.  The kernel is
// latency-bound, so every global load (keys of up to 16384 items, slot ranks)
// is issued before the first barrier and the rest runs out of registers and
// LDS.
#include "discover.hpp"

namespace aa {

namespace {

constexpr int kSegWaves = kSegThreads / kWave;

// Exclusive scan of one int per thread over the 1024-thread block (DPP wave
// scans, then one over the 16 wave totals).
__device__ int block_exclusive_scan(int v, int *total, int *wsum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
        const int s = lane < kSegWaves ? wsum[lane] : 0;
        const int si = wave_incl_scan(s);
        if (lane < kSegWaves) wsum[kSegWaves + lane] = si - s;   // exclusive wave offsets
        if (lane == kSegWaves - 1) wsum[2 * kSegWaves] = si;       // total
    }
    __syncthreads();
    int r = wsum[kSegWaves + w] + incl - v;
    *total = wsum[2 * kSegWaves];
    __syncthreads();
    return r;
}

// The lanes of a wave whose key equals this lane's (keys in [0, 2^nbits),
// -1 = none): one ballot per key bit, so the cost does not grow with the
// number of distinct keys in the step.
__device__ __forceinline__ uint64_t same_key(int key, int nbits) {
    uint64_t m = __ballot(key >= 0);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return key >= 0 ? m : 0ull;
}

// Counting of one 64-item step of a wave: the lowest lane of each group of
// lanes with the same key adds the group size to the wave's count.
__device__ __forceinline__ void count_step(int s, int nbits, int lane, int32_t *mycnt) {
    const uint64_t peers = same_key(s, nbits);
    if (s >= 0 && lane == __ffsll((unsigned long long)peers) - 1) mycnt[s] += __popcll(peers);
}

// Same grouping; each lane writes its item at the group's cursor plus its
// rank among lower lanes of the group (stable order).  Every lane reads the
// cursor before the group's lowest lane advances it (one instruction each).
__device__ __forceinline__ void scatter_step(int s, int t, int nbits, int lane, int32_t *mycnt,
                                             int32_t *perm) {
    const uint64_t peers = same_key(s, nbits);
    const int pos = s >= 0 ? mycnt[s] : 0;
    if (s >= 0) {
        perm[pos + __popcll(peers & ((1ull << lane) - 1ull))] = t;
        if (lane == __ffsll((unsigned long long)peers) - 1) mycnt[s] = pos + __popcll(peers);
    }
}

constexpr int kSegSpin = 1 << 20;

__device__ __forceinline__ void st_co32(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_co32(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// block_exclusive_scan with barriers that wait for LDS only
__device__ int block_exclusive_scan_lds(int v, int *total, int *wsum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[w] = incl;
    lds_barrier();
    if (w == 0) {
        const int s = lane < kSegWaves ? wsum[lane] : 0;
        const int si = wave_incl_scan(s);
        if (lane < kSegWaves) wsum[kSegWaves + lane] = si - s;
        if (lane == kSegWaves - 1) wsum[2 * kSegWaves] = si;
    }
    lds_barrier();
    int r = wsum[kSegWaves + w] + incl - v;
    *total = wsum[2 * kSegWaves];
    lds_barrier();
    return r;
}

constexpr int kRegSteps = 16;  // 64-item steps per wave held in registers (<= 16384 items)

// Work tiles of both paths (key-major, item ranges of at most the tile size)
// and the header.  Thread tid stands for key tid: cnt items from `start`.
// Every thread of the block calls it.  Its scans use LDS barriers, which do
// not wait for the scatter's stores still in flight.
__device__ void emit_tiles(int cnt, int start, int n_active, int n_invalid, const SegPtrs &seg,
                           int *wsum) {
    const int tid = threadIdx.x;
    int n_dec = 0, n_pre = 0;
    const int td = (cnt + kDecTile - 1) / kDecTile;
    const int tp = (cnt + kPreTile - 1) / kPreTile;
    const int od = block_exclusive_scan_lds(td, &n_dec, wsum);
    const int op = block_exclusive_scan_lds(tp, &n_pre, wsum);
    for (int q = 0; q < td; ++q)
        seg.tiles_dec[od + q] = make_int4(tid, start + q * kDecTile,
                                          min(start + (q + 1) * kDecTile, start + cnt), 0);
    for (int q = 0; q < tp; ++q)
        seg.tiles_pre[op + q] = make_int4(tid, start + q * kPreTile,
                                          min(start + (q + 1) * kPreTile, start + cnt), 0);
    if (tid == 0) {
        seg.header[0] = n_active;
        seg.header[1] = n_invalid;
        seg.header[2] = n_dec;
        seg.header[3] = n_pre;
    }
}

// Items are tokens (topk == nullptr: key = slot of the token) or (token, k)
// pairs p = t * k + j (key = slot(t) * E + topk[p]); nkeys = L or L * E.
__global__ __launch_bounds__(kSegThreads) void k_segments(const int32_t *__restrict__ idx,
                                                          const int32_t *__restrict__ slot_rank,
                                                          const int32_t *__restrict__ topk,
                                                          int32_t k, int32_t E, int32_t T,
                                                          int32_t L, int32_t R, SegPtrs seg) {
    extern __shared__ int32_t lds[];
    const int nkeys = topk ? L * E : L;
    int32_t *wcnt = lds;                       // [kSegWaves][nkeys]
    int32_t *srank = lds + kSegWaves * nkeys;  // [L]
    __shared__ int32_t wsum[2 * kSegWaves + 1];
    __shared__ int32_t s_invalid;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    const int chunk = (T + kSegWaves - 1) / kSegWaves;
    const int b0 = w * chunk;
    const int b1 = min(T, b0 + chunk);
    const int nsteps = b1 > b0 ? (b1 - b0 + kWave - 1) / kWave : 0;
    const bool inreg = chunk <= kWave * kRegSteps;   // uniform over the block

    // Every global load first: the slot indices (and experts) into registers,
    // the ranks into LDS.
    int raw[kRegSteps], rex[kRegSteps];
#pragma unroll
    for (int u = 0; u < kRegSteps; ++u) {
        const int t = b0 + u * kWave + lane;
        const bool in = inreg && t < b1;
        raw[u] = in ? idx[topk ? t / k : t] : -1;
        rex[u] = (in && topk) ? topk[t] : 0;
    }
    for (int i = tid; i < L; i += kSegThreads) srank[i] = slot_rank ? slot_rank[i] : R;
    for (int i = tid; i < kSegWaves * nkeys; i += kSegThreads) wcnt[i] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();

    int inv = 0;
    // key of an item from its slot v and expert e; -1 = carries no adapter
    auto filt = [&](int v, int e) -> int {
        if (v >= L) { ++inv; return -1; }
        if (v < 0 || srank[v] <= 0) return -1;
        if (!topk) return v;
        return (e >= 0 && e < E) ? v * E + e : -1;
    };
    auto key_of = [&](int t) -> int {     // reload path for large item counts
        return filt(idx[topk ? t / k : t], topk ? topk[t] : 0);
    };
    int sl[kRegSteps];
#pragma unroll
    for (int u = 0; u < kRegSteps; ++u) sl[u] = filt(raw[u], rex[u]);
    int32_t *mycnt = wcnt + w * nkeys;

    // Pass 1: per-wave, per-slot counts.
    if (inreg) {
#pragma unroll
        for (int u = 0; u < kRegSteps; ++u)
            if (u < nsteps) count_step(sl[u], nbits, lane, mycnt);
    } else {
        for (int base = b0; base < b1; base += kWave) {
            const int t = base + lane;
            count_step(t < b1 ? key_of(t) : -1, nbits, lane, mycnt);
        }
    }
    if (inv) atomicAdd(&s_invalid, inv);
    __syncthreads();

    // Key totals -> slot_start (one entry per key); per-wave counts -> write cursors.
    int tot = 0;
    if (tid < nkeys)
        for (int q = 0; q < kSegWaves; ++q) tot += wcnt[q * nkeys + tid];
    int n_active = 0;
    const int start = block_exclusive_scan(tot, &n_active, wsum);
    if (tid < nkeys) {
        seg.slot_start[tid] = start;
        int run = start;
        for (int q = 0; q < kSegWaves; ++q) {
            const int c = wcnt[q * nkeys + tid];
            wcnt[q * nkeys + tid] = run;
            run += c;
        }
    }
    if (tid == 0) seg.slot_start[nkeys] = n_active;
    __syncthreads();

    // Pass 2: scatter token ids in stable order.
    if (inreg) {
#pragma unroll
        for (int u = 0; u < kRegSteps; ++u)
            if (u < nsteps) scatter_step(sl[u], b0 + u * kWave + lane, nbits, lane, mycnt, seg.perm);
    } else {
        for (int base = b0; base < b1; base += kWave) {
            const int t = base + lane;
            int kk = -1;
            if (t < b1) {
                const int v = idx[topk ? t / k : t];
                const int e = topk ? topk[t] : 0;
                kk = (v >= 0 && v < L && srank[v] > 0) ? (topk ? ((e >= 0 && e < E) ? v * E + e : -1) : v) : -1;
            }
            scatter_step(kk, t, nbits, lane, mycnt, seg.perm);
        }
    }
    for (int i = n_active + tid; i < T; i += kSegThreads) seg.perm[i] = -1;

    emit_tiles(tid < nkeys ? tot : 0, start, n_active, s_invalid, seg, wsum);
}

// ---- split build for large item counts: one 64-item step per wave --------
// Pass 1: work-group b counts its 1024 items per key into counts[b][key] and
// the slot ids past L into counts[b][nkeys].  Pass 2: every work-group sums
// the counts of all work-groups per key (totals, and the part before its
// own), scans the totals into key starts, recounts its own items per wave and
// scatters them; the order is the single-pass stable order.  Work-group 0
// also writes slot_start, the tail of perm, the tiles and the header.

// Key of an item from its slot v and expert e (keyed: slot * E + expert),
// -1 = carries no adapter; *inv += 1 for a slot id past L.
__device__ __forceinline__ int filt_key(int v, int e, const int32_t *srank, bool keyed, int E, int L,
                                        int *inv) {
    if (v >= L) { ++*inv; return -1; }
    if (v < 0 || srank[v] <= 0) return -1;
    if (!keyed) return v;
    return (e >= 0 && e < E) ? v * E + e : -1;
}

// Work-group blockIdx.x of a split launch: its job and its index in that job.
__device__ __forceinline__ SegJob seg_job(const SegJobs &a, int *b) {
    const bool second = a.n_jobs > 1 && (int)blockIdx.x >= a.job[0].n_wg;
    *b = (int)blockIdx.x - (second ? a.job[0].n_wg : 0);
    return second ? a.job[1] : a.job[0];
}

__global__ __launch_bounds__(kSegThreads) void k_seg_count(SegJobs a) {
    extern __shared__ int32_t lds[];
    int b = 0;
    const SegJob jb = seg_job(a, &b);
    const int L = a.L;
    const int nkeys = jb.topk ? L * jb.E : L;
    int32_t *wcnt = lds;                       // [kSegWaves][nkeys]
    int32_t *srank = lds + kSegWaves * nkeys;  // [L]
    __shared__ int32_t s_invalid;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    const int t = b * kSegThreads + tid;
    const bool in = t < jb.n_items;
    const int v = in ? a.idx[jb.topk ? t / jb.k : t] : -1;
    const int e = (in && jb.topk) ? jb.topk[t] : 0;
    for (int i = tid; i < L; i += kSegThreads) srank[i] = a.slot_rank ? a.slot_rank[i] : a.R;
    for (int i = tid; i < kSegWaves * nkeys; i += kSegThreads) wcnt[i] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();
    int inv = 0;
    const int key = filt_key(v, e, srank, jb.topk != nullptr, jb.E, L, &inv);
    count_step(key, nbits, lane, wcnt + w * nkeys);
    if (inv) atomicAdd(&s_invalid, inv);
    __syncthreads();
    int32_t *mine = jb.counts + (int64_t)b * (nkeys + 1);
    for (int kk = tid; kk < nkeys; kk += kSegThreads) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < kSegWaves; ++q) c += wcnt[q * nkeys + kk];
        mine[kk] = c;
    }
    if (tid == 0) mine[nkeys] = s_invalid;
}

__global__ __launch_bounds__(kSegThreads) void k_seg_place(SegJobs a) {
    extern __shared__ int32_t lds[];
    int b = 0;
    const SegJob jb = seg_job(a, &b);
    const int L = a.L;
    const int nkeys = jb.topk ? L * jb.E : L;  // <= kSegThreads
    const int n_wg = jb.n_wg;
    const SegPtrs &seg = jb.seg;
    int32_t *wcnt = lds;                       // [kSegWaves][nkeys]
    int32_t *srank = lds + kSegWaves * nkeys;  // [L]
    __shared__ int32_t wsum[2 * kSegWaves + 1];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    const int t = b * kSegThreads + tid;
    const bool in = t < jb.n_items;
    const int v = in ? a.idx[jb.topk ? t / jb.k : t] : -1;
    const int e = (in && jb.topk) ? jb.topk[t] : 0;
    // Column col of the counts (a key, or nkeys: the invalid ids) summed over
    // all work-groups, and over those before this one; 16 loads in flight.
    auto col_sums = [&](int col, int &all, int &pre) {
        all = 0; pre = 0;
        for (int q0 = 0; q0 < n_wg; q0 += 16) {
            int c[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) c[u] = jb.counts[(int64_t)min(q0 + u, n_wg - 1) * (nkeys + 1) + col];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (q0 + u < n_wg) { all += c[u]; pre += q0 + u < b ? c[u] : 0; }
        }
    };
    int tot = 0, before = 0, n_inv = 0, unused = 0;
    if (tid < nkeys) col_sums(tid, tot, before);
    if (tid == 0 && b == 0) col_sums(nkeys, n_inv, unused);
    for (int i = tid; i < L; i += kSegThreads) srank[i] = a.slot_rank ? a.slot_rank[i] : a.R;
    for (int i = tid; i < kSegWaves * nkeys; i += kSegThreads) wcnt[i] = 0;
    __syncthreads();
    int inv = 0;
    const int key = filt_key(v, e, srank, jb.topk != nullptr, jb.E, L, &inv);
    int32_t *mycnt = wcnt + w * nkeys;
    count_step(key, nbits, lane, mycnt);
    int n_active = 0;
    const int start = block_exclusive_scan(tid < nkeys ? tot : 0, &n_active, wsum);   // has barriers
    if (tid < nkeys) {
        int run = start + before;
        for (int q = 0; q < kSegWaves; ++q) {
            const int c = wcnt[q * nkeys + tid];
            wcnt[q * nkeys + tid] = run;
            run += c;
        }
        if (b == 0) seg.slot_start[tid] = start;
    }
    if (b == 0 && tid == 0) seg.slot_start[nkeys] = n_active;
    __syncthreads();
    scatter_step(key, t, nbits, lane, mycnt, seg.perm);
    if (b != 0) return;   // uniform: work-group 0 of each job writes the rest
    for (int i = n_active + tid; i < jb.n_items; i += kSegThreads) seg.perm[i] = -1;
    emit_tiles(tid < nkeys ? tot : 0, start, n_active, n_inv, seg, wsum);
}

// ---- single-launch build for up to kSegOneMaxWg work-groups per job -------
// The two passes above in one launch: each work-group counts its 1024 items
// per key, publishes the counts (stored plus one, so that zero means "not
// written yet", through agent-scope relaxed atomic stores), then reads every
// work-group's counts (the loads repeat while any is zero, bounded: past
// kSegSpin polls the workspace's error word is set and the build goes on),
// and places its items as the second pass does.  The last work-group to have
// read them (a done counter) writes the counts and the counter back to zero.
// Every work-group waits for all of its job's work-groups, so a launch has at
// most 2 * kSegOneMaxWg work-groups of 1024 threads, resident together on any
// GPU that is not full.  After the counts are published only LDS barriers
// are used (a block barrier would also wait for the stores).

__global__ __launch_bounds__(kSegThreads) void k_seg_one(SegJobs a) {
    extern __shared__ int32_t lds[];
    int b = 0;
    const SegJob jb = seg_job(a, &b);
    const int L = a.L;
    const int nkeys = jb.topk ? L * jb.E : L;  // <= kSegThreads
    const int n_wg = jb.n_wg;                  // <= kSegOneMaxWg
    const SegPtrs &seg = jb.seg;
    int32_t *wcnt = lds;                       // [kSegWaves][nkeys]
    int32_t *srank = lds + kSegWaves * nkeys;  // [L]
    __shared__ int32_t wsum[2 * kSegWaves + 1];
    __shared__ int32_t s_invalid, s_last;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    const int t = b * kSegThreads + tid;
    const bool in = t < jb.n_items;
    const int v = in ? a.idx[jb.topk ? t / jb.k : t] : -1;
    const int e = (in && jb.topk) ? jb.topk[t] : 0;
    for (int i = tid; i < L; i += kSegThreads) srank[i] = a.slot_rank ? a.slot_rank[i] : a.R;
    for (int i = tid; i < kSegWaves * nkeys; i += kSegThreads) wcnt[i] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();
    int inv = 0;
    const int key = filt_key(v, e, srank, jb.topk != nullptr, jb.E, L, &inv);
    int32_t *mycnt = wcnt + w * nkeys;
    count_step(key, nbits, lane, mycnt);
    if (inv) atomicAdd(&s_invalid, inv);
    __syncthreads();

    // publish this work-group's counts per key, and its slot ids past L
    const int stride = nkeys + 1;
    for (int kk = tid; kk < nkeys; kk += kSegThreads) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < kSegWaves; ++q) c += wcnt[q * nkeys + kk];
        st_co32(seg.xcounts + (int64_t)b * stride + kk, c + 1);
    }
    if (tid == 0) st_co32(seg.xcounts + (int64_t)b * stride + nkeys, s_invalid + 1);

    // Column col of every work-group's counts: the sum over all, and over
    // those before this one.
    auto col_sums = [&](int col, int &all, int &pre) {
        int c[kSegOneMaxWg];
        for (int n = 0;; ++n) {
            bool ok = true;
#pragma unroll
            for (int u = 0; u < kSegOneMaxWg; ++u) {
                c[u] = ld_co32(seg.xcounts + (int64_t)min(u, n_wg - 1) * stride + col);
                ok = ok && c[u] != 0;
            }
            if (ok) break;
            if (n >= kSegSpin) {
                st_co32(seg.err, 1);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        all = 0; pre = 0;
#pragma unroll
        for (int u = 0; u < kSegOneMaxWg; ++u)
            if (u < n_wg) { all += c[u] - 1; pre += u < b ? c[u] - 1 : 0; }
    };
    int tot = 0, before = 0, n_inv = 0, unused = 0;
    if (tid < nkeys) col_sums(tid, tot, before);
    if (tid == 0 && b == 0) col_sums(nkeys, n_inv, unused);
    lds_barrier();
    // every thread of this work-group has read the counts; the count of such
    // work-groups is used only at the end
    int done = 0;
    if (tid == 0) done = __hip_atomic_fetch_add(seg.xdone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    int n_active = 0;
    const int start = block_exclusive_scan_lds(tid < nkeys ? tot : 0, &n_active, wsum);
    if (tid < nkeys) {
        int run = start + before;
        for (int q = 0; q < kSegWaves; ++q) {
            const int c = wcnt[q * nkeys + tid];
            wcnt[q * nkeys + tid] = run;
            run += c;
        }
        if (b == 0) seg.slot_start[tid] = start;
    }
    if (b == 0 && tid == 0) seg.slot_start[nkeys] = n_active;
    lds_barrier();
    scatter_step(key, t, nbits, lane, mycnt, seg.perm);
    if (b == 0) {
        // work-group 0 of the job: the tail of perm, the tiles and the header
        for (int i = n_active + tid; i < jb.n_items; i += kSegThreads) seg.perm[i] = -1;
        emit_tiles(tid < nkeys ? tot : 0, start, n_active, n_inv, seg, wsum);
    }
    // the last work-group to have read the counts zeroes them for the next call
    if (tid == 0) s_last = done == n_wg - 1;
    lds_barrier();
    if (s_last) {
        for (int i = tid; i < n_wg * stride; i += kSegThreads) st_co32(seg.xcounts + i, 0);
        if (tid == 0) st_co32(seg.xdone, 0);
    }
}

__global__ void k_fill_zero(uint4 *__restrict__ p, size_t n16, uint8_t *__restrict__ tail,
                            size_t ntail) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0)
        for (size_t k = threadIdx.x; k < ntail; k += blockDim.x) tail[k] = 0;
}

}  // namespace

hipError_t launch_segments(const int32_t *idx, const int32_t *slot_rank, int32_t T, int32_t L,
                           int32_t R, const SegPtrs &seg, hipStream_t st) {
    return launch_segments_keyed(idx, slot_rank, nullptr, 1, 1, T, L, R, seg, st);
}

hipError_t launch_segments_keyed(const int32_t *idx, const int32_t *slot_rank,
                                 const int32_t *topk, int32_t k, int32_t E, int32_t n_items,
                                 int32_t L, int32_t R, const SegPtrs &seg, hipStream_t st) {
    const int nkeys = topk ? L * E : L;
    const size_t lds = sizeof(int32_t) * ((size_t)kSegWaves * nkeys + L);
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_segments),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (n_items > kSegSplitItems && seg.counts) {
        const SegJob job = seg_job_of(topk, k, E, n_items, seg);
        return launch_segments_split(idx, slot_rank, L, R, &job, 1, st);
    }
    hipLaunchKernelGGL(k_segments, dim3(1), dim3(kSegThreads), lds, st, idx, slot_rank, topk, k, E,
                       n_items, L, R, seg);
    return hipGetLastError();
}

SegJob seg_job_of(const int32_t *topk, int32_t k, int32_t E, int32_t n_items, const SegPtrs &seg) {
    SegJob j{};
    j.topk = topk;
    j.k = k;
    j.E = E;
    j.n_items = n_items;
    j.n_wg = n_items > 0 ? (n_items + kSegThreads - 1) / kSegThreads : 1;
    j.counts = seg.counts;
    j.seg = seg;
    return j;
}

hipError_t launch_segments_split(const int32_t *idx, const int32_t *slot_rank, int32_t L, int32_t R,
                                 const SegJob *jobs, int n_jobs, hipStream_t st) {
    SegJobs a{};
    a.idx = idx; a.slot_rank = slot_rank; a.L = L; a.R = R; a.n_jobs = n_jobs;
    size_t lds = 0;
    int n_wg = 0;
    for (int j = 0; j < n_jobs; ++j) {
        a.job[j] = jobs[j];
        const int nkeys = jobs[j].topk ? L * jobs[j].E : L;
        const size_t l = sizeof(int32_t) * ((size_t)kSegWaves * nkeys + L);
        lds = l > lds ? l : lds;
        n_wg += jobs[j].n_wg;
    }
    if (lds > 48 * 1024) {
        for (const void *f : {reinterpret_cast<const void *>(k_seg_count),
                              reinterpret_cast<const void *>(k_seg_place)}) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
    }
    // one launch when every job has its exchange region (and so at most
    // kSegOneMaxWg work-groups), else count and place apart
    bool one = true;
    for (int j = 0; j < n_jobs; ++j)
        one = one && jobs[j].seg.xcounts && jobs[j].seg.xdone && jobs[j].seg.err &&
              jobs[j].n_wg <= kSegOneMaxWg;
    if (one) {
        if (lds > 48 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_seg_one),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_seg_one, dim3(n_wg), dim3(kSegThreads), lds, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_seg_count, dim3(n_wg), dim3(kSegThreads), lds, st, a);
    hipLaunchKernelGGL(k_seg_place, dim3(n_wg), dim3(kSegThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const size_t ntail = bytes - n16 * 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<uint4 *>(p), n16, static_cast<uint8_t *>(p) + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace aa
