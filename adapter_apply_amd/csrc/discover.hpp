// Token-group discovery inside a work-group.
//
// A group is a run of at most G tokens of one slot in the order a stable sort
// of the active tokens by slot gives ([SGL] header credit to S-LoRA/Punica:
// the tokens of one adapter are gathered into a segment).  Group ids are
// slot-major: slot 0's groups first.  Every work-group of the decode kernels
// derives its own group from idx, so no segment kernel and no second global
// round trip are needed.
//
// Fast path (L <= 64 and T <= 1024; lane s of a wave stands for slot s): one
// wave loads idx and the slot ranks, counts tokens per slot in its own LDS
// histogram (slots of rank 0 then count as empty), scans groups and tokens
// over the slots with DPP, picks the group's slot by ballot, writes the
// group's tokens by ballot rank, and publishes the result; one barrier.
// Generic path (larger L or T): idx staged in LDS, ballot-leader histogram, a
// one-wave scan over slots and a one-wave ballot compaction.
#pragma once

#include "common.hpp"

namespace aa {

struct GroupSel {
    int slot;       // -1: this work-group has no group
    int first;      // rank in the slot of the group's first token
    int ntok;       // tokens in the group (1..G)
    int pos0;       // position of the first token in slot-sorted order
    int rank;       // the slot's rank, min(slot_rank[slot], R)
    int n_groups;   // groups of the whole batch
};

constexpr int kOneWaveChunks = 16;   // one-wave discovery: T <= 1024

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4 and 8 within each row of 16 lanes, then row 0's total into row 1 and row
// 2's into row 3 (row_bcast:15), then lane 31's running total into rows 2 and
// 3 (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// LDS scratch of the discovery.  MAXT: largest T; NW: waves per work-group.
template <int G, int MAXT, int NW>
struct DiscLds {
    int32_t cnt[NW * kWave];   // fast path: per-wave slot histograms
    int32_t tok[G];
    int32_t info[6];
    // generic path
    int32_t slot[MAXT];
    int32_t rank[kMaxSlots];
    int32_t gcnt[kMaxSlots];
};

// One-wave discovery for T <= 64 * MC, L <= 64 (lane s stands for slot s);
// writes d.tok and d.info (slot or -1, first, ntok, pos0, n_groups, rank).
// Every token with a slot in [0, L) is counted; slots of rank 0 then get no
// tokens, which removes their tokens without a per-token rank lookup.
template <int G, int MC, typename DL, typename Pick>
__device__ __forceinline__ void one_wave_group(const int32_t *__restrict__ idx,
                                               const int32_t *__restrict__ slot_rank, int T, int L,
                                               int R, DL &d, Pick pick) {
    const int lane = threadIdx.x & 63;
    int v[MC];
#pragma unroll
    for (int c = 0; c < MC; ++c) v[c] = idx[min(kWave * c + lane, T - 1)];
    const int rk = slot_rank ? min(slot_rank[min(lane, L - 1)], R) : R;
    d.cnt[lane] = 0;
#pragma unroll
    for (int c = 0; c < MC; ++c) {
        const int vv = v[c];
        const bool ok = kWave * c + lane < T && vv >= 0 && vv < L;
        v[c] = ok ? vv : -1;
        // this wave's histogram: LDS program order, no barrier
        if (ok) atomicAdd(&d.cnt[vv], 1);
    }
    const int tot = rk > 0 ? d.cnt[lane] : 0;   // lane s: tokens of slot s
    const int ng = (tot + G - 1) / G;
    // inclusive scans over the slots, groups in the high half-word
    const int inc = wave_incl_scan(tot | (ng << 16));
    const int gi = inc >> 16, ti = inc & 0xffff;
    const int n_groups = __builtin_amdgcn_readlane(gi, kWave - 1);
    const int group = pick(n_groups);
    int info0 = -1, first = 0, ntok = 0, pos0 = 0, rank = 0;
    if (group >= 0 && group < n_groups) {
        const uint64_t hit = __ballot(group >= gi - ng && group < gi);
        const int s = __ffsll((unsigned long long)hit) - 1;
        first = (group - __builtin_amdgcn_readlane(gi - ng, s)) * G;
        ntok = min(G, __builtin_amdgcn_readlane(tot, s) - first);
        pos0 = __builtin_amdgcn_readlane(ti - tot, s) + first;
        rank = __builtin_amdgcn_readlane(rk, s);
        info0 = s;
        uint64_t bal[MC];
#pragma unroll
        for (int c = 0; c < MC; ++c) bal[c] = __ballot(v[c] == s);
        int seen = 0;
#pragma unroll
        for (int c = 0; c < MC; ++c) {
            const int rkk = seen + __popcll(bal[c] & ((1ull << lane) - 1ull));
            if (v[c] == s && rkk >= first && rkk < first + ntok) d.tok[rkk - first] = kWave * c + lane;
            seen += __popcll(bal[c]);
        }
    }
    if (lane == 0) {
        d.info[0] = info0; d.info[1] = first; d.info[2] = ntok;
        d.info[3] = pos0; d.info[4] = n_groups; d.info[5] = rank;
    }
}

// Every thread of the work-group calls this with the same arguments; `pick`
// maps the batch's group count to this work-group's group id (or -1) and must
// be uniform.  On return d.tok[0 .. ntok) holds the group's tokens ascending.
template <int G, int MAXT, int NW, typename Pick>
__device__ GroupSel find_group(const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_rank,
                               int T, int L, int R, DiscLds<G, MAXT, NW> &d, Pick pick) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    GroupSel sel{-1, 0, 0, 0, 0, 0};
    if (L <= kWave && T <= kWave * kOneWaveChunks) {
        // One wave finds the group; the others wait at the single barrier.
        if (w == 0) {
            if (T <= 4 * kWave) one_wave_group<G, 4>(idx, slot_rank, T, L, R, d, pick);
            else if (T <= 8 * kWave) one_wave_group<G, 8>(idx, slot_rank, T, L, R, d, pick);
            else one_wave_group<G, kOneWaveChunks>(idx, slot_rank, T, L, R, d, pick);
        }
        __syncthreads();
        sel.slot = d.info[0];
        sel.first = d.info[1];
        sel.ntok = d.info[2];
        sel.pos0 = d.info[3];
        sel.n_groups = d.info[4];
        sel.rank = d.info[5];
        return sel;
    }

    // ---- generic path ------------------------------------------------------
    constexpr int NT = NW * kWave;
    for (int i = tid; i < L; i += NT) {
        d.rank[i] = slot_rank ? min(slot_rank[i], R) : R;
        d.gcnt[i] = 0;
    }
    for (int i = tid; i < T; i += NT) d.slot[i] = idx[i];
    __syncthreads();
    for (int base = w * kWave; base < T; base += NT) {
        const int i = base + lane;
        int v = i < T ? d.slot[i] : -1;
        v = (v >= 0 && v < L && d.rank[v] > 0) ? v : -1;
        if (i < T) d.slot[i] = v;
        // one LDS atomic per (wave, slot): the lanes of a slot are counted by ballot
        uint64_t rem = __ballot(v >= 0);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int ls = __shfl(v, leader);
            const uint64_t peers = __ballot(v == ls);
            if (lane == leader) atomicAdd(&d.gcnt[ls], __popcll(peers));
            rem &= ~peers;
        }
    }
    __syncthreads();
    if (w == 0) {
        const int per = (L + kWave - 1) / kWave;
        const int lo = lane * per, hi = min(L, lo + per);
        int ng_tot = 0, nt_tot = 0;
        for (int s = lo; s < hi; ++s) {
            ng_tot += (d.gcnt[s] + G - 1) / G;
            nt_tot += d.gcnt[s];
        }
        int ng_inc = ng_tot, nt_inc = nt_tot;
#pragma unroll
        for (int dd = 1; dd < kWave; dd <<= 1) {
            const int a = __shfl_up(ng_inc, dd), b = __shfl_up(nt_inc, dd);
            if (lane >= dd) { ng_inc += a; nt_inc += b; }
        }
        const int n_groups = __shfl(ng_inc, kWave - 1);
        const int group = pick(n_groups);
        if (lane == 0) {
            d.info[0] = -1;
            d.info[4] = n_groups;
        }
        int grun = ng_inc - ng_tot, trun = nt_inc - nt_tot;
        for (int s = lo; s < hi; ++s) {
            const int c = d.gcnt[s];
            const int ngs = (c + G - 1) / G;
            if (group >= grun && group < grun + ngs) {
                const int first = (group - grun) * G;
                d.info[0] = s;
                d.info[1] = first;
                d.info[2] = min(G, c - first);
                d.info[3] = trun + first;
            }
            grun += ngs;
            trun += c;
        }
    }
    __syncthreads();
    sel.n_groups = d.info[4];
    const int s = d.info[0];
    if (s < 0) return sel;
    sel.slot = s;
    sel.first = d.info[1];
    sel.ntok = d.info[2];
    sel.pos0 = d.info[3];
    sel.rank = d.rank[s];
    if (w == 0) {
        int seen = 0;
        for (int base = 0; base < T && seen < sel.first + sel.ntok; base += kWave) {
            const int t = base + lane;
            const bool m = t < T && d.slot[t] == s;
            const uint64_t bal = __ballot(m);
            const int rkk = seen + __popcll(bal & ((1ull << lane) - 1ull));
            if (m && rkk >= sel.first && rkk < sel.first + sel.ntok) d.tok[rkk - sel.first] = t;
            seen += __popcll(bal);
        }
    }
    __syncthreads();
    return sel;
}

}  // namespace aa
