"""Pins for the CPU oracle: each test checks it against something other than
itself -- a hand-worked example, a closed form, an exact integer or float64
computation with a different association, a library sort, or an invariant
that the mathematics fixes.  All run on the CPU."""
import itertools
import json
import os

import numpy as np
import pytest

import synth
from tests import bounds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _arr(v, dt=np.float32):
    return np.asarray(v, dtype=dt)


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------

def test_hand_example_linear(oracle_mod):
    g = _golden()["linear_packed"]
    A = [_arr(a) for a in g["A"]]
    B = [_arr(b) for b in g["B"]]
    y, buf = oracle_mod.lora_apply(_arr(g["y0"]), _arr(g["x"]), A, B, _arr(g["idx"], np.int32),
                                   _arr(g["slot_rank"], np.int32), _arr(g["scale"]))
    assert np.array_equal(y, _arr(g["expected_y"]))
    assert np.array_equal(buf, _arr(g["expected_buf"]))
    perm, start, ninv = oracle_mod.segments(_arr(g["idx"], np.int32),
                                            _arr(g["slot_rank"], np.int32), g["L"])
    assert perm.tolist() == g["expected_perm"]
    assert start.tolist() == g["expected_slot_start"]
    assert ninv == 0


def test_hand_example_moe(oracle_mod):
    gd = _golden()
    g = gd["moe_w13"]
    y = oracle_mod.moe_lora_apply(0, _arr(g["y0"]), _arr(g["x"]), [_arr(a) for a in g["A"]],
                                  [_arr(b) for b in g["B"]], _arr(g["topk_ids"], np.int32), None,
                                  _arr(g["idx"], np.int32), _arr(g["slot_rank"], np.int32),
                                  _arr(g["scale"]), g["E"])
    assert np.array_equal(y, _arr(g["expected_y"]))
    g = gd["moe_w2"]
    args = (_arr(g["x"]), [_arr(a) for a in g["A"]], [_arr(b) for b in g["B"]],
            _arr(g["topk_ids"], np.int32), _arr(g["topk_w"]), _arr(g["idx"], np.int32),
            _arr(g["slot_rank"], np.int32), _arr(g["scale"]), g["E"])
    y = oracle_mod.moe_lora_apply(1, _arr(g["y0"]), *args)
    assert np.array_equal(y, _arr(g["expected_y"]))
    y = oracle_mod.moe_lora_apply(1, np.zeros((g["T"], 3), np.float32), *args, reduce_k=True)
    assert np.array_equal(y, _arr(g["expected_y_reduced"]))


@pytest.mark.parametrize("bm", [2, 4])
def test_hand_example_moe_align(oracle_mod, bm):
    g = _golden()["moe_align"]
    so, be, npp = oracle_mod.moe_align(_arr(g["topk_ids"], np.int32), _arr(g["idx"], np.int32),
                                       _arr(g["slot_rank"], np.int32), g["E"], g["L"], bm)
    exp = g[f"block_m_{bm}"]
    assert so.tolist() == exp["sorted_ids"]
    assert be.tolist() == exp["block_expert"]
    assert npp.tolist() == exp["num_post_padded"]


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_zero_b_is_identity_bit_exact(oracle_mod):
    c = synth.config_tiny()
    B0 = [np.zeros_like(b) for b in c.B]
    y, buf = oracle_mod.lora_apply(c.y0, c.x, c.A, B0, c.idx, c.slot_rank, c.scale)
    assert np.array_equal(y.view(np.uint32), c.y0.view(np.uint32))
    assert np.any(buf != 0)


def test_passthrough_rows_bit_exact(oracle_mod):
    c = synth.make_linear("pt", 12, 32, [16, 8], 4, 3,
                          idx=[-1, 0, 3, 1, 7, 2, -5, 0, 1, 2, 3, -1],
                          slot_rank=[4, 0, 2], scale=[1.0, 1.0, 3.0], dtype="f32", seed=7,
                          w_std=0.5)
    y, buf = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    untouched = [t for t in range(c.T) if c.idx[t] < 0 or c.idx[t] >= 3 or c.slot_rank[c.idx[t]] == 0]
    touched = [t for t in range(c.T) if t not in untouched]
    assert untouched and touched
    for t in untouched:
        assert np.array_equal(y[t].view(np.uint32), c.y0[t].view(np.uint32))
        assert np.all(buf[:, t, :] == 0)
    for t in touched:
        assert np.any(y[t] != c.y0[t])
    perm, start, ninv = oracle_mod.segments(c.idx, c.slot_rank, c.L)
    assert ninv == 3  # idx 3, 7, 3 (>= L); -1 and -5 are "no adapter", not invalid


def test_rank1_outer_product_closed_form(oracle_mod):
    rng = np.random.default_rng(3)
    T, K, N = 9, 37, 23
    x = rng.standard_normal((T, K)).astype(np.float32)
    a = rng.standard_normal((1, 1, K)).astype(np.float32)
    b = rng.standard_normal((1, N, 1)).astype(np.float32)
    y0 = rng.standard_normal((T, N)).astype(np.float32)
    idx = np.zeros(T, np.int32)
    scale = np.array([0.75], np.float32)
    y, _ = oracle_mod.lora_apply(y0, x, [a], [b], idx, np.array([1], np.int32), scale)
    xd, ad, bd = x.astype(np.float64), a[0, 0].astype(np.float64), b[0, :, 0].astype(np.float64)
    exact = y0.astype(np.float64) + 0.75 * np.outer(xd @ ad, bd)
    M = np.abs(y0) + 0.75 * np.outer(np.abs(xd) @ np.abs(ad), np.abs(bd))
    assert np.all(np.abs(y - exact) <= bounds.fp32_bound(M, K, 1))


def test_tiny_bruteforce_all_index_vectors(oracle_mod):
    """All 3^T assignments (slot 0, slot 1, none) on T=4 tokens, each slot
    rank from 1 to R, against the float64 dense product W = scale B A."""
    rng = np.random.default_rng(11)
    T, K, N, R, L = 4, 7, [5, 3], 3, 2
    x = rng.standard_normal((T, K)).astype(np.float32)
    A = [rng.standard_normal((L, R, K)).astype(np.float32) for _ in N]
    B = [rng.standard_normal((L, n, R)).astype(np.float32) for n in N]
    y0 = rng.standard_normal((T, sum(N))).astype(np.float32)
    scale = np.array([1.5, -0.5], np.float32)
    for ranks in itertools.product(range(1, R + 1), repeat=L):
        sr = np.array(ranks, np.int32)
        Ap = [a.copy() for a in A]
        Bp = [b.copy() for b in B]
        for a, b in zip(Ap, Bp):
            for s, r in enumerate(sr):
                a[s, r:] = 0
                b[s, :, r:] = 0
        for combo in itertools.product([-1, 0, 1], repeat=T):
            idx = np.array(combo, np.int32)
            y, _ = oracle_mod.lora_apply(y0, x, Ap, Bp, idx, sr, scale)
            ex = bounds.linear_exact_f64(x, Ap, Bp, idx, sr, scale, y0)
            M = bounds.linear_magnitude(x, Ap, Bp, idx, sr, scale, y0)
            assert np.all(np.abs(y - ex) <= bounds.fp32_bound(M, K, R)), (ranks, combo)


def test_shrink_and_expand_separately_vs_f64(oracle_mod):
    rng = np.random.default_rng(5)
    T, K, N, R, L = 10, 19, [6, 4, 9], 5, 3
    x = rng.standard_normal((T, K)).astype(np.float32)
    A = [rng.standard_normal((L, R, K)).astype(np.float32) for _ in N]
    B = [rng.standard_normal((L, n, R)).astype(np.float32) for n in N]
    idx = rng.integers(-1, L, T).astype(np.int32)
    sr = np.array([5, 2, 4], np.int32)
    buf = oracle_mod.lora_shrink(x, A, idx, sr)
    for sig, a in enumerate(A):
        for t in range(T):
            s = idx[t]
            if s < 0:
                assert np.all(buf[sig, t] == 0)
                continue
            r = sr[s]
            ex = a[s, :r].astype(np.float64) @ x[t].astype(np.float64)
            Mb = np.abs(a[s, :r].astype(np.float64)) @ np.abs(x[t].astype(np.float64))
            assert np.all(np.abs(buf[sig, t, :r] - ex) <= 2 * bounds.gamma(K) * Mb)
            assert np.all(buf[sig, t, r:] == 0)
    # expand with an arbitrary buffer (non-zero beyond rank must be ignored)
    bufr = rng.standard_normal((len(N), T, R)).astype(np.float32)
    y0 = rng.standard_normal((T, 3 + sum(N))).astype(np.float32)
    scale = np.array([0.5, 2.0, -1.0], np.float32)
    y = oracle_mod.lora_expand(y0, bufr, B, idx, sr, scale, y_col_offset=3)
    assert np.array_equal(y[:, :3], y0[:, :3])
    off = 3
    for sig, b in enumerate(B):
        for t in range(T):
            s = idx[t]
            if s < 0:
                assert np.array_equal(y[t, off:off + N[sig]], y0[t, off:off + N[sig]])
                continue
            r = sr[s]
            d = b[s, :, :r].astype(np.float64) @ bufr[sig, t, :r].astype(np.float64)
            ex = y0[t, off:off + N[sig]] + float(scale[s]) * d
            M = np.abs(y0[t, off:off + N[sig]]) + abs(float(scale[s])) * (
                np.abs(b[s, :, :r].astype(np.float64)) @ np.abs(bufr[sig, t, :r]))
            assert np.all(np.abs(y[t, off:off + N[sig]] - ex) <= 2 * bounds.gamma(R + 3) * M)
        off += N[sig]


def test_integer_vectors_exact(oracle_mod):
    c = synth.make_integer_linear(40, 96, [24, 8, 8], 8, 5, seed=21, dtype="f32")
    y, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    ex = bounds.linear_exact_int(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(y, ex.astype(np.float32))
    assert np.max(np.abs(ex)) <= 256


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_scale_doubling_bit_exact(oracle_mod):
    c = synth.config_tiny()
    z = np.zeros_like(c.y0)
    y1, _ = oracle_mod.lora_apply(z, c.x, c.A, c.B, c.idx, c.slot_rank, np.ones(3, np.float32))
    y2, _ = oracle_mod.lora_apply(z, c.x, c.A, c.B, c.idx, c.slot_rank, np.full(3, 2, np.float32))
    assert np.array_equal(y2, 2 * y1)
    assert np.any(y1 != 0)


def test_slot_relabel_and_token_permutation_bit_exact(oracle_mod):
    c = synth.make_linear("perm", 20, 48, [16, 12], 6, 4, idx=np.arange(20) % 5 - 1,
                          slot_rank=[6, 3, 5, 1], scale=[1, 2, 0.5, -1], dtype="f32", seed=9,
                          w_std=0.3)
    y, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    sigma = np.array([2, 0, 3, 1])           # new slot of old slot s
    inv = np.argsort(sigma)
    A2 = [a[inv] for a in c.A]
    B2 = [b[inv] for b in c.B]
    idx2 = np.where(c.idx >= 0, sigma[np.maximum(c.idx, 0)], c.idx).astype(np.int32)
    y2, _ = oracle_mod.lora_apply(c.y0, c.x, A2, B2, idx2, c.slot_rank[inv], c.scale[inv])
    assert np.array_equal(y, y2)
    tp = np.random.default_rng(1).permutation(c.T)
    y3, _ = oracle_mod.lora_apply(c.y0[tp], c.x[tp], c.A, c.B, c.idx[tp], c.slot_rank, c.scale)
    assert np.array_equal(y3, y[tp])


def test_packed_equals_single_slices_bit_exact(oracle_mod):
    c = synth.config_decode(T=24)
    c = synth.make_linear("pk", 24, 64, [32, 8, 8], 4, 3, idx=np.arange(24) % 4 - 1,
                          slot_rank=[4, 2, 3], scale=[2.0, 1.0, 0.5], dtype="bf16", seed=4)
    y, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    ys = c.y0.copy()
    off = 0
    for a, b in zip(c.A, c.B):
        ys, _ = oracle_mod.lora_apply(ys, c.x, [a], [b], c.idx, c.slot_rank, c.scale,
                                      y_col_offset=off)
        off += b.shape[1]
    assert np.array_equal(y, ys)


def test_zero_padding_invariance_bit_exact(oracle_mod):
    rng = np.random.default_rng(2)
    T, K, N, r, L = 8, 40, [12], 3, 2
    x = rng.standard_normal((T, K)).astype(np.float32)
    A = [rng.standard_normal((L, r, K)).astype(np.float32)]
    B = [rng.standard_normal((L, N[0], r)).astype(np.float32)]
    idx = (np.arange(T) % 3 - 1).astype(np.int32)
    y0 = rng.standard_normal((T, N[0])).astype(np.float32)
    sc = np.array([1.0, 0.25], np.float32)
    y, _ = oracle_mod.lora_apply(y0, x, A, B, idx, np.array([r, r], np.int32), sc)
    Rp = 8
    Ap = [np.zeros((L, Rp, K), np.float32)]
    Bp = [np.zeros((L, N[0], Rp), np.float32)]
    Ap[0][:, :r] = A[0]
    Bp[0][:, :, :r] = B[0]
    yp, _ = oracle_mod.lora_apply(y0, x, Ap, Bp, idx, np.array([r, r], np.int32), sc)
    assert np.array_equal(y, yp)
    # the padded slot with rank = R gives the same (adds exact zeros)
    yq, _ = oracle_mod.lora_apply(y0, x, Ap, Bp, idx, np.array([Rp, Rp], np.int32), sc)
    assert np.array_equal(y, yq)


# --------------------------------------------------------------------------
# segments: the stable counting sort against numpy's stable argsort
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,T,L", [(0, 0, 3), (1, 1, 1), (2, 257, 8), (3, 1000, 128), (4, 64, 5)])
def test_segments_vs_stable_argsort(oracle_mod, seed, T, L):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-2, L + 2, size=T).astype(np.int32)
    sr = rng.integers(0, 3, size=L).astype(np.int32)
    perm, start, ninv = oracle_mod.segments(idx, sr, L)
    active = np.array([(0 <= i < L) and sr[i] > 0 for i in idx], bool) if T else np.zeros(0, bool)
    toks = np.nonzero(active)[0]
    order = toks[np.argsort(idx[toks], kind="stable")]
    n = len(order)
    assert perm[:n].tolist() == order.tolist()
    assert np.all(perm[n:] == -1)
    counts = np.bincount(idx[toks], minlength=L) if n else np.zeros(L, int)
    assert start.tolist() == [0] + np.cumsum(counts).tolist()
    assert ninv == int(np.sum(idx >= L))


# --------------------------------------------------------------------------
# fused MoE
# --------------------------------------------------------------------------

def _small_moe(shared, seed=31, T=6, k=2, E=4, K=24, I=10, R=4, L=3):
    return synth.make_moe("small", T, k, E, K, I, R, L, "f32", seed, shared_outer=shared,
                          w_std=0.5, idx=np.array([0, 1, -1, 2, 0, 1][:T], np.int32),
                          slot_rank=np.array([4, 2, 3], np.int32),
                          scale=np.array([1.0, 0.5, 2.0], np.float32))


@pytest.mark.parametrize("shared", [True, False])
def test_moe_vs_f64(oracle_mod, shared):
    c = _small_moe(shared)
    y13 = oracle_mod.moe_lora_apply(0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx,
                                    c.slot_rank, c.scale, c.E)
    ex = bounds.moe_exact_f64(0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx,
                              c.slot_rank, c.scale, c.E)
    M = bounds.moe_magnitude(0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx,
                             c.slot_rank, c.scale, c.E)
    assert np.all(np.abs(y13 - ex) <= bounds.fp32_bound(M, c.K, c.R))
    y2 = oracle_mod.moe_lora_apply(1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                                   c.slot_rank, c.scale, c.E)
    ex = bounds.moe_exact_f64(1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                              c.slot_rank, c.scale, c.E)
    M = bounds.moe_magnitude(1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                             c.slot_rank, c.scale, c.E)
    assert np.all(np.abs(y2 - ex) <= bounds.fp32_bound(M, c.I, c.R, extra=6))
    assert np.any(y2 != c.out0)


def test_moe_shared_outer_equals_broadcast_bit_exact(oracle_mod):
    c = _small_moe(True)
    A13b = [np.repeat(a, c.E, axis=1) for a in c.A13]
    B2b = np.repeat(c.B2, c.E, axis=1)
    y = oracle_mod.moe_lora_apply(0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx,
                                  c.slot_rank, c.scale, c.E)
    yb = oracle_mod.moe_lora_apply(0, c.gate_up0, c.x, A13b, c.B13, c.topk_ids, None, c.idx,
                                   c.slot_rank, c.scale, c.E)
    assert np.array_equal(y, yb)
    y = oracle_mod.moe_lora_apply(1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                                  c.slot_rank, c.scale, c.E)
    yb = oracle_mod.moe_lora_apply(1, c.out0, c.h, [c.A2], [B2b], c.topk_ids, c.topk_w, c.idx,
                                   c.slot_rank, c.scale, c.E)
    assert np.array_equal(y, yb)


def test_moe_single_expert_equals_linear_bit_exact(oracle_mod):
    c = synth.make_linear("lin", 9, 32, [8, 8], 4, 2, idx=[0, 1, -1, 1, 0, 0, 1, -1, 0],
                          slot_rank=[4, 3], scale=[1.0, 2.0], dtype="f32", seed=3, w_std=0.4)
    y, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    A4 = [a[:, None] for a in c.A]
    B4 = [b[:, None] for b in c.B]
    ids = np.zeros((c.T, 1), np.int32)
    ym = oracle_mod.moe_lora_apply(0, c.y0, c.x, A4, B4, ids, None, c.idx, c.slot_rank, c.scale, 1)
    assert np.array_equal(y, ym)
    ym2 = oracle_mod.moe_lora_apply(1, c.y0, c.x, A4, B4, ids, np.ones((c.T, 1), np.float32),
                                    c.idx, c.slot_rank, c.scale, 1)
    assert np.array_equal(y, ym2)


def test_moe_reduced_equals_sum_over_k(oracle_mod):
    c = _small_moe(True)
    z3 = np.zeros_like(c.out0)
    y3 = oracle_mod.moe_lora_apply(1, z3, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                                   c.slot_rank, c.scale, c.E)
    yr = oracle_mod.moe_lora_apply(1, np.zeros((c.T, c.K), np.float32), c.h, [c.A2], [c.B2],
                                   c.topk_ids, c.topk_w, c.idx, c.slot_rank, c.scale, c.E,
                                   reduce_k=True)
    acc = np.zeros((c.T, c.K), np.float32)
    for j in range(c.k):
        acc = acc + y3.reshape(c.T, c.k, c.K)[:, j]
    assert np.array_equal(yr, acc)


def _moe_align_bruteforce(topk_ids, idx, sr, E, L, bm):
    T, k = topk_ids.shape
    P = T * k
    cap = -(-(P + E * (bm - 1)) // bm) * bm
    so = np.full((L, cap), P, np.int32)
    be = np.full((L, cap // bm), -1, np.int32)
    npp = np.zeros(L, np.int32)
    for s in range(L):
        if sr[s] <= 0:
            continue
        groups = {}
        for p in range(P):
            if idx[p // k] == s and 0 <= topk_ids.flat[p] < E:
                groups.setdefault(int(topk_ids.flat[p]), []).append(p)
        out, blocks = [], []
        for e in sorted(groups):
            g = groups[e]
            padded = g + [P] * ((-len(g)) % bm)
            out += padded
            blocks += [e] * (len(padded) // bm)
        so[s, :len(out)] = out
        be[s, :len(blocks)] = blocks
        npp[s] = len(out)
    return so, be, npp


@pytest.mark.parametrize("seed,T,k,E,L,bm", [(0, 7, 2, 4, 3, 4), (1, 64, 8, 16, 4, 16),
                                              (2, 1, 1, 1, 1, 1), (3, 33, 3, 5, 6, 8)])
def test_moe_align_vs_bruteforce(oracle_mod, seed, T, k, E, L, bm):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx = rng.integers(-1, L, size=T).astype(np.int32)
    sr = rng.integers(0, 2, size=L).astype(np.int32)
    got = oracle_mod.moe_align(ids, idx, sr, E, L, bm)
    exp = _moe_align_bruteforce(ids, idx, sr, E, L, bm)
    for g, e in zip(got, exp):
        assert np.array_equal(g, e)
