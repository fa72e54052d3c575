"""GPU parity of the fused-MoE LoRA path (alignment, w13 and w2 deltas)
against the CPU oracle, through the C ABI."""
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import adapter_apply_amd as aa  # noqa: E402
import synth  # noqa: E402
from tests import bounds, oracle_par  # noqa: E402
from tests.gpu_util import canaries_intact, dev, guarded, host_f32, log  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
W13, W2 = aa.MOE_LORA_W13, aa.MOE_LORA_W2
BF = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aa.lib()


def pad_to(a, axis, n):
    pad = [(0, 0)] * a.ndim
    pad[axis] = (0, n - a.shape[axis])
    return np.pad(a, pad)


def run_moe(kind, y0, x, A, B, topk_ids, topk_w, idx, rank, scale, E, reduce_k=False, ws=None,
            flags=0, guard=True, align=False):
    """One moe_lora_apply call.  align=True runs moe_lora_align first and
    passes its segments (the aligned path at any size); otherwise a call of a
    few pairs takes the path without alignment."""
    T, k = topk_ids.shape
    L, _, R, _ = A[0].shape
    if ws is None:
        ws = aa.alloc_moe_workspace(T, k, len(A), R, L, E)
    if align:
        aa.moe_lora_align(dev(topk_ids), dev(idx), dev(rank), E, L, R, 16, ws)
        flags |= aa.LORA_FLAG_SEGMENTS_READY
    if guard:
        yfull, y = guarded(y0, BF)
    else:
        yfull, y = None, dev(y0, BF)
    aa.moe_lora_apply(kind, y, dev(x, BF), [dev(a, BF) for a in A], [dev(b, BF) for b in B],
                      dev(topk_ids), None if topk_w is None else dev(topk_w), dev(idx), dev(rank),
                      dev(scale), E, ws, reduce_k=reduce_k, flags=flags)
    torch.cuda.synchronize()
    if guard:
        assert canaries_intact(yfull)
    return host_f32(y)


def test_hand_examples_padded():
    """The hand-worked w13 / w2 examples, zero-padded to K % 8, R % 16 and
    N % 4 (padding adds exact zeros), reproduce the hand results bit for bit."""
    with open(GOLDEN) as f:
        g = json.load(f)
    for key, kind in (("moe_w13", W13), ("moe_w2", W2)):
        c = g[key]
        x = pad_to(np.asarray(c["x"], np.float32), 1, 8)
        A = [pad_to(pad_to(np.asarray(a, np.float32), 3, 8), 2, 16) for a in c["A"]]
        Bs = [np.asarray(b, np.float32) for b in c["B"]]
        n = Bs[0].shape[2]
        B = [pad_to(pad_to(b, 3, 16), 2, 4) for b in Bs]
        y0 = pad_to(np.asarray(c["y0"], np.float32), 1, 4)
        topk_w = np.asarray(c["topk_w"], np.float32) if "topk_w" in c else None
        args = (x, A, B, np.asarray(c["topk_ids"], np.int32), topk_w,
                np.asarray(c["idx"], np.int32), np.asarray(c["slot_rank"], np.int32),
                np.asarray(c["scale"], np.float32), c["E"])
        for align in (False, True):       # without, then with the alignment
            y = run_moe(kind, y0, *args, align=align)
            assert np.array_equal(y[:, :n], np.asarray(c["expected_y"], np.float32)), (key, align)
            assert np.all(y[:, n:] == 0)
        if key == "moe_w2":
            y = run_moe(kind, np.zeros((c["T"], 4), np.float32), *args, reduce_k=True)
            assert np.array_equal(y[:, :n], np.asarray(c["expected_y_reduced"], np.float32))


def integer_moe(seed, T, k, E, K, I, R, L, shared, p_none=0.1, full_rank=False,
                weights=(0.5, 0.25, 1.0)):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, L, size=T).astype(np.int32)
    idx[rng.random(T) < p_none] = -1
    rank = (np.full(L, R, np.int32) if full_rank else
            rng.integers(1, R + 1, size=L).astype(np.int32))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    Ea = 1 if shared else E
    x = rng.integers(-1, 2, size=(T, K)).astype(np.float32)
    h = rng.integers(-1, 2, size=(T * k, I)).astype(np.float32)
    A13 = [synth.ternary_sparse(rng, (L, Ea, R, K), 32) for _ in range(2)]
    B13 = [synth.ternary_sparse(rng, (L, E, I, R), 2) for _ in range(2)]
    A2 = synth.ternary_sparse(rng, (L, E, R, I), 32)
    B2 = synth.ternary_sparse(rng, (L, Ea, K, R), 2)
    for s in range(L):
        for a in A13:
            a[s, :, rank[s]:] = 0
        for b in B13:
            b[s, :, :, rank[s]:] = 0
        A2[s, :, rank[s]:] = 0
        B2[s, :, :, rank[s]:] = 0
    w = rng.choice(np.array(weights, np.float32), size=(T, k))
    g0 = rng.integers(-8, 9, size=(T * k, 2 * I)).astype(np.float32)
    o0 = rng.integers(-8, 9, size=(T * k, K)).astype(np.float32)
    scale = np.full(L, 2.0, np.float32)
    return dict(x=x, h=h, A13=A13, B13=B13, A2=A2, B2=B2, ids=ids, w=w, g0=g0, o0=o0, idx=idx,
                rank=rank, scale=scale, E=E)


@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("seed,T,k,E,K,I,R,L", [
    (1, 37, 2, 4, 64, 40, 16, 3),
    (2, 130, 8, 16, 256, 96, 32, 4),
    (3, 1, 1, 1, 8, 8, 16, 1),
    (4, 300, 4, 64, 128, 64, 16, 16),     # L * E = 1024 keys
    (5, 40, 4, 8, 2048, 1024, 16, 3),     # small batch, long K: the shrinks split over K
    (6, 30, 2, 4, 256, 128, 512, 2),      # the largest rank the library takes
    (7, 128, 8, 16, 256, 96, 16, 4),      # 1024 pairs: the most the unaligned path takes
    (8, 129, 8, 16, 256, 96, 16, 4),      # 1032 pairs: aligned only
])
def test_integer_vectors_bit_exact(oracle_mod, shared, seed, T, k, E, K, I, R, L):
    d = integer_moe(seed, T, k, E, K, I, R, L, shared)
    ref13 = oracle_mod.moe_lora_apply(0, d["g0"], d["x"], d["A13"], d["B13"], d["ids"], None,
                                      d["idx"], d["rank"], d["scale"], E)
    ref2 = oracle_mod.moe_lora_apply(1, d["o0"], d["h"], [d["A2"]], [d["B2"]], d["ids"], d["w"],
                                     d["idx"], d["rank"], d["scale"], E)
    assert aa.moe_lora_plan(T, k, R) == (T * k <= 1024 and R == 16)
    # both paths where a call is small enough for the one without alignment
    for align in ((False, True) if aa.moe_lora_plan(T, k, R) else (False,)):
        log(f"case moe integer shared={shared} T={T} k={k} E={E} L={L} align={align}")
        y = run_moe(W13, d["g0"], d["x"], d["A13"], d["B13"], d["ids"], None, d["idx"], d["rank"],
                    d["scale"], E, align=align)
        assert np.array_equal(y, ref13), np.max(np.abs(y - ref13))
        y = run_moe(W2, d["o0"], d["h"], [d["A2"]], [d["B2"]], d["ids"], d["w"], d["idx"],
                    d["rank"], d["scale"], E, align=align)
        assert np.array_equal(y, ref2), np.max(np.abs(y - ref2))
    if shared:
        z = np.zeros((T, K), np.float32)
        y = run_moe(W2, z, d["h"], [d["A2"]], [d["B2"]], d["ids"], None, d["idx"], d["rank"],
                    d["scale"], E, reduce_k=True)
        ref = oracle_mod.moe_lora_apply(1, z, d["h"], [d["A2"]], [d["B2"]], d["ids"], None,
                                        d["idx"], d["rank"], d["scale"], E, reduce_k=True)
        assert np.array_equal(y, ref), np.max(np.abs(y - ref))


@pytest.mark.parametrize("shared", [True, False])
def test_w13_single_slice_and_interleaved(oracle_mod, shared):
    """[vLLM] FusedMoE3DWithLoRA: one w13 slice, lora_b [L][E][2I][R] under
    one lora_a, its gate and up rows either concatenated or interleaved (the
    order its slicing keeps for GPT-OSS).  Interleaving permutes lora_b's rows
    and the output columns alike, so the interleaved result is the
    concatenated one with its columns interleaved, bit for bit."""
    d = integer_moe(5, 90, 4, 8, 128, 48, 16, 3, shared)
    E = d["E"]
    A = [d["A13"][0]]
    Bcat = [np.concatenate(d["B13"], axis=2)]
    I = d["B13"][0].shape[2]
    perm = np.empty(2 * I, np.int64)
    perm[0::2] = np.arange(I)
    perm[1::2] = I + np.arange(I)          # interleaved column c = concatenated column perm[c]
    Bint = [np.ascontiguousarray(Bcat[0][:, :, perm, :])]
    log(f"case moe w13 single slice shared={shared}")
    y_cat = run_moe(W13, d["g0"], d["x"], A, Bcat, d["ids"], None, d["idx"], d["rank"], d["scale"], E)
    ref = oracle_mod.moe_lora_apply(0, d["g0"], d["x"], A, Bcat, d["ids"], None, d["idx"], d["rank"],
                                    d["scale"], E)
    assert np.array_equal(y_cat, ref), np.max(np.abs(y_cat - ref))
    y_int = run_moe(W13, np.ascontiguousarray(d["g0"][:, perm]), d["x"], A, Bint, d["ids"], None,
                    d["idx"], d["rank"], d["scale"], E)
    assert np.array_equal(y_int, y_cat[:, perm])


@pytest.mark.parametrize("align", [False, True])
def test_small_batch_invalid_experts_and_empty_slots(oracle_mod, align):
    """Pairs whose expert is outside [0, E), tokens without an adapter and a
    slot of rank 0 leave their rows bit-exact, on both paths of a small call."""
    T, k, E, K, I, R, L = 12, 4, 8, 1024, 256, 16, 3
    d = integer_moe(7, T, k, E, K, I, R, L, shared=True, p_none=0.2)
    ids = d["ids"].copy()
    ids[0, 1] = -1
    ids[3, 2] = E
    ids[5, 0] = E + 7
    rank = d["rank"].copy()
    rank[1] = 0
    log(f"case moe small invalid experts align={align}")
    for kind, y0, x, A, B, w in ((W13, d["g0"], d["x"], d["A13"], d["B13"], None),
                                 (W2, d["o0"], d["h"], [d["A2"]], [d["B2"]], d["w"])):
        y = run_moe(kind, y0, x, A, B, ids, w, d["idx"], rank, d["scale"], E, align=align)
        ref = oracle_mod.moe_lora_apply(kind, y0, x, A, B, ids, w, d["idx"], rank, d["scale"], E)
        assert np.array_equal(y, ref), np.max(np.abs(y - ref))
        t_of = np.arange(T * k) // k
        dead = (ids.reshape(-1) < 0) | (ids.reshape(-1) >= E) | (d["idx"][t_of] < 0) | \
               (rank[np.maximum(d["idx"][t_of], 0)] == 0)
        assert dead.any()
        assert np.array_equal(y[dead], y0[dead])


def test_w2_shared_lora_b_pair_runs_invalid_experts(oracle_mod):
    """w2 with one lora_b for every expert walks runs of 64 (token, k) pairs of
    the token tiles: several runs per slot, a top_k that does not divide 64, and
    pairs whose expert lies outside [0, E) inside full runs stay untouched; bit
    for bit against the oracle."""
    T, k, E, K, I, R, L = 700, 6, 16, 256, 128, 16, 3
    d = integer_moe(11, T, k, E, K, I, R, L, shared=True, p_none=0.1)
    rng = np.random.default_rng(12)
    ids = d["ids"].copy()
    bad = rng.random(ids.shape) < 0.05
    ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + 3)
    log("case moe w2 pair runs with invalid experts")
    y = run_moe(W2, d["o0"], d["h"], [d["A2"]], [d["B2"]], ids, d["w"], d["idx"], d["rank"],
                d["scale"], E)
    ref = oracle_mod.moe_lora_apply(1, d["o0"], d["h"], [d["A2"]], [d["B2"]], ids, d["w"],
                                    d["idx"], d["rank"], d["scale"], E)
    assert np.array_equal(y, ref), np.max(np.abs(y - ref))
    t_of = np.arange(T * k) // k
    dead = (ids.reshape(-1) < 0) | (ids.reshape(-1) >= E) | (d["idx"][t_of] < 0)
    assert dead.sum() > 100
    assert np.array_equal(y[dead], d["o0"][dead])


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, n)])).astype(np.int64)


def oracle_rows(oracle_mod, c, kind, rows, reduce_k=False):
    """Oracle on a token subset (the delta of a token depends on nothing else)."""
    ids = c.topk_ids[rows]
    pr = (rows[:, None] * c.k + np.arange(c.k)[None, :]).reshape(-1)
    if kind == 0:
        return oracle_mod.moe_lora_apply(0, c.gate_up0[pr], c.x[rows], c.A13, c.B13, ids, None,
                                         c.idx[rows], c.slot_rank, c.scale, c.E)
    y0 = np.zeros((len(rows), c.K), np.float32) if reduce_k else c.out0[pr]
    return oracle_mod.moe_lora_apply(1, y0, c.h[pr], [c.A2], [c.B2], ids, c.topk_w[rows],
                                     c.idx[rows], c.slot_rank, c.scale, c.E, reduce_k=reduce_k)


def test_moe_config_shared_outer(oracle_mod):
    """2048 tokens, 64 experts top-8, d_model 4096, d_mlp 1536, rank 16, 8
    adapters, shared-outer: w13 and w2 (per pair and k-reduced) on the same
    alignment; every output of every token against the oracle (run in token
    blocks on the host cores)."""
    c = synth.config_moe()
    log("case moe config (shared-outer), all tokens")
    T, k = c.T, c.k
    ws = aa.alloc_moe_workspace(T, k, 2, c.R, c.L, c.E)
    aa.moe_lora_align(dev(c.topk_ids), dev(c.idx), dev(c.slot_rank), c.E, c.L, c.R, 16, ws)
    ready = aa.LORA_FLAG_SEGMENTS_READY
    y = run_moe(W13, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx, c.slot_rank, c.scale,
                c.E, ws=ws, flags=ready)
    ref = oracle_par.moe_lora_apply(oracle_mod, 0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids,
                                    None, c.idx, c.slot_rank, c.scale, c.E)
    err, rel = bounds.check_bf16_tolerance(y, ref)
    log(f"  w13 all {T * k} pairs: max abs err {err:.3e} rel {rel:.3e}")
    y = run_moe(W2, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx, c.slot_rank, c.scale,
                c.E, ws=ws, flags=ready)
    ref = oracle_par.moe_lora_apply(oracle_mod, 1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids,
                                    c.topk_w, c.idx, c.slot_rank, c.scale, c.E)
    err, rel = bounds.check_bf16_tolerance(y, ref)
    log(f"  w2 all {T * k} pairs: max abs err {err:.3e} rel {rel:.3e}")
    z = np.zeros((T, c.K), np.float32)
    yr = run_moe(W2, z, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx, c.slot_rank, c.scale,
                 c.E, ws=ws, flags=ready, reduce_k=True)
    ref = oracle_par.moe_lora_apply(oracle_mod, 1, z, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w,
                                    c.idx, c.slot_rank, c.scale, c.E, reduce_k=True)
    err, rel = bounds.check_bf16_tolerance(yr, ref)
    log(f"  w2 k-reduced all {T} tokens: max abs err {err:.3e} rel {rel:.3e}")


def test_moe_config_shape_integer_bit_exact(oracle_mod):
    """Integer vectors at exactly the fused-MoE workload's shape (2048 tokens,
    64 experts top-8, d_model 4096, d_mlp 1536, rank 16, 8 adapters,
    shared-outer) on the aligned path: w13, w2 per pair and k-reduced w2 equal
    the oracle bit for bit on every output."""
    T, k, E, K, I, R, L = 2048, 8, 64, 4096, 1536, 16, 8
    # weights 1 and 1/2 with scale 2: every per-pair and k-summed result is an
    # integer far inside bf16's exact range
    d = integer_moe(81, T, k, E, K, I, R, L, shared=True, p_none=0.0, full_rank=True,
                    weights=(1.0, 0.5))
    log("case moe config-shape integer (aligned)")
    ws = aa.alloc_moe_workspace(T, k, 2, R, L, E)
    aa.moe_lora_align(dev(d["ids"]), dev(d["idx"]), dev(d["rank"]), E, L, R, 16, ws)
    ready = aa.LORA_FLAG_SEGMENTS_READY
    for kind, y0, x, A, B, w, red in ((W13, d["g0"], d["x"], d["A13"], d["B13"], None, False),
                                      (W2, d["o0"], d["h"], [d["A2"]], [d["B2"]], d["w"], False),
                                      (W2, np.zeros((T, K), np.float32), d["h"], [d["A2"]],
                                       [d["B2"]], d["w"], True)):
        log(f"  kind={kind} reduce_k={red}")
        y = run_moe(kind, y0, x, A, B, d["ids"], w, d["idx"], d["rank"], d["scale"], E,
                    reduce_k=red, ws=ws, flags=ready)
        ref = oracle_par.moe_lora_apply(oracle_mod, kind, y0, x, A, B, d["ids"], w, d["idx"],
                                        d["rank"], d["scale"], E, reduce_k=red)
        bad = np.argwhere(y != ref)
        assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("T,align", [(4, False), (8, False), (12, False), (24, False), (4, True),
                                     (8, True), (40, False), (40, True)])
def test_moe_config_small_batch(oracle_mod, T, align):
    """The fused-MoE workload's shapes at decode-sized batches (d_model 4096,
    d_mlp 1536, 64 experts top-8, rank 16, 8 adapters): a call of few pairs
    skips the alignment (4 and 8 tokens: one output column per thread; 12
    tokens: two for w2; 24 tokens: four); aligned, the few tiles make both
    shrinks run split over K."""
    c = synth.config_moe(T=T)
    rows = np.arange(T)
    log(f"case moe small batch T={T} align={align} unsorted={aa.moe_lora_plan(T, c.k, c.R)}")
    y = run_moe(W13, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx, c.slot_rank, c.scale,
                c.E, align=align)
    bounds.check_bf16_tolerance(y, oracle_rows(oracle_mod, c, 0, rows))
    y = run_moe(W2, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx, c.slot_rank, c.scale,
                c.E, align=align)
    bounds.check_bf16_tolerance(y, oracle_rows(oracle_mod, c, 1, rows))


def test_moe_per_expert_layout(oracle_mod):
    """The non-shared layout (expert dim E on every tensor) at a reduced size."""
    c = synth.make_moe("per_expert", 256, 4, 16, 512, 384, 16, 4, "bf16", 77, shared_outer=False)
    rows = np.arange(c.T)
    log("case moe per-expert")
    y = run_moe(W13, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx, c.slot_rank, c.scale,
                c.E)
    bounds.check_bf16_tolerance(y, oracle_rows(oracle_mod, c, 0, rows))
    y = run_moe(W2, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx, c.slot_rank, c.scale,
                c.E)
    bounds.check_bf16_tolerance(y, oracle_rows(oracle_mod, c, 1, rows))


@pytest.mark.parametrize("seed,T,k,E,L,bm", [(0, 7, 2, 4, 3, 4), (1, 2048, 8, 64, 8, 16),
                                              (2, 1, 1, 1, 1, 1), (3, 333, 3, 5, 6, 8),
                                              # 1024 (slot, expert) keys over 5 work-groups of the
                                              # two-pass segment build
                                              (4, 700, 7, 128, 8, 32)])
def test_moe_align_bit_exact(oracle_mod, seed, T, k, E, L, bm):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)     # includes out-of-range experts
    idx = rng.integers(-1, L + 1, size=T).astype(np.int32)
    rank = (rng.integers(0, 3, size=L) * 16).astype(np.int32)
    cap = aa.moe_lora_align_capacity(T, k, E, bm)
    so = torch.full((L, cap), -7, dtype=torch.int32, device="cuda")
    be = torch.full((L, cap // bm), -7, dtype=torch.int32, device="cuda")
    npp = torch.full((L,), -7, dtype=torch.int32, device="cuda")
    ws = aa.alloc_moe_workspace(T, k, 1, 16, L, E)
    aa.moe_lora_align(dev(ids), dev(idx), dev(rank), E, L, 16, bm, ws, so, be, npp)
    torch.cuda.synchronize()
    eso, ebe, enpp = oracle_mod.moe_align(ids, idx, rank, E, L, bm)
    assert np.array_equal(npp.cpu().numpy(), enpp)
    assert np.array_equal(so.cpu().numpy(), eso)
    assert np.array_equal(be.cpu().numpy(), ebe)


def test_moe_passthrough_and_zero_b(oracle_mod):
    """Tokens without adapter keep their rows bit-exact; zero lora_b leaves
    every row bit-exact."""
    c = synth.make_moe("pt", 200, 4, 8, 256, 128, 16, 3, "bf16", 5,
                       idx=np.where(np.arange(200) % 3 == 0, -1, np.arange(200) % 3).astype(np.int32),
                       slot_rank=np.array([16, 0, 16], np.int32))
    y = run_moe(W13, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx, c.slot_rank, c.scale,
                c.E)
    dead = [p for p in range(c.T * c.k) if c.idx[p // c.k] < 0 or c.slot_rank[c.idx[p // c.k]] == 0]
    assert np.array_equal(y[dead].view(np.uint32), c.gate_up0[dead].view(np.uint32))
    Bz = [np.zeros_like(b) for b in c.B13]
    y = run_moe(W13, c.gate_up0, c.x, c.A13, Bz, c.topk_ids, None, c.idx, c.slot_rank, c.scale, c.E)
    assert np.array_equal(y.view(np.uint32), c.gate_up0.view(np.uint32))


@pytest.mark.parametrize("T,align", [(64, False), (64, True), (2048, True)])
def test_side_stream_equals_default_stream(T, align):
    """The fused-MoE calls (the alignment, w13 and w2) on a stream of their own,
    with the default stream current, give the same bits as on the default
    stream, without alignment and with it."""
    c = synth.config_moe(T=T)
    ids, idx, rank, scale = dev(c.topk_ids), dev(c.idx), dev(c.slot_rank), dev(c.scale)
    tw = dev(c.topk_w)
    x, h = dev(c.x, BF), dev(c.h, BF)
    A13, B13 = [dev(a, BF) for a in c.A13], [dev(b, BF) for b in c.B13]
    A2, B2 = [dev(c.A2, BF)], [dev(c.B2, BF)]
    L, R = c.A13[0].shape[0], c.A13[0].shape[2]
    ws = aa.alloc_moe_workspace(T, c.k, 2, R, L, c.E)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def call(stream):
        g, o = dev(c.gate_up0, BF), dev(c.out0, BF)
        flags = 0
        if stream is not None:
            stream.wait_stream(main)
        if align:
            aa.moe_lora_align(ids, idx, rank, c.E, L, R, 16, ws, stream=stream)
            flags = aa.LORA_FLAG_SEGMENTS_READY
        aa.moe_lora_apply(W13, g, x, A13, B13, ids, None, idx, rank, scale, c.E, ws, flags=flags,
                          stream=stream)
        aa.moe_lora_apply(W2, o, h, A2, B2, ids, tw, idx, rank, scale, c.E, ws, flags=flags,
                          stream=stream)
        if stream is not None:
            main.wait_stream(stream)
        torch.cuda.synchronize()
        return host_f32(g), host_f32(o)

    log(f"case moe side stream T={T} align={align}")
    want = call(None)
    for rnd in range(2):
        got = call(side)
        for w_, g_ in zip(want, got):
            assert np.array_equal(g_.view(np.uint32), w_.view(np.uint32)), rnd


def window(t, lead, tail, fill):
    """t's values as a column window of wider rows (the other columns = fill)."""
    T, K = t.shape
    wide = torch.full((T, lead + K + tail), fill, dtype=t.dtype, device=t.device)
    wide[:, lead:lead + K] = t
    return wide, wide[:, lead:lead + K]


@pytest.mark.parametrize("T,align", [(64, False), (64, True), (512, True)])
def test_row_strides_wider_than_rows(T, align):
    """x / h and y given as windows of wider rows (row strides past K and N,
    starting 16 columns in) give the bits of contiguous tensors, and the
    columns outside the windows keep their values."""
    c = synth.config_moe(T=T)
    args13 = (c.gate_up0, c.x, c.A13, c.B13, None)
    args2 = (c.out0, c.h, [c.A2], [c.B2], c.topk_w)
    for kind, (y0, xin, A, B, tw) in ((W13, args13), (W2, args2)):
        log(f"case moe row strides T={T} align={align} kind={kind}")
        L, _, R, _ = A[0].shape
        want = run_moe(kind, y0, xin, A, B, c.topk_ids, tw, c.idx, c.slot_rank, c.scale, c.E,
                       align=align, guard=False)
        ws = aa.alloc_moe_workspace(T, c.k, len(A), R, L, c.E)
        flags = 0
        if align:
            aa.moe_lora_align(dev(c.topk_ids), dev(c.idx), dev(c.slot_rank), c.E, L, R, 16, ws)
            flags = aa.LORA_FLAG_SEGMENTS_READY
        _, xs = window(dev(xin, BF), 16, 48, 1024.0)
        ywide, ys = window(dev(y0, BF), 16, 16, -7.0)
        aa.moe_lora_apply(kind, ys, xs, [dev(a, BF) for a in A], [dev(b, BF) for b in B],
                          dev(c.topk_ids), None if tw is None else dev(tw), dev(c.idx),
                          dev(c.slot_rank), dev(c.scale), c.E, ws, flags=flags)
        torch.cuda.synchronize()
        got = host_f32(ys)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        outside = torch.cat([ywide[:, :16], ywide[:, 16 + ys.shape[1]:]], dim=1)
        assert bool(torch.all(outside == -7.0))
