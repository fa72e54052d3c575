"""Seeded random sweep over shapes and paths, integer vectors, bit for bit
against the oracle.

Each case draws its own shape (tokens, hidden size, slices and their widths,
rank, slots, slot ranks with zeros, tokens without an adapter or with an
out-of-range slot, a column offset into a wider y, one lora_a shared by every
slice or not) and runs lora_apply_packed on auto and on every path that takes
the shape (the library's own lora_plan_packed decides which).  x, A, B are in
{-1, 0, 1} and y0 is an integer, so every partial sum is exact and each path
must equal the oracle exactly; the columns of y outside the slices and the
canary bands around y stay untouched; an fp32 part does the same on the
paths that take fp32.  The fused-MoE half draws
(T, top_k, E, K, I, rank, slots) with out-of-range experts, one lora_a / lora_b
shared by the experts or not, the aligned path or the one without alignment,
and the k-reduced w2."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import adapter_apply_amd as aa  # noqa: E402
import synth  # noqa: E402
from tests import bounds  # noqa: E402
from tests.gpu_util import canaries_intact, dev, guarded, host_f32, log  # noqa: E402
from tests.test_gpu_moe import W13, W2, integer_moe, run_moe  # noqa: E402

PATHS = [aa.LORA_PATH_AUTO, aa.LORA_PATH_DECODE, aa.LORA_PATH_PREFILL, aa.LORA_PATH_FUSED,
         aa.LORA_PATH_GROUPED, aa.LORA_PATH_RELAY, aa.LORA_PATH_TOKEN]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aa.lib()


def draw_linear(rng):
    T = int(np.exp(rng.uniform(0.0, np.log(1200.0))))
    K = int(rng.choice([64, 256, 512, 1000, 1024, 2048, 2056, 4096]))
    S = int(rng.integers(1, 5))
    N = [int(rng.choice([8, 64, 200, 256, 520, 1024, 1032, 2048])) for _ in range(S)]
    if rng.random() < 0.15:
        N[0] = int(rng.choice([12, 36]))            # not a multiple of 8
    R = int(rng.choice([8, 16, 16, 24, 32, 32, 64, 128]))   # bf16 rows: R % 8 == 0
    L = int(rng.choice([1, 2, 3, 8, 16, 40, 100, 200]))
    return T, K, N, R, L


@pytest.mark.parametrize("case", range(120))
def test_linear_sweep_bit_exact(oracle_mod, case):
    rng = np.random.default_rng(9000 + case)
    T, K, N, R, L = draw_linear(rng)
    shared = len(N) > 1 and rng.random() < 0.3
    c = synth.make_integer_linear(T, K, N, R, L, seed=9100 + case, dtype="bf16",
                                  p_none=float(rng.choice([0.0, 0.1, 0.5])))
    rank = c.slot_rank.copy()
    rank[rng.random(L) < 0.2] = 0                    # slots switched off
    idx = c.idx.copy()
    idx[rng.random(T) < 0.05] = L + 3                # out-of-range slot: no adapter
    A = [c.A[0]] * len(N) if shared else c.A
    if shared:                                       # zero rows past each slot's rank, as every slice
        for s in range(L):
            A[0][s, rank[s]:] = 0
    for b in c.B:
        for s in range(L):
            b[s, :, rank[s]:] = 0
    ncol = int(sum(N))
    off = int(rng.choice([0, 0, 8, 24, 4]))
    pad = int(rng.choice([0, 8, 40]))
    y_host = rng.integers(-8, 9, size=(T, off + ncol + pad)).astype(np.float32)
    ref = oracle_mod.lora_apply(y_host[:, off:off + ncol].copy(), c.x, A, c.B, idx, rank, c.scale)[0]
    exact = bounds.linear_exact_int_by_slot(c.x, A, c.B, idx, rank, c.scale, y_host[:, off:off + ncol])
    assert np.array_equal(ref, exact.astype(np.float32))

    bf = torch.bfloat16
    x = dev(c.x, bf)
    Ad = [dev(A[0], bf)] * len(N) if shared else [dev(a, bf) for a in A]
    Bd = [dev(b, bf) for b in c.B]
    idx_d, rank_d, scale_d = dev(idx), dev(rank), dev(c.scale)
    ws = aa.alloc_workspace(T, K, len(N), R, L)
    log(f"case sweep {case}: T={T} K={K} N={N} R={R} L={L} shared={shared} off={off}")
    ran = []
    for path in PATHS:
        yfull, y = guarded(y_host, bf)
        try:
            taken = aa.lora_plan_packed(y, x, Ad, Bd, idx_d, rank_d, scale_d, ws,
                                        y_col_offset=off, path=path)
        except aa.LoraError as e:
            assert path != aa.LORA_PATH_AUTO and e.code == aa.LORA_E_PATH, str(e)
            continue
        aa.lora_apply_packed(y, x, Ad, Bd, idx_d, rank_d, scale_d, ws, y_col_offset=off, path=path)
        got = host_f32(y)
        assert np.array_equal(got[:, off:off + ncol], ref), \
            f"path {aa.PATH_NAMES[taken]}: max diff {np.max(np.abs(got[:, off:off + ncol] - ref))}"
        assert np.array_equal(got[:, :off], y_host[:, :off])
        assert np.array_equal(got[:, off + ncol:], y_host[:, off + ncol:])
        assert canaries_intact(yfull)
        ran.append(aa.PATH_NAMES[taken])
    aa.lora_workspace_check(ws)                      # raises if a hand-over wait gave up
    log(f"  paths {ran}")


@pytest.mark.parametrize("case", range(40))
def test_fp32_sweep_bit_exact(oracle_mod, case):
    """fp32 on the paths that take it (auto, DECODE, TOKEN): random shapes,
    ranks in steps of 4, slots switched off, out-of-range slots and a column
    offset, bit for bit against the oracle."""
    rng = np.random.default_rng(9800 + case)
    T = int(np.exp(rng.uniform(0.0, np.log(600.0))))
    K = int(rng.choice([8, 64, 520, 1024, 4096]))
    S = int(rng.integers(1, 4))
    N = [int(rng.choice([4, 64, 252, 256, 1028, 4096])) for _ in range(S)]
    R = int(rng.choice([4, 8, 12, 16, 32, 64]))
    L = int(rng.choice([1, 3, 8, 40]))
    c = synth.make_integer_linear(T, K, N, R, L, seed=9900 + case, dtype="f32",
                                  p_none=float(rng.choice([0.0, 0.2])))
    rank = c.slot_rank.copy()
    rank[rng.random(L) < 0.2] = 0
    idx = c.idx.copy()
    idx[rng.random(T) < 0.05] = L + 1
    for b in c.B:
        for sl in range(L):
            b[sl, :, rank[sl]:] = 0
    ncol = int(sum(N))
    off = int(rng.choice([0, 4, 12]))
    y_host = rng.integers(-8, 9, size=(T, off + ncol + 4)).astype(np.float32)
    ref = oracle_mod.lora_apply(y_host[:, off:off + ncol].copy(), c.x, c.A, c.B, idx, rank, c.scale)[0]
    f32 = torch.float32
    x = dev(c.x, f32)
    Ad, Bd = [dev(a, f32) for a in c.A], [dev(b, f32) for b in c.B]
    idx_d, rank_d, scale_d = dev(idx), dev(rank), dev(c.scale)
    ws = aa.alloc_workspace(T, K, len(N), R, L)
    log(f"case fp32 sweep {case}: T={T} K={K} N={N} R={R} L={L} off={off}")
    ran = []
    for path in (aa.LORA_PATH_AUTO, aa.LORA_PATH_DECODE, aa.LORA_PATH_TOKEN):
        yfull, y = guarded(y_host, f32)
        taken = aa.lora_plan_packed(y, x, Ad, Bd, idx_d, rank_d, scale_d, ws, y_col_offset=off,
                                    path=path)
        aa.lora_apply_packed(y, x, Ad, Bd, idx_d, rank_d, scale_d, ws, y_col_offset=off, path=path)
        got = host_f32(y)
        assert np.array_equal(got[:, off:off + ncol], ref), \
            f"path {aa.PATH_NAMES[taken]}: max diff {np.max(np.abs(got[:, off:off + ncol] - ref))}"
        assert np.array_equal(got[:, :off], y_host[:, :off])
        assert np.array_equal(got[:, off + ncol:], y_host[:, off + ncol:])
        assert canaries_intact(yfull)
        ran.append(aa.PATH_NAMES[taken])
    log(f"  paths {ran}")


@pytest.mark.parametrize("case", range(48))
def test_moe_sweep_bit_exact(oracle_mod, case):
    rng = np.random.default_rng(9500 + case)
    T = int(np.exp(rng.uniform(0.0, np.log(700.0))))
    k = int(rng.choice([1, 2, 4, 6, 8]))
    E = int(rng.choice([1, 4, 16, 64]))
    k = min(k, E)
    K = int(rng.choice([64, 256, 1024, 2048]))
    I = int(rng.choice([64, 128, 512]))
    R = int(rng.choice([16, 16, 32, 64]))
    L = int(rng.choice([1, 3, 8]))
    shared = bool(rng.random() < 0.6)
    d = integer_moe(9600 + case, T, k, E, K, I, R, L, shared, p_none=float(rng.choice([0.0, 0.2])))
    ids = d["ids"].copy()
    bad = rng.random(ids.shape) < 0.05
    ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + 2)
    rank = d["rank"].copy()
    if L > 1:
        rank[0] = 0
    aligns = (False, True) if aa.moe_lora_plan(T, k, R) else (False,)
    log(f"case moe sweep {case}: T={T} k={k} E={E} K={K} I={I} R={R} L={L} shared={shared}")
    ref13 = oracle_mod.moe_lora_apply(0, d["g0"], d["x"], d["A13"], d["B13"], ids, None, d["idx"],
                                      rank, d["scale"], E)
    ref2 = oracle_mod.moe_lora_apply(1, d["o0"], d["h"], [d["A2"]], [d["B2"]], ids, d["w"],
                                     d["idx"], rank, d["scale"], E)
    for align in aligns:
        y = run_moe(W13, d["g0"], d["x"], d["A13"], d["B13"], ids, None, d["idx"], rank, d["scale"],
                    E, align=align)
        assert np.array_equal(y, ref13), f"w13 align={align}: {np.max(np.abs(y - ref13))}"
        y = run_moe(W2, d["o0"], d["h"], [d["A2"]], [d["B2"]], ids, d["w"], d["idx"], rank,
                    d["scale"], E, align=align)
        assert np.array_equal(y, ref2), f"w2 align={align}: {np.max(np.abs(y - ref2))}"
    if shared:
        z = np.zeros((T, K), np.float32)
        y = run_moe(W2, z, d["h"], [d["A2"]], [d["B2"]], ids, d["w"], d["idx"], rank, d["scale"], E,
                    reduce_k=True)
        ref = oracle_mod.moe_lora_apply(1, z, d["h"], [d["A2"]], [d["B2"]], ids, d["w"], d["idx"],
                                        rank, d["scale"], E, reduce_k=True)
        assert np.array_equal(y, ref), f"w2 reduced: {np.max(np.abs(y - ref))}"
