"""GPU parity of the linear (packed-slice) path against the CPU oracle, through
the C ABI.  Both paths (decode VALU, prefill MFMA) are forced on the same
inputs where they apply.  Tolerance for bf16 outputs: max abs error <= 2e-2
and normwise relative error <= 1e-2 against the fp32 oracle; fp32 outputs
within the a-priori fp32 rounding bound; integer-exact vectors and every
passthrough row bit-exact."""
import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import adapter_apply_amd as aa  # noqa: E402
import synth  # noqa: E402
from tests import bounds, oracle_par  # noqa: E402
from tests.gpu_util import LinearOnDevice, canaries_intact, dev, host_f32, log  # noqa: E402

DEC, PRE, FUS, GRP, RLY, TOK = (aa.LORA_PATH_DECODE, aa.LORA_PATH_PREFILL, aa.LORA_PATH_FUSED,
                                aa.LORA_PATH_GROUPED, aa.LORA_PATH_RELAY, aa.LORA_PATH_TOKEN)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aa.lib()


def passthrough_rows(c):
    return [t for t in range(c.T)
            if c.idx[t] < 0 or c.idx[t] >= c.L or c.slot_rank[c.idx[t]] <= 0]


def assert_passthrough(c, y):
    rows = passthrough_rows(c)
    if rows:
        got = y[rows]
        exp = c.y0[rows]
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), "passthrough row changed"


def oracle_y(oracle_mod, c, rows=None):
    if rows is None:
        y, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
        return y
    rows = np.asarray(rows)
    y, _ = oracle_mod.lora_apply(c.y0[rows], c.x[rows], c.A, c.B, c.idx[rows], c.slot_rank, c.scale)
    return y


# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, TOK])
def test_tiny_fp32_decode(oracle_mod, path):
    c = synth.config_tiny()
    log(f"case tiny fp32 T={c.T} path={path}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    M = bounds.linear_magnitude(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.all(np.abs(y - ref) <= bounds.fp32_bound(M, c.K, c.R))
    assert_passthrough(c, y)
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, TOK])
@pytest.mark.parametrize("seed,T,K,N,R,L", [
    (61, 16, 64, [64], 4, 3),                      # the fp32 workload's shape
    (62, 64, 4096, [4096, 1024, 1024], 16, 8),     # QKV at 64 tokens: auto takes TOKEN
    (63, 300, 520, [36, 1028], 12, 5),             # ragged columns, rank 12: one 16-row pass
    (64, 1, 8, [4], 4, 1),                         # one token, K 8, one 4-column slice
    (65, 40, 1024, [300], 40, 3),                  # rank 40: three passes of the token shrink
])
def test_fp32_integer_vectors_bit_exact(oracle_mod, path, seed, T, K, N, R, L):
    """fp32 on the paths that take it (the split VALU kernels, the one-launch
    token kernel and auto's choice between them): integer vectors, bit for bit."""
    c = synth.make_integer_linear(T, K, N, R, L, seed=seed, dtype="f32")
    log(f"case fp32 integer path={path} T={T} K={K} N={N} R={R} L={L}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    exact = bounds.linear_exact_int(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(ref, exact.astype(np.float32))
    assert np.array_equal(y, ref), f"max diff {np.max(np.abs(y - ref))}"
    assert canaries_intact(d.yfull)


def fusable(c):
    """Shapes the single-launch decode kernel takes."""
    return (c.dtype == "bf16" and c.R % 16 == 0 and c.R <= 32 and c.T <= 1024
            and c.K % 1024 == 0 and all(n % 8 == 0 for n in c.N))


def groupable(c):
    """Shapes the slot-grouped split decode kernels take."""
    return (c.dtype == "bf16" and c.R % 16 == 0 and c.R <= 128 and c.T <= 4096
            and c.K % 64 == 0 and c.K <= 8192 and all(n % 8 == 0 for n in c.N))


def relayable(c):
    """Shapes the single-launch decode kernel with the K-split shrink takes."""
    return (c.dtype == "bf16" and c.R in (16, 32) and c.T <= 1024 and c.L <= 64
            and c.K % 256 == 0 and c.K <= 8192 and all(n % 8 == 0 for n in c.N))


def skip_unless_path_takes(path, c):
    if path == FUS and not fusable(c):
        pytest.skip("shape outside the single-launch kernel")
    if path == RLY and not relayable(c):
        pytest.skip("shape outside the single-launch K-split kernel")
    if path == GRP and not groupable(c):
        pytest.skip("shape outside the slot-grouped kernels")


INTEGER_CASES = [
    (21, 200, 512, [256, 64, 64], 16, 5),
    (22, 333, 1024, [128, 128], 32, 3),
    (23, 97, 2056, [520], 64, 7),          # K not a multiple of the K chunk, ragged tail
    (24, 1, 64, [4], 16, 1),
    (25, 1024, 256, [16, 1028], 48, 1024),   # one token per slot, 1024 slots
    (26, 200, 1024, [256, 64, 64], 16, 5),
    (27, 333, 2048, [1032, 128], 32, 3),     # last 1024-column chunk partial
    (28, 1, 1024, [8], 16, 1),
    (29, 1024, 1024, [16, 1032], 32, 1024),
    (30, 1024, 1024, [256, 64], 16, 40),     # 40 slots x 16 token chunks: work-group discovery
    (31, 300, 1024, [512, 64], 128, 9),      # rank 128
    (32, 1500, 2048, [512, 264], 128, 100),  # 100 slots, rank 128: K-split shrink on the MFMA paths
    (33, 64, 1024, [32768], 16, 4),          # one vocabulary-wide slice (lm_head LoRA)
    (34, 150, 1024, [256, 64], 512, 3),      # the largest rank the library takes
    (35, 400, 512, [128, 200], 256, 5),      # rank 256: several 128-rank passes
    (36, 1024, 8192, [1024, 264], 32, 64),   # the K-split single launch at its largest T, K, L
    (37, 256, 8192, [20480], 16, 8),         # ... with 16-token expand items over 32 K chunks
]


@pytest.mark.parametrize("path", [DEC, PRE, FUS, GRP, RLY, TOK])
@pytest.mark.parametrize("seed,T,K,N,R,L", INTEGER_CASES)
def test_integer_vectors_bit_exact(oracle_mod, path, seed, T, K, N, R, L):
    c = synth.make_integer_linear(T, K, N, R, L, seed=seed, dtype="bf16")
    skip_unless_path_takes(path, c)
    log(f"case integer path={path} T={T} K={K} N={N} R={R} L={L}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    exact = bounds.linear_exact_int(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(ref, exact.astype(np.float32))
    assert np.array_equal(y, ref), f"max diff {np.max(np.abs(y - ref))}"
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("path", [DEC, PRE, FUS, GRP, RLY, TOK])
def test_decode_config_qkv(oracle_mod, path):
    """256 tokens, hidden 4096, QKV 4096/1024/1024, rank 16, 8 slots, 10% idx=-1."""
    c = synth.config_decode()
    log(f"case decode_qkv path={path}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    err, rel = bounds.check_bf16_tolerance(y, ref)
    log(f"  max abs err {err:.3e} rel {rel:.3e}")
    assert_passthrough(c, y)
    assert canaries_intact(d.yfull)


def test_prefill_config_gate_up_full(oracle_mod):
    """8192 tokens in 32 sequences, 16 slots, gate_up 2x14336, rank 64, on the
    auto path (the MFMA tile kernels): all 8192 x 28672 outputs against the
    oracle (run in token blocks on the host cores)."""
    c = synth.config_prefill()
    log("case prefill_gate_up full size (auto path)")
    d = LinearOnDevice(c)
    d.apply(aa.LORA_PATH_AUTO)
    y = d.y_host()
    assert canaries_intact(d.yfull)
    ref = oracle_par.lora_apply(oracle_mod, c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    err, rel = bounds.check_bf16_tolerance(y, ref)
    log(f"  all {c.T} x {c.Ntot} outputs: max abs err {err:.3e} rel {rel:.3e}")


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, PRE])
def test_prefill_config_shape_integer_bit_exact(oracle_mod, path):
    """Integer vectors at exactly the prefill workload's shape (8192 tokens in
    its 32 sequences, 16 slots, hidden 4096, gate_up 2x14336, rank 64): every
    output bit-exact, so each of the persistent expand's items (about 30 per
    work-group here) and each shrink tile is checked at full size."""
    c0 = synth.config_prefill()
    c = synth.make_integer_linear(c0.T, c0.K, c0.N, c0.R, c0.L, seed=71, idx=c0.idx,
                                  slot_rank=np.full(c0.L, c0.R, np.int32))
    del c0
    log(f"case prefill-shape integer path={path}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    assert canaries_intact(d.yfull)
    ref = oracle_par.lora_apply(oracle_mod, c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    exact = bounds.linear_exact_int_by_slot(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(ref, exact.astype(np.float32))
    bad = np.argwhere(y != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("path", [DEC, PRE])
def test_prefill_shape_reduced_both_paths(oracle_mod, path):
    """Prefill-shaped (long per-slot runs) at a size the oracle checks fully."""
    rng = np.random.default_rng(7)
    lens = synth.prefill_lengths(rng, n_seq=6, total=1200, lo=64, hi=400)
    idx = np.repeat(rng.integers(0, 4, size=6), lens).astype(np.int32)
    c = synth.make_linear("prefill_small", 1200, 768, [1024, 1024], 64, 4, idx, [64, 48, 16, 64],
                          [1.0, 0.5, 2.0, 1.0], "bf16", seed=8)
    log(f"case prefill_small path={path}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    bounds.check_bf16_tolerance(y, ref)
    assert canaries_intact(d.yfull)


def test_logits_vocab_32000_every_path(oracle_mod):
    """lm_head LoRA: 256 decode tokens, hidden 4096, vocabulary 32000 (the
    smallest the logits layer accepts), rank 16, 8 slots; every path against
    one oracle result."""
    c = synth.config_logits(vocab=32000)
    ref = oracle_y(oracle_mod, c)
    for path in (aa.LORA_PATH_AUTO, DEC, PRE, FUS, GRP, RLY, TOK):
        log(f"case logits vocab=32000 path={path}")
        d = LinearOnDevice(c)
        d.apply(path)
        y = d.y_host()
        err, rel = bounds.check_bf16_tolerance(y, ref)
        log(f"  max abs err {err:.3e} rel {rel:.3e}")
        assert_passthrough(c, y)
        assert canaries_intact(d.yfull)


def test_logits_vocab_128256_auto(oracle_mod):
    """The lm_head workload at its measured size (vocabulary 128256) on the
    auto path, which takes the K-split single launch (expand items of four
    512-column chunks) for outputs this wide."""
    c = synth.config_logits()
    log("case logits vocab=128256 auto")
    d = LinearOnDevice(c)
    d.apply(aa.LORA_PATH_AUTO)
    y = d.y_host()
    err, rel = bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
    log(f"  max abs err {err:.3e} rel {rel:.3e}")
    assert_passthrough(c, y)
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, GRP])
def test_many_adapter_config(oracle_mod, path):
    """1024 tokens, 128 slots with Zipf(1.1) popularity, ranks {8..128} padded to 128."""
    c = synth.config_many()
    log(f"case many_adapter path={path}")
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    err, rel = bounds.check_bf16_tolerance(y, ref)
    log(f"  max abs err {err:.3e} rel {rel:.3e}")
    assert canaries_intact(d.yfull)


def test_many_adapter_shape_integer_bit_exact(oracle_mod):
    """Integer vectors at exactly the many-adapter workload's shape (1024
    tokens, 128 slots with Zipf(1.1) popularity and its slot ranks {8..128}
    padded to 128, hidden and output 8192) on auto and PREFILL, which take the
    tile kernels: the shrink split over K and its ordered reduce, and the
    rank-128 persistent expand with its loads masked to the rows and rank
    units that exist and its LDS writes limited to them.  Every output bit
    for bit."""
    m = synth.config_many()
    c = synth.make_integer_linear(m.T, m.K, m.N, m.R, m.L, seed=1010, idx=m.idx,
                                  slot_rank=m.slot_rank)
    del m
    ref = oracle_par.lora_apply(oracle_mod, c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    exact = bounds.linear_exact_int_by_slot(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(ref, exact.astype(np.float32))
    for path in (aa.LORA_PATH_AUTO, PRE):
        d = LinearOnDevice(c)
        taken = aa.lora_plan_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
        log(f"case many-adapter-shape integer path={aa.PATH_NAMES[path]}")
        assert taken == PRE, aa.PATH_NAMES[taken]
        d.apply(path)
        y = d.y_host()
        assert canaries_intact(d.yfull)
        bad = np.argwhere(y != ref)
        assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:4].tolist()}"


def test_many_adapter_separate_calls_auto(oracle_mod):
    """lora_shrink then lora_expand on auto, apart, for the many-slot batch:
    both take the tile kernels and exchange the token-ordered buffer."""
    c = synth.config_many(T=512)
    log("case many_adapter separate calls (auto)")
    d = LinearOnDevice(c)
    buf = torch.full((c.S, c.T, c.R), 3.0, dtype=torch.float32, device="cuda")
    aa.lora_shrink(buf, d.x, d.A, d.idx, d.rank, d.ws)
    aa.lora_expand(d.y, buf, d.B, d.idx, d.rank, d.scale, d.ws)
    y = d.y_host()
    bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
    assert canaries_intact(d.yfull)


def test_many_adapter_alpha_scales(oracle_mod):
    c = synth.config_many(T=512, scale_mode="alpha")
    log("case many_adapter alpha scales")
    d = LinearOnDevice(c)
    d.apply(DEC)
    bounds.check_bf16_tolerance(d.y_host(), oracle_y(oracle_mod, c))


# ---------------------------------------------------------------------------
# shrink and expand as separate entry points
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", [DEC, PRE, GRP])
def test_shrink_buffer(oracle_mod, path):
    c = synth.make_linear("sh", 300, 1024, [256, 128], 32, 5,
                          idx=np.random.default_rng(3).integers(-1, 6, 300),
                          slot_rank=[32, 8, 0, 16, 24], scale=[1, 1, 1, 1, 1], dtype="bf16",
                          seed=31)
    log(f"case shrink path={path}")
    d = LinearOnDevice(c)
    buf = torch.full((c.S, c.T, c.R), 123.0, dtype=torch.float32, device="cuda")
    aa.lora_shrink(buf, d.x, d.A, d.idx, d.rank, d.ws, path=path)
    g = host_f32(buf)
    ref = oracle_mod.lora_shrink(c.x, c.A, c.idx, c.slot_rank)
    # both sides sum exact bf16 products in fp32; only the order differs
    Mb = np.zeros_like(ref, dtype=np.float64)
    for sg, a in enumerate(c.A):
        for t in range(c.T):
            s = c.idx[t]
            if 0 <= s < c.L and c.slot_rank[s] > 0:
                Mb[sg, t] = np.abs(a[s].astype(np.float64)) @ np.abs(c.x[t].astype(np.float64))
    assert np.all(np.abs(g - ref) <= 2 * bounds.gamma(c.K) * Mb + 0.0)
    zero_mask = ref == 0
    assert np.all(g[zero_mask & (Mb == 0)] == 0)


@pytest.mark.parametrize("path", [DEC, PRE, GRP])
def test_expand_from_given_buffer(oracle_mod, path):
    rng = np.random.default_rng(41)
    c = synth.make_linear("ex", 257, 64, [512, 128, 128], 32, 6, idx=rng.integers(-1, 7, 257),
                          slot_rank=[32, 16, 8, 32, 0, 24], scale=[2, 1, .5, 1, 1, 3],
                          dtype="bf16", seed=42)
    buf = rng.standard_normal((c.S, c.T, c.R)).astype(np.float32)
    if path in (PRE, GRP):
        # the MFMA expands consume the buffer in bf16; give them bf16-exact values
        buf = synth.round_bf16(buf)
    log(f"case expand path={path}")
    d = LinearOnDevice(c)
    aa.lora_expand(d.y, dev(buf), d.B, d.idx, d.rank, d.scale, d.ws, path=path)
    y = d.y_host()
    ref = oracle_mod.lora_expand(c.y0, buf, c.B, c.idx, c.slot_rank, c.scale)
    bounds.check_bf16_tolerance(y, ref)
    assert_passthrough(c, y)
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("cfg,path", [("decode", DEC), ("many", DEC), ("decode", GRP),
                                      ("many64", GRP)])
def test_partial_flag_split_calls(oracle_mod, cfg, path):
    """lora_shrink(PARTIAL) + lora_expand(PARTIAL): partial sums stay in the
    workspace, the caller's buffer is never touched.  many64: 128 slots, so the
    grouped kernels read their groups from the segment table."""
    c = (synth.config_decode(T=200) if cfg == "decode" else
         synth.config_many(T=300, R=64, K=2048, N=1024) if cfg == "many64" else
         synth.config_many(T=300))
    log(f"case partial flag {cfg} path={path}")
    d = LinearOnDevice(c)
    buf = torch.full((c.S, c.T, c.R), 5.0, dtype=torch.float32, device="cuda")
    aa.lora_shrink(buf, d.x, d.A, d.idx, d.rank, d.ws, path=path, flags=aa.LORA_FLAG_PARTIAL)
    aa.lora_expand(d.y, buf, d.B, d.idx, d.rank, d.scale, d.ws, path=path,
                   flags=aa.LORA_FLAG_PARTIAL | aa.LORA_FLAG_SEGMENTS_READY)
    y = d.y_host()
    assert bool(torch.all(buf == 5.0))
    bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
    assert_passthrough(c, y)
    assert canaries_intact(d.yfull)


# ---------------------------------------------------------------------------
# segments and edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,T,L", [(0, 1, 1), (1, 256, 8), (2, 8192, 16), (3, 1000, 128),
                                      (4, 4097, 1024), (5, 70, 3), (6, 20000, 5)])
def test_segments_bit_exact(oracle_mod, seed, T, L):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-2, L + 2, size=T).astype(np.int32)
    rank = rng.integers(0, 3, size=L).astype(np.int32) * 8
    log(f"case segments T={T} L={L}")
    ws = aa.alloc_workspace(T, 64, 1, 16, L)
    for _ in range(3):      # a build leaves its exchange region zero for the next one
        aa.lora_build_segments(dev(idx), dev(rank), L, 16, ws)
    torch.cuda.synchronize()
    # the end area (exchange regions of the single-launch build): zero again
    n_wg = -(-T // 1024)
    xb = 0 if T <= 4096 else (-(-4 * min(n_wg, 16) * (L + 1) // 256) * 256 + 256)
    assert int(torch.count_nonzero(ws[ws.numel() - 256 - xb:])) == 0
    lay = aa.lora_segment_layout(T, L)
    w = ws.cpu().numpy()

    def ints(off, n):
        return w[off:off + 4 * n].view(np.int32)

    perm, start, ninv = oracle_mod.segments(idx, rank, L, 16)
    hdr = ints(lay["header"], 4)
    assert hdr[0] == start[L] and hdr[1] == ninv
    assert np.array_equal(ints(lay["slot_start"], L + 1), start)
    assert np.array_equal(ints(lay["perm"], T), perm)
    for key, G, k in (("tiles_decode", lay["tile_decode_tokens"], 2),
                      ("tiles_prefill", lay["tile_prefill_tokens"], 3)):
        tiles = ints(lay[key], 4 * hdr[k]).reshape(-1, 4)
        exp = [(s, b, min(b + G, start[s + 1]))
               for s in range(L) for b in range(start[s], start[s + 1], G)]
        assert [tuple(t[:3]) for t in tiles] == exp


def test_all_tokens_without_adapter_unchanged():
    c = synth.config_decode(T=64)
    c.idx[:] = -1
    d = LinearOnDevice(c)
    for path in (DEC, PRE, FUS, GRP, RLY, TOK):
        d.apply(path)
        y = d.y_host()
        assert np.array_equal(y.view(np.uint32), c.y0.view(np.uint32))
    assert canaries_intact(d.yfull)


def test_zero_b_identity_and_invalid_slots(oracle_mod):
    c = synth.config_decode(T=128)
    c.idx[::7] = 8        # >= L: passthrough
    c.idx[::11] = 100
    c.slot_rank[3] = 0    # empty slot
    c.B = [np.zeros_like(b) for b in c.B]
    for path in (DEC, PRE, FUS, GRP, RLY, TOK):
        d = LinearOnDevice(c)
        d.apply(path)
        y = d.y_host()
        assert np.array_equal(y.view(np.uint32), c.y0.view(np.uint32))


def test_column_offset_and_wide_rows(oracle_mod):
    """y_col_offset > 0 inside a wider row: the columns outside the packed
    slices stay bit-identical."""
    rng = np.random.default_rng(5)
    c = synth.make_linear("off", 90, 1024, [64, 32], 16, 3, idx=rng.integers(-1, 3, 90),
                          slot_rank=[16, 8, 16], scale=[1, 2, 1], dtype="bf16", seed=6)
    wide = rng.standard_normal((c.T, 200)).astype(np.float32)
    wide = synth.round_bf16(wide)
    off = 40
    for path in (DEC, PRE, FUS, GRP, RLY, TOK):
        yw = dev(wide, torch.bfloat16)
        d = LinearOnDevice(c, guard=False)
        aa.lora_apply_packed(yw, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, y_col_offset=off,
                             path=path)
        got = host_f32(yw)
        y0 = wide[:, off:off + c.Ntot]
        ref, _ = oracle_mod.lora_apply(y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
        bounds.check_bf16_tolerance(got[:, off:off + c.Ntot], ref)
        assert np.array_equal(got[:, :off], wide[:, :off])
        assert np.array_equal(got[:, off + c.Ntot:], wide[:, off + c.Ntot:])


@pytest.mark.parametrize("T,L", [(200, 6), (300, 100)])
def test_segments_reused_across_layers(oracle_mod, T, L):
    """Segments built once per batch and reused by several layer shapes (with
    100 slots the grouped kernels read their groups from these segments)."""
    rng = np.random.default_rng(9)
    idx = rng.integers(-1, L, T).astype(np.int32)
    ranks = np.resize(np.array([16, 8, 16, 0, 16, 8], np.int32), L)
    ws = aa.alloc_workspace(T, 2048, 3, 16, L)
    idx_d, rank_d = dev(idx), dev(ranks)
    aa.lora_build_segments(idx_d, rank_d, L, 16, ws)
    for li, (K, N) in enumerate([(512, [256, 64, 64]), (2048, [512]), (256, [128, 128])]):
        c = synth.make_linear(f"layer{li}", T, K, N, 16, L, idx, ranks, [1.5] * L, "bf16",
                              seed=100 + li)
        d = LinearOnDevice(c, guard=False)
        for path in (DEC, PRE, GRP):
            d.reset_y()
            aa.lora_apply_packed(d.y, d.x, d.A, d.B, idx_d, rank_d, d.scale, ws, path=path,
                                 flags=aa.LORA_FLAG_SEGMENTS_READY)
            bounds.check_bf16_tolerance(d.y_host(), oracle_y(oracle_mod, c))


@pytest.mark.parametrize("cfg,path", [("many", DEC), ("decode", FUS), ("decode", PRE),
                                      ("decode", GRP), ("decode", RLY)])
def test_deterministic_run_twice(cfg, path):
    c = synth.config_many(T=512) if cfg == "many" else synth.config_decode()
    outs = []
    for _ in range(2):
        d = LinearOnDevice(c, guard=False)
        d.apply(path)
        outs.append(d.y_host())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("path", [FUS, GRP, RLY])
def test_fused_skewed_slots(oracle_mod, path):
    """All tokens on one slot (many groups of one slot) and ranks below 16."""
    rng = np.random.default_rng(12)
    idx = np.zeros(700, np.int32)
    idx[rng.random(700) < 0.05] = 3
    idx[::50] = -1
    c = synth.make_linear("skew", 700, 1024, [64, 256], 32, 4, idx, [32, 8, 16, 8],
                          [1.0, 1.0, 1.0, 0.5], "bf16", seed=13)
    d = LinearOnDevice(c)
    d.apply(path)
    y = d.y_host()
    bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
    assert_passthrough(c, y)
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("path", [FUS, GRP, RLY])
def test_fused_rejects_unsupported(path):
    # rank 128 is past the single-launch kernels, rank 160 past the grouped ones
    c = synth.config_many(T=64, R=160 if path == GRP else 128)
    d = LinearOnDevice(c, guard=False)
    with pytest.raises(aa.LoraError) as e:
        d.apply(path)
    assert e.value.code == aa.LORA_E_PATH


@pytest.mark.parametrize("seed,T,K,N,R,L", [
    (41, 4096, 512, [64] * 8, 64, 7),        # most tokens, 8 slices, rank 64
    (42, 64, 8192, [520, 1024], 64, 3),      # 16 K chunks, ragged 512-column chunk
    (43, 300, 576, [8, 16, 24], 48, 2),      # K not a multiple of 512, 3 rank blocks
    (44, 200, 2048, [264, 128], 128, 5),     # rank 128 (two rank passes), ragged column chunk
    (45, 150, 512, [80], 80, 3),             # rank 80: second pass of 16 ranks
    (46, 1500, 1024, [512, 264], 128, 100),  # 100 slots, 1500 tokens: groups from the segment table
    (47, 1100, 512, [128], 32, 8),           # past 1024 tokens with few slots: segment table
    (48, 700, 4096, [264], 96, 80),          # rank 96, 80 slots: K-split row shrink (8 splits)
])
def test_grouped_limits_bit_exact(oracle_mod, seed, T, K, N, R, L):
    c = synth.make_integer_linear(T, K, N, R, L, seed=seed, dtype="bf16")
    assert groupable(c)
    log(f"case grouped limits T={T} K={K} N={N} R={R} L={L}")
    d = LinearOnDevice(c)
    d.apply(GRP)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    assert np.array_equal(y, ref), f"max diff {np.max(np.abs(y - ref))}"
    assert canaries_intact(d.yfull)


def shared_a_case(c):
    """The same case with slice 0's lora_a used by every slice."""
    return dataclasses.replace(c, A=[c.A[0]] * len(c.A))


def on_device_shared_a(c):
    d = LinearOnDevice(c)
    d.A = [d.A[0]] * len(d.A)       # one tensor, so one pointer for every slice
    return d


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, PRE, FUS, GRP, RLY, TOK])
@pytest.mark.parametrize("seed,T,K,N,R,L", [
    (51, 600, 1024, [256, 64, 64], 16, 3),     # long runs per slot: auto takes the tile kernels
    (52, 300, 2048, [512, 512], 64, 100),      # 100 slots: auto takes the tile kernels, K split
    (53, 200, 1024, [256, 128, 128], 32, 5),   # auto takes the single-launch kernel
])
def test_shared_lora_a_bit_exact(oracle_mod, path, seed, T, K, N, R, L):
    """One lora_a pointer for every slice ([vLLM] MergedQKVParallelLinearWithLoRA
    duplicates a single checkpoint lora_a per slice): the tile path computes
    its shrink once; every path stays bit-exact on integer vectors."""
    c = shared_a_case(synth.make_integer_linear(T, K, N, R, L, seed=seed, dtype="bf16"))
    skip_unless_path_takes(path, c)
    log(f"case shared lora_a path={path} T={T} N={N} R={R} L={L}")
    d = on_device_shared_a(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    assert np.array_equal(y, ref), f"max diff {np.max(np.abs(y - ref))}"
    assert canaries_intact(d.yfull)


def test_shared_lora_a_prefill_shape(oracle_mod):
    """gate_up-like prefill (2048 tokens, 4 slots, two 2048-column slices,
    rank 64) with one shared lora_a, on the auto (tile) path."""
    rng = np.random.default_rng(61)
    idx = np.repeat(rng.integers(0, 4, 8), 256).astype(np.int32)
    c = shared_a_case(synth.make_linear("shared_a", 2048, 1024, [2048, 2048], 64, 4, idx,
                                        [64, 32, 64, 16], [1.0] * 4, "bf16", seed=62))
    d = on_device_shared_a(c)
    d.apply(aa.LORA_PATH_AUTO)
    y = d.y_host()
    err, rel = bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
    log(f"  max abs err {err:.3e} rel {rel:.3e}")
    assert canaries_intact(d.yfull)


# [SGL] the DeepSeek MLA fused_qkv_a_proj_with_mqa module: one lora_a, and the
# output split at q_lora_rank into two lora_b partitions (q_a: 1536 columns;
# kv_a with the rope part: 512 + 64), hidden 7168.
MLA_K, MLA_N = 7168, [1536, 576]


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, PRE, FUS, GRP, RLY, TOK])
@pytest.mark.parametrize("seed,T,R,L", [
    (55, 48, 16, 4),       # decode batch: auto takes the single-launch kernel
    (56, 900, 64, 6),      # long runs per slot: auto takes the tile kernels, one shrink
])
def test_mla_two_partition_lora_b_bit_exact(oracle_mod, path, seed, T, R, L):
    """Two output partitions behind one lora_a are two slices with equal
    lora_a pointers: bit-exact on integer vectors on every path."""
    c = shared_a_case(synth.make_integer_linear(T, MLA_K, MLA_N, R, L, seed=seed, dtype="bf16"))
    skip_unless_path_takes(path, c)
    log(f"case mla two partitions path={path} T={T} R={R} L={L}")
    d = on_device_shared_a(c)
    d.apply(path)
    y = d.y_host()
    ref = oracle_y(oracle_mod, c)
    assert np.array_equal(y, ref), f"max diff {np.max(np.abs(y - ref))}"
    assert canaries_intact(d.yfull)


def test_mla_two_partition_lora_b_tolerance(oracle_mod):
    """The MLA shape at a decode batch on gaussian inputs (rank 16, 8 slots,
    10 % of tokens without an adapter), auto path."""
    rng = np.random.default_rng(57)
    idx = rng.integers(0, 8, size=256).astype(np.int32)
    idx[rng.random(256) < 0.1] = -1
    c = shared_a_case(synth.make_linear("mla_qkv_a", 256, MLA_K, MLA_N, 16, 8, idx, [16] * 8,
                                        [2.0] * 8, "bf16", seed=58))
    d = on_device_shared_a(c)
    d.apply(aa.LORA_PATH_AUTO)
    y = d.y_host()
    err, rel = bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
    log(f"  max abs err {err:.3e} rel {rel:.3e}")
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("N", [[64, 128, 8, 256, 32, 1024, 16, 512],          # rows of 8
                               [12, 36, 4, 1028, 64, 20, 8, 300]])             # ragged widths
def test_max_slices_bit_exact(oracle_mod, N):
    """LORA_MAX_SLICES (8) slices of different widths, integer vectors, on auto
    and every path lora_plan_packed accepts for the shape, bit for bit."""
    c = synth.make_integer_linear(300, 1024, N, 16, 5, seed=71, dtype="bf16")
    ref = oracle_y(oracle_mod, c)
    ran = []
    for path in (aa.LORA_PATH_AUTO, DEC, PRE, FUS, GRP, RLY, TOK):
        d = LinearOnDevice(c)
        try:
            taken = aa.lora_plan_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
        except aa.LoraError as e:
            assert path != aa.LORA_PATH_AUTO and e.code == aa.LORA_E_PATH, str(e)
            continue
        log(f"case max slices N={N} path={aa.PATH_NAMES[taken]}")
        d.apply(path)
        y = d.y_host()
        assert np.array_equal(y, ref), f"path {aa.PATH_NAMES[taken]}: {np.max(np.abs(y - ref))}"
        assert canaries_intact(d.yfull)
        ran.append(aa.PATH_NAMES[taken])
    assert len(ran) >= 3, ran


@pytest.mark.parametrize("seed,T,K,N,R,L,shared,auto_path", [
    # two chunks per expand item: 36 expected groups x 28 items x 2 token blocks
    (81, 1024, 1024, [14336, 14336], 16, 8, False, RLY),
    (81, 1024, 1024, [14336, 14336], 16, 8, True, RLY),
    # four chunks per item over three slices of 79, 48 and 17 chunks: each
    # slice's last item is short, the last chunk of the third holds 8 columns
    (82, 512, 1024, [40000, 24576, 8200], 16, 8, False, RLY),
    (82, 512, 1024, [40000, 24576, 8200], 16, 8, True, RLY),
    (83, 512, 1024, [40000, 24576, 8200], 32, 8, False, RLY),
    (83, 512, 1024, [40000, 24576, 8200], 32, 8, True, RLY),
    # vocabularies: rank 32 at 64 tokens, and K = 8192 (32 K chunks)
    (84, 64, 1024, [128256], 32, 8, False, RLY),
    (85, 256, 8192, [128256], 16, 8, False, RLY),
    # a few tokens (two chunks per item): a vocabulary at 4 tokens (auto:
    # TOKEN, whose 2004 work-groups re-read 66 MB of lora_a), two wide slices
    # at 12 tokens and rank 32
    (86, 4, 1024, [128256], 16, 8, False, TOK),
    (87, 12, 1024, [40000, 24576], 32, 8, False, RLY),
])
def test_relay_wide_items_bit_exact(oracle_mod, seed, T, K, N, R, L, shared, auto_path):
    """Wide outputs on the K-split single launch, whose expand work-groups walk
    up to four consecutive column chunks of one slice: integer vectors bit
    for bit on RELAY and on auto (which takes it, or TOKEN for a few tokens),
    with one lora_a for every slice too (every item of every slice then
    reads slice 0's partials); the workspace is all zero after each call."""
    c = synth.make_integer_linear(T, K, N, R, L, seed=seed, dtype="bf16")
    if shared:
        c = shared_a_case(c)
    ref = oracle_y(oracle_mod, c)
    for path in (aa.LORA_PATH_AUTO, RLY):
        d = on_device_shared_a(c) if shared else LinearOnDevice(c)
        taken = aa.lora_plan_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
        log(f"case relay wide T={T} K={K} N={N} R={R} shared={shared} path={aa.PATH_NAMES[path]}")
        assert taken == (auto_path if path == aa.LORA_PATH_AUTO else RLY), aa.PATH_NAMES[taken]
        d.apply(path)
        y = d.y_host()
        assert np.array_equal(y, ref), f"max diff {np.max(np.abs(y - ref))}"
        assert canaries_intact(d.yfull)
        assert int(torch.count_nonzero(d.ws)) == 0


def test_relay_largest_shape_bit_exact(oracle_mod):
    """The largest call the K-split single launch takes: 1024 tokens, K = 8192
    (32 K chunks), rank 32, and a 257024-column vocabulary (the widest the
    logits layer lists), 8 slots; integer vectors on RELAY and on auto (which
    takes it), every output bit for bit, the workspace zero afterwards."""
    T, K, N, R, L = 1024, 8192, [257024], 32, 8
    c = synth.make_integer_linear(T, K, N, R, L, seed=91, dtype="bf16")
    ref = oracle_par.lora_apply(oracle_mod, c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    exact = bounds.linear_exact_int_by_slot(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(ref, exact.astype(np.float32))
    del exact
    for path in (aa.LORA_PATH_AUTO, RLY):
        d = LinearOnDevice(c)
        taken = aa.lora_plan_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
        log(f"case relay largest shape path={aa.PATH_NAMES[path]}")
        assert taken == RLY, aa.PATH_NAMES[taken]
        d.apply(path)
        y = d.y_host()
        assert canaries_intact(d.yfull)
        bad = np.argwhere(y != ref)
        assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:4].tolist()}"
        assert int(torch.count_nonzero(d.ws)) == 0
        del d, y


def test_zero_tokens_noop():
    c = synth.config_decode(T=8)
    d = LinearOnDevice(c)
    x0 = d.x[:0]
    y0 = d.y[:0]
    aa.lora_apply_packed(y0, x0, d.A, d.B, d.idx[:0], d.rank, d.scale, d.ws)
    torch.cuda.synchronize()
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("T,L,R,N", [(256, 8, 16, [1024, 256, 264]), (700, 4, 32, [1024, 256, 264]),
                                     (33, 64, 16, [1024, 256, 264]), (1024, 64, 32, [1024, 256, 264]),
                                     (256, 8, 16, [20480]), (200, 5, 32, [16384, 8])])
def test_relay_repeated_calls_leave_counters_zero(oracle_mod, T, L, R, N):
    """Calls in a row on one workspace: each equals the first bit for bit and
    within tolerance of the oracle, and the workspace (partial sums, reader
    counters, the error word of the bounded waits) is all zero again after
    every call."""
    rng = np.random.default_rng(T + L)
    idx = rng.integers(-1, L, T).astype(np.int32)
    c = synth.make_linear("relay", T, 2048, N, R, L, idx,
                          rng.choice([R, R // 2, 8], L).astype(np.int32), [2.0] * L, "bf16",
                          seed=T)
    d = LinearOnDevice(c, guard=False)
    assert d.ws.numel() == aa.lora_workspace_size(T, c.K, c.S, c.R, c.L)
    first = None
    for call in range(3):
        log(f"case relay repeat T={T} L={L} R={R} N={N} call={call}")
        d.reset_y()
        d.apply(RLY)
        y = d.y_host()
        nz = int(torch.count_nonzero(d.ws))
        assert nz == 0, f"{nz} workspace bytes left non-zero"
        if first is None:
            first = y
            bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
            assert_passthrough(c, y)
        else:
            assert np.array_equal(y.view(np.uint32), first.view(np.uint32))


def test_relay_after_other_paths_on_one_workspace(oracle_mod):
    """One workspace, sized for the largest call, serves calls of other paths
    and shapes that leave split-K partial sums in it; the single-launch K-split
    kernel keeps its zero-on-entry region at the end of the buffer, clear of
    every other call's regions, so its results stay exact to tolerance."""
    rng = np.random.default_rng(77)
    big = synth.make_linear("big", 1500, 4096, [1024, 264, 256], 16, 100,
                            rng.integers(-1, 100, 1500).astype(np.int32),
                            rng.choice([16, 8], 100).astype(np.int32), [1.0] * 100, "bf16", seed=78)
    ws = aa.alloc_workspace(big.T, big.K, big.S, big.R, big.L)
    cases = [synth.config_decode(T=256), synth.config_decode(T=64)]
    for i, c in enumerate(cases):
        cases[i] = synth.make_linear(f"small{i}", c.T, 4096, big.N, 16, 8, c.idx, c.slot_rank,
                                     c.scale, "bf16", seed=80 + i)
    db = LinearOnDevice(big, guard=False)
    ds = [LinearOnDevice(c, guard=False) for c in cases]
    for rnd in range(2):
        for path in (PRE, DEC):
            log(f"case shared ws round={rnd} big path={path}")
            db.reset_y()
            aa.lora_apply_packed(db.y, db.x, db.A, db.B, db.idx, db.rank, db.scale, ws, path=path)
            torch.cuda.synchronize()
        for c, d in zip(cases, ds):
            aa.lora_apply_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, ws, path=DEC)
            d.reset_y()
            log(f"case shared ws round={rnd} relay T={c.T}")
            aa.lora_apply_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, ws, path=RLY)
            y = d.y_host()
            bounds.check_bf16_tolerance(y, oracle_y(oracle_mod, c))
            assert_passthrough(c, y)


def test_relay_back_to_back_calls_bit_identical(oracle_mod):
    """300 single-launch K-split calls back to back on one workspace, rotating
    over three slot assignments (so a partial sum left over from the previous
    call would be wrong data for the next): every call's output equals the
    first call of its assignment bit for bit, and that one the oracle."""
    c = synth.config_decode()
    rng = np.random.default_rng(21)
    idxs = [c.idx, rng.permutation(c.idx).astype(np.int32),
            np.where(rng.random(c.T) < 0.3, -1, rng.integers(0, c.L, c.T)).astype(np.int32)]
    d = LinearOnDevice(c, guard=False)
    idx_d = [dev(i) for i in idxs]
    y0 = d.y.clone()
    snaps = []
    for call in range(300):
        v = call % 3
        d.y.copy_(y0)
        aa.lora_apply_packed(d.y, d.x, d.A, d.B, idx_d[v], d.rank, d.scale, d.ws, path=RLY)
        snaps.append(d.y.clone())
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(d.ws)) == 0
    for v in range(3):
        first = host_f32(snaps[v])
        ref, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, idxs[v], c.slot_rank, c.scale)
        bounds.check_bf16_tolerance(first, ref)
        for call in range(v + 3, 300, 3):
            assert torch.equal(snaps[call], snaps[v]), f"call {call} (assignment {v}) differs"


def test_relay_forced_give_up_reported_and_repaired(oracle_mod):
    """The host forces every hand-over wait of a RELAY call to give up after its
    first poll (LORA_FLAG_RELAY_GIVE_UP; every kernel still ends normally):
    lora_workspace_check reports LORA_E_TIMEOUT and zero-fills the workspace,
    after which a normal call on the same workspace equals a call on a fresh
    workspace bit for bit, and the check reports LORA_OK again."""
    c = synth.config_decode()
    d = LinearOnDevice(c, guard=False)
    fresh = LinearOnDevice(c, guard=False)
    fresh.apply(RLY)
    want = fresh.y_host()
    bounds.check_bf16_tolerance(want, oracle_y(oracle_mod, c))
    aa.lora_workspace_check(d.ws)                      # nothing to report yet
    for rnd in range(3):
        log(f"case relay forced give-up round={rnd}")
        d.reset_y()
        d.apply(RLY, flags=aa.LORA_FLAG_RELAY_GIVE_UP)
        with pytest.raises(aa.LoraError) as e:
            aa.lora_workspace_check(d.ws)
        assert e.value.code == aa.LORA_E_TIMEOUT
        assert int(torch.count_nonzero(d.ws)) == 0
        d.reset_y()
        d.apply(RLY)
        got = d.y_host()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        aa.lora_workspace_check(d.ws)
        assert int(torch.count_nonzero(d.ws)) == 0


@pytest.mark.parametrize("path", [RLY, GRP])
def test_shared_lora_a_decode_config_repeated(oracle_mod, path):
    """The decode QKV workload with one lora_a for every slice: the shrink runs
    once (slice 0's) and the expands of all three slices add it.  Three calls in
    a row on one workspace equal each other bit for bit and the oracle within
    tolerance, and the K-split region is all zero after each call (the last of
    the readers over every slice clears the shared partials)."""
    c = shared_a_case(synth.config_decode())
    d = on_device_shared_a(c)
    ref = oracle_y(oracle_mod, c)
    first = None
    for call in range(3):
        log(f"case shared lora_a decode config path={path} call={call}")
        d.reset_y()
        d.apply(path)
        y = d.y_host()
        if path == RLY:
            assert int(torch.count_nonzero(d.ws)) == 0
        if first is None:
            first = y
            err, rel = bounds.check_bf16_tolerance(y, ref)
            log(f"  max abs err {err:.3e} rel {rel:.3e}")
            assert_passthrough(c, y)
        else:
            assert np.array_equal(y.view(np.uint32), first.view(np.uint32))
    assert canaries_intact(d.yfull)


@pytest.mark.parametrize("nbytes", [0, 1, 15, 16, 17, 4096 + 7, (1 << 20) + 3, (70 << 20) + 13])
def test_workspace_init_exact_range(nbytes):
    """lora_workspace_init zero-fills exactly ws_bytes bytes from a 256-byte
    aligned start, whole 16-byte units and a ragged tail alike, and leaves
    the bytes past the end as they were."""
    log(f"case workspace init bytes={nbytes}")
    pad = 4096
    raw = torch.empty(nbytes + pad + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    buf = raw[off:off + nbytes + pad]
    buf.fill_(0xAB)
    rc = aa.lib().lora_workspace_init(aa.C.c_void_p(buf.data_ptr()), nbytes, None)
    torch.cuda.synchronize()
    assert rc == aa.LORA_OK
    assert int(torch.count_nonzero(buf[:nbytes])) == 0
    assert bool(torch.all(buf[nbytes:] == 0xAB))
    if nbytes:
        # a start that is not 256-byte aligned is refused before any launch
        rc = aa.lib().lora_workspace_init(aa.C.c_void_p(buf.data_ptr() + 16), nbytes, None)
        assert rc == aa.LORA_E_ALIGN
        torch.cuda.synchronize()
        assert bool(torch.all(buf[nbytes:] == 0xAB))


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, PRE, FUS, GRP, RLY, TOK])
def test_side_stream_equals_default_stream(oracle_mod, path):
    """A call on a stream of its own (the stream argument, with the default
    stream current) gives the same bits as the call on the default stream:
    every launch of the call, fills included, goes to the stream it is given."""
    c = synth.config_decode()
    d = LinearOnDevice(c, guard=False)
    try:
        aa.lora_plan_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
    except aa.LoraError:
        pytest.skip("the path does not take this shape")
    log(f"case side stream path={path}")
    d.apply(path)
    want = d.y_host()
    bounds.check_bf16_tolerance(want, oracle_y(oracle_mod, c))
    s = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for rnd in range(3):
        d.reset_y()
        s.wait_stream(main)
        aa.lora_apply_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path, stream=s)
        main.wait_stream(s)
        got = d.y_host()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), rnd


def strided_rows(t, lead, tail):
    """The same values as the 2-D tensor t, as a column window of a wider
    tensor (row stride K + lead + tail) whose other columns hold large values
    that would show in y if a kernel read them."""
    T, K = t.shape
    wide = torch.full((T, lead + K + tail), 1024.0, dtype=t.dtype, device=t.device)
    wide[:, lead:lead + K] = t
    return wide[:, lead:lead + K]


@pytest.mark.parametrize("cfg", ["decode", "prefill_small"])
@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, DEC, PRE, FUS, GRP, RLY, TOK])
def test_x_row_stride_wider_than_k(oracle_mod, cfg, path):
    """x given as a window of wider rows (ldx = K + 72, starting 16 columns in)
    gives the same bits as a contiguous x on every path that takes the shape."""
    if cfg == "decode":
        c = synth.config_decode()
    else:
        c = synth.config_prefill(seed=91, n_seq=5, total=700, K=1024, Nslice=512, R=64, L=6)
    d = LinearOnDevice(c, guard=False)
    try:
        aa.lora_plan_packed(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
    except aa.LoraError:
        pytest.skip("the path does not take this shape")
    log(f"case x row stride cfg={cfg} path={path}")
    d.apply(path)
    want = d.y_host()
    bounds.check_bf16_tolerance(want, oracle_y(oracle_mod, c))
    xs = strided_rows(d.x, 16, 56)
    assert xs.stride(0) == c.x.shape[1] + 72
    d.reset_y()
    aa.lora_apply_packed(d.y, xs, d.A, d.B, d.idx, d.rank, d.scale, d.ws, path=path)
    got = d.y_host()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("path", [DEC, PRE, GRP])
def test_shrink_x_row_stride(path):
    """lora_shrink with x as a window of wider rows (ldx = K + 72) writes the
    buffer bits of a contiguous x."""
    c = synth.make_linear("sh_stride", 300, 1024, [256, 128], 32, 5,
                          idx=np.random.default_rng(4).integers(-1, 6, 300),
                          slot_rank=[32, 8, 0, 16, 24], scale=[1, 1, 1, 1, 1], dtype="bf16",
                          seed=32)
    log(f"case shrink x stride path={path}")
    d = LinearOnDevice(c, guard=False)
    want = torch.zeros((c.S, c.T, c.R), dtype=torch.float32, device="cuda")
    got = torch.full_like(want, 123.0)
    aa.lora_shrink(want, d.x, d.A, d.idx, d.rank, d.ws, path=path)
    aa.lora_shrink(got, strided_rows(d.x, 16, 56), d.A, d.idx, d.rank, d.ws, path=path)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
