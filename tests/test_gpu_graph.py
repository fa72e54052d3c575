"""One HIP graph of lora_apply_packed, captured once for a fixed token count
and replayed with the batch metadata (slot per token, slot ranks) rewritten in
place between replays, as a serving loop does with a graph captured per batch
size ([SGL] the two-phase graph set-up and the in-place prepare_lora_batch).
Every replay must read the metadata current at replay time: it equals the
eager call on the same metadata bit for bit, and the oracle within the bf16
tolerance.  The library allocates nothing and records no memset, so the calls
can be captured as they are."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import adapter_apply_amd as aa  # noqa: E402
import synth  # noqa: E402
from tests import bounds  # noqa: E402
from tests.gpu_util import LinearOnDevice, dev, host_f32, log  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aa.lib()


def metadata_sets(c):
    """The captured batch's own metadata, then other slot assignments and
    ranks for the same token count."""
    rng = np.random.default_rng(5)
    yield "captured", c.idx, c.slot_rank
    yield "permuted slots", rng.permutation(c.idx).astype(np.int32), c.slot_rank
    rank = c.slot_rank.copy()
    rank[::2] = 0                                   # even slots switched off: passthrough
    yield "half the slots off", c.idx, rank
    yield "no adapter", np.full(c.T, -1, np.int32), c.slot_rank
    idx = rng.integers(0, c.L, size=c.T).astype(np.int32)
    yield "every token on a slot", idx, c.slot_rank


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, aa.LORA_PATH_GROUPED, aa.LORA_PATH_PREFILL,
                                  aa.LORA_PATH_DECODE, aa.LORA_PATH_RELAY, aa.LORA_PATH_TOKEN])
def test_graph_replays_read_current_metadata(oracle_mod, path):
    replay_check(oracle_mod, synth.config_decode(), path)


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, aa.LORA_PATH_RELAY, aa.LORA_PATH_PREFILL])
def test_graph_replays_wide_output(oracle_mod, path):
    """The lm_head shape (256 tokens, a 128256-column vocabulary): auto and
    RELAY take the K-split single launch with expand items of four column
    chunks, PREFILL the tile kernels."""
    replay_check(oracle_mod, synth.config_logits(), path)


def replay_check(oracle_mod, c, path):
    d = LinearOnDevice(c, guard=False)
    y0 = d.y.clone()
    # warm-up on a side stream, then capture one call
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.apply(path)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.apply(path)
    torch.cuda.synchronize()
    for name, idx, rank in metadata_sets(c):
        log(f"case graph path={path} metadata={name}")
        d.idx.copy_(dev(idx))
        d.rank.copy_(dev(rank))
        d.y.copy_(y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host_f32(d.y)
        d.y.copy_(y0)
        d.apply(path)
        torch.cuda.synchronize()
        eager = host_f32(d.y)
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), name
        ref, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, idx, rank, c.scale)
        bounds.check_bf16_tolerance(got, ref)
        off = [t for t in range(c.T) if idx[t] < 0 or rank[idx[t]] <= 0]
        assert np.array_equal(got[off].view(np.uint32), c.y0[off].view(np.uint32)), name
    del g


def moe_metadata_sets(c):
    """The captured batch's routing and slots, then other routings, slot
    assignments and ranks for the same token count."""
    rng = np.random.default_rng(15)
    yield "captured", c.topk_ids, c.idx, c.slot_rank
    ids = np.stack([rng.permutation(c.E)[:c.k] for _ in range(c.T)]).astype(np.int32)
    yield "rerouted", ids, c.idx, c.slot_rank
    yield "slots permuted", c.topk_ids, rng.permutation(c.idx).astype(np.int32), c.slot_rank
    rank = c.slot_rank.copy()
    rank[1::2] = 0
    yield "half the slots off", c.topk_ids, c.idx, rank
    ids = c.topk_ids.copy()
    ids[::3, 0] = -1                                  # pairs routed nowhere carry no delta
    ids[1::5, 1] = c.E
    yield "some pairs without an expert", ids, c.idx, c.slot_rank
    yield "no adapter", c.topk_ids, np.full(c.T, -1, np.int32), c.slot_rank


@pytest.mark.parametrize("T", [256, 16])
def test_moe_graph_replays_read_current_routing(oracle_mod, T):
    """Fused-MoE LoRA in one captured graph: alignment, w13 and w2 (T = 256:
    2048 pairs, the aligned path) or w13 and w2 without the alignment (T = 16:
    128 pairs).  Replayed with topk_ids, idx and slot_rank rewritten in place;
    each replay equals the eager calls on the same metadata bit for bit and the
    oracle within the bf16 tolerance, and rows without an adapter stay
    bit-exact."""
    c = synth.make_moe("moe_graph", T, 8, 64, 1024, 512, 16, 8, "bf16", 31)
    bf = torch.bfloat16
    x, h = dev(c.x, bf), dev(c.h, bf)
    A13, B13 = [dev(a, bf) for a in c.A13], [dev(b, bf) for b in c.B13]
    A2, B2 = [dev(c.A2, bf)], [dev(c.B2, bf)]
    g0, o0 = dev(c.gate_up0, bf), dev(c.out0, bf)
    g, o = g0.clone(), o0.clone()
    ids, idx, rank = dev(c.topk_ids), dev(c.idx), dev(c.slot_rank)
    w, scale = dev(c.topk_w), dev(c.scale)
    ws = aa.alloc_moe_workspace(T, c.k, 2, c.R, c.L, c.E)
    aligned = T * c.k > 256
    ready = aa.LORA_FLAG_SEGMENTS_READY if aligned else 0

    def step():
        if aligned:
            aa.moe_lora_align(ids, idx, rank, c.E, c.L, c.R, 16, ws)
        aa.moe_lora_apply(aa.MOE_LORA_W13, g, x, A13, B13, ids, None, idx, rank, scale, c.E, ws,
                          flags=ready)
        aa.moe_lora_apply(aa.MOE_LORA_W2, o, h, A2, B2, ids, w, idx, rank, scale, c.E, ws,
                          flags=ready)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for name, ids_h, idx_h, rank_h in moe_metadata_sets(c):
        log(f"case moe graph T={T} metadata={name}")
        ids.copy_(dev(ids_h))
        idx.copy_(dev(idx_h))
        rank.copy_(dev(rank_h))
        g.copy_(g0)
        o.copy_(o0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_g, got_o = host_f32(g), host_f32(o)
        g.copy_(g0)
        o.copy_(o0)
        step()
        torch.cuda.synchronize()
        assert np.array_equal(got_g.view(np.uint32), host_f32(g).view(np.uint32)), name
        assert np.array_equal(got_o.view(np.uint32), host_f32(o).view(np.uint32)), name
        ref_g = oracle_mod.moe_lora_apply(0, c.gate_up0, c.x, c.A13, c.B13, ids_h, None, idx_h,
                                          rank_h, c.scale, c.E)
        ref_o = oracle_mod.moe_lora_apply(1, c.out0, c.h, [c.A2], [c.B2], ids_h, c.topk_w, idx_h,
                                          rank_h, c.scale, c.E)
        bounds.check_bf16_tolerance(got_g, ref_g)
        bounds.check_bf16_tolerance(got_o, ref_o)
        t_of = np.arange(T * c.k) // c.k
        ids_f = ids_h.reshape(-1)
        dead = ((idx_h[t_of] < 0) | (rank_h[np.maximum(idx_h[t_of], 0)] <= 0) |
                (ids_f < 0) | (ids_f >= c.E))
        assert np.array_equal(got_g[dead].view(np.uint32), c.gate_up0[dead].view(np.uint32)), name
        assert np.array_equal(got_o[dead].view(np.uint32), c.out0[dead].view(np.uint32)), name
    del graph
