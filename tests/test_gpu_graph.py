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
                                  aa.LORA_PATH_DECODE, aa.LORA_PATH_RELAY])
def test_graph_replays_read_current_metadata(oracle_mod, path):
    c = synth.config_decode()
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
