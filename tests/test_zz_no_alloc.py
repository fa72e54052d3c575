"""lora_apply_packed_noalloc (the library's static per-GPU scratch instead of a
workspace) against lora_apply_packed with a workspace, through the C ABI: two
calls in a row, the second with a smaller batch, on the paths a decode batch
takes; every output equal bit for bit (same kernels) and within the bf16
tolerance of the oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import adapter_apply_amd as aa  # noqa: E402
import synth  # noqa: E402
from tests import bounds  # noqa: E402
from tests.gpu_util import LinearOnDevice, canaries_intact, dev, host_f32, log  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aa.lib()


def run_pair(c, path):
    ref = LinearOnDevice(c, guard=False)
    ref.apply(path)
    want = ref.y_host()
    d = LinearOnDevice(c)
    aa.lora_apply_packed_noalloc(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale, path=path)
    got = d.y_host()
    assert canaries_intact(d.yfull)
    return want, got


@pytest.mark.parametrize("path", [aa.LORA_PATH_AUTO, aa.LORA_PATH_RELAY, aa.LORA_PATH_GROUPED,
                                  aa.LORA_PATH_PREFILL, aa.LORA_PATH_DECODE, aa.LORA_PATH_FUSED,
                                  aa.LORA_PATH_TOKEN])
def test_noalloc_equals_workspace_call(oracle_mod, path):
    big = synth.config_decode()                  # 256 tokens, QKV 4096/1024/1024
    small = synth.config_decode(seed=77, T=40)   # then a smaller batch on the same array
    for c in (big, small):
        log(f"case noalloc path={path} T={c.T}")
        want, got = run_pair(c, path)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        ref, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
        bounds.check_bf16_tolerance(got, ref)
    aa.lora_static_scratch_check()


def test_noalloc_integer_vectors_and_size_limit(oracle_mod):
    """Integer vectors (bit-exact against the oracle), two shapes in a row;
    a batch past the array's size is refused with LORA_E_SCRATCH."""
    for seed, T, K, N, R, L in ((91, 300, 2048, [512, 128, 128], 32, 6),
                                (92, 70, 1024, [256, 64], 16, 3)):
        c = synth.make_integer_linear(T, K, N, R, L, seed=seed)
        log(f"case noalloc integer T={T} K={K} R={R}")
        d = LinearOnDevice(c)
        aa.lora_apply_packed_noalloc(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale)
        y = d.y_host()
        ref, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
        assert np.array_equal(y, ref)
        assert canaries_intact(d.yfull)
    # 4096 tokens at rank 128: 16.8 MB of split-K partials, past half the array
    c = synth.make_linear("big", 4096, 2048, [1024], 128, 8,
                          np.zeros(4096, np.int32), [128] * 8, [1.0] * 8, "bf16", seed=93)
    d = LinearOnDevice(c, guard=False)
    with pytest.raises(aa.LoraError) as e:
        aa.lora_apply_packed_noalloc(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale)
    assert e.value.code == aa.LORA_E_SCRATCH
    torch.cuda.synchronize()
    aa.lora_static_scratch_check()


def test_noalloc_relay_give_up_reported():
    """A forced give-up of the RELAY waits in the static array is reported by
    lora_workspace_check(NULL) and repaired; the next call is exact again."""
    c = synth.config_decode(T=128)
    ref = LinearOnDevice(c, guard=False)
    ref.apply(aa.LORA_PATH_RELAY)
    want = ref.y_host()
    d = LinearOnDevice(c, guard=False)
    aa.lora_apply_packed_noalloc(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale,
                                 path=aa.LORA_PATH_RELAY, flags=aa.LORA_FLAG_RELAY_GIVE_UP)
    with pytest.raises(aa.LoraError) as e:
        aa.lora_static_scratch_check()
    assert e.value.code == aa.LORA_E_TIMEOUT
    d.reset_y()
    aa.lora_apply_packed_noalloc(d.y, d.x, d.A, d.B, d.idx, d.rank, d.scale,
                                 path=aa.LORA_PATH_RELAY)
    got = d.y_host()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    aa.lora_static_scratch_check()
