"""The Python binding rejects tensors of the wrong dtype, shape or device with
ValueError before it calls into the library (CPU tensors: the dtype and
shape checks run before the device check, and a well-formed call on CPU
tensors is refused for its device); bench.py refuses a multi-GPU run."""
import os
import pytest
import torch

import adapter_apply_amd as aa

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32
T, K, L, R = 12, 64, 3, 16
N = [32, 16]


def linear(**over):
    a = dict(y=torch.zeros(T, sum(N), dtype=BF), x=torch.zeros(T, K, dtype=BF),
             A=[torch.zeros(L, R, K, dtype=BF) for _ in N],
             B=[torch.zeros(L, n, R, dtype=BF) for n in N],
             idx=torch.zeros(T, dtype=I32), rank=torch.full((L,), R, dtype=I32),
             scale=torch.ones(L, dtype=F32), ws=torch.zeros(4096, dtype=torch.uint8))
    a.update(over)
    return a


def apply(a):
    aa.lora_apply_packed(a["y"], a["x"], a["A"], a["B"], a["idx"], a["rank"], a["scale"], a["ws"])


BAD_PACKED = {
    "int64 idx": dict(idx=torch.zeros(T, dtype=torch.int64)),
    "short idx": dict(idx=torch.zeros(T - 1, dtype=I32)),
    "float rank": dict(rank=torch.full((L,), R, dtype=F32)),
    "short rank": dict(rank=torch.full((L - 1,), R, dtype=I32)),
    "bf16 scale": dict(scale=torch.ones(L, dtype=BF)),
    "long scale": dict(scale=torch.ones(L + 1, dtype=F32)),
    "fp32 y, bf16 x": dict(y=torch.zeros(T, sum(N), dtype=F32)),
    "short y": dict(y=torch.zeros(T - 2, sum(N), dtype=BF)),
    "fp16 x": dict(x=torch.zeros(T, K, dtype=torch.float16), y=torch.zeros(T, sum(N), dtype=torch.float16)),
    "A of other L": dict(A=[torch.zeros(L, R, K, dtype=BF), torch.zeros(L + 1, R, K, dtype=BF)]),
    "A of other K": dict(A=[torch.zeros(L, R, K + 8, dtype=BF)] * 2),
    "A fp32": dict(A=[torch.zeros(L, R, K, dtype=F32)] * 2),
    "B of other R": dict(B=[torch.zeros(L, 32, R, dtype=BF), torch.zeros(L, 16, R + 16, dtype=BF)]),
    "B of other L": dict(B=[torch.zeros(L + 2, 32, R, dtype=BF), torch.zeros(L, 16, R, dtype=BF)]),
    "B count": dict(B=[torch.zeros(L, 32, R, dtype=BF)]),
    "empty A": dict(A=[], B=[]),
    "2-D ws": dict(ws=torch.zeros(64, 64, dtype=torch.uint8)),
}


@pytest.mark.parametrize("name", sorted(BAD_PACKED))
def test_packed_rejects(name):
    with pytest.raises(ValueError):
        apply(linear(**BAD_PACKED[name]))


def test_packed_rejects_cpu_tensors():
    with pytest.raises(ValueError, match="GPU"):
        apply(linear())


def test_shrink_and_expand_reject():
    a = linear()
    buf = torch.zeros(len(N), T, R, dtype=F32)
    for bad in (torch.zeros(len(N), T, R, dtype=BF), torch.zeros(len(N), T + 1, R, dtype=F32),
                torch.zeros(len(N) + 1, T, R, dtype=F32)):
        with pytest.raises(ValueError):
            aa.lora_shrink(bad, a["x"], a["A"], a["idx"], a["rank"], a["ws"])
    with pytest.raises(ValueError):
        aa.lora_shrink(buf, a["x"], a["A"], torch.zeros(T, dtype=torch.int64), a["rank"], a["ws"])
    with pytest.raises(ValueError, match="GPU"):
        aa.lora_shrink(buf, a["x"], a["A"], a["idx"], a["rank"], a["ws"])
    for bad in (dict(y=torch.zeros(T + 1, sum(N), dtype=BF)),
                dict(B=[torch.zeros(L, 32, R, dtype=BF)]),
                dict(scale=torch.ones(L, dtype=torch.float64))):
        b = linear(**bad)
        with pytest.raises(ValueError):
            aa.lora_expand(b["y"], buf, b["B"], b["idx"], b["rank"], b["scale"], b["ws"])
    with pytest.raises(ValueError, match="GPU"):
        aa.lora_expand(a["y"], buf, a["B"], a["idx"], a["rank"], a["scale"], a["ws"])


def test_segments_reject():
    ws = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError):
        aa.lora_build_segments(torch.zeros(T, dtype=torch.int64), None, L, R, ws)
    with pytest.raises(ValueError):
        aa.lora_build_segments(torch.zeros(T, dtype=I32), torch.zeros(L + 1, dtype=I32), L, R, ws)


Tm, k, E, I = 6, 2, 4, 24


def moe(**over):
    a = dict(kind=aa.MOE_LORA_W13, y=torch.zeros(Tm * k, 2 * I, dtype=BF),
             x=torch.zeros(Tm, K, dtype=BF), A=[torch.zeros(L, 1, R, K, dtype=BF)] * 2,
             B=[torch.zeros(L, E, I, R, dtype=BF)] * 2, ids=torch.zeros(Tm, k, dtype=I32),
             w=None, idx=torch.zeros(Tm, dtype=I32), rank=torch.full((L,), R, dtype=I32),
             scale=torch.ones(L, dtype=F32), ws=torch.zeros(4096, dtype=torch.uint8),
             reduce_k=False)
    a.update(over)
    return a


def moe_apply(a):
    aa.moe_lora_apply(a["kind"], a["y"], a["x"], a["A"], a["B"], a["ids"], a["w"], a["idx"],
                      a["rank"], a["scale"], E, a["ws"], reduce_k=a["reduce_k"])


BAD_MOE = {
    "int64 topk_ids": dict(ids=torch.zeros(Tm, k, dtype=torch.int64)),
    "y rows per token for w13": dict(y=torch.zeros(Tm, 2 * I, dtype=BF)),
    "x rows per pair for w13": dict(x=torch.zeros(Tm * k, K, dtype=BF)),
    "w2 x rows per token": dict(kind=aa.MOE_LORA_W2, x=torch.zeros(Tm, I, dtype=BF),
                                A=[torch.zeros(L, E, R, I, dtype=BF)],
                                B=[torch.zeros(L, 1, K, R, dtype=BF)],
                                y=torch.zeros(Tm * k, K, dtype=BF)),
    "w2 reduce_k y per pair": dict(kind=aa.MOE_LORA_W2, x=torch.zeros(Tm * k, I, dtype=BF),
                                   A=[torch.zeros(L, E, R, I, dtype=BF)],
                                   B=[torch.zeros(L, 1, K, R, dtype=BF)],
                                   y=torch.zeros(Tm * k, K, dtype=BF), reduce_k=True),
    "topk_w shape": dict(w=torch.ones(Tm, k + 1, dtype=F32)),
    "topk_w bf16": dict(w=torch.ones(Tm, k, dtype=BF)),
    "A of other experts": dict(A=[torch.zeros(L, 1, R, K, dtype=BF), torch.zeros(L, E, R, K, dtype=BF)]),
    "B of other rank": dict(B=[torch.zeros(L, E, I, R, dtype=BF), torch.zeros(L, E, I, 2 * R, dtype=BF)]),
    "short idx": dict(idx=torch.zeros(Tm - 1, dtype=I32)),
    "fp32 y": dict(y=torch.zeros(Tm * k, 2 * I, dtype=F32)),
}


@pytest.mark.parametrize("name", sorted(BAD_MOE))
def test_moe_rejects(name):
    with pytest.raises(ValueError):
        moe_apply(moe(**BAD_MOE[name]))


def test_moe_rejects_cpu_tensors():
    with pytest.raises(ValueError, match="GPU"):
        moe_apply(moe())


def test_moe_align_rejects():
    ws = torch.zeros(4096, dtype=torch.uint8)
    ids = torch.zeros(Tm, k, dtype=I32)
    idx = torch.zeros(Tm, dtype=I32)
    with pytest.raises(ValueError):
        aa.moe_lora_align(ids.long(), idx, None, E, L, R, 16, ws)
    with pytest.raises(ValueError):
        aa.moe_lora_align(ids, idx[:-1], None, E, L, R, 16, ws)
    cap = aa.moe_lora_align_capacity(Tm, k, E, 16)
    with pytest.raises(ValueError):          # outputs of the wrong capacity
        aa.moe_lora_align(ids, idx, None, E, L, R, 16, ws, torch.zeros(L, cap - 16, dtype=I32),
                          torch.zeros(L, cap // 16, dtype=I32), torch.zeros(L, dtype=I32))
    with pytest.raises(ValueError):          # only some outputs
        aa.moe_lora_align(ids, idx, None, E, L, R, 16, ws, torch.zeros(L, cap, dtype=I32))
    with pytest.raises(ValueError, match="GPU"):
        aa.moe_lora_align(ids, idx, None, E, L, R, 16, ws)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU only: --gpus above 1 exits with status 2 and a
    message, before anything touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
