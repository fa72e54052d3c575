"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
launching anything (the pointers passed here are never dereferenced)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import adapter_apply_amd as aa

# The pointers below are fake: never let a validation bug turn one of these
# calls into a launch on a real device.
try:
    import torch
    _HAS_GPU = torch.cuda.device_count() > 0
except Exception:  # pragma: no cover
    _HAS_GPU = False
pytestmark = pytest.mark.skipif(_HAS_GPU, reason="fake-pointer ABI checks run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adapter_apply.h")

FAKE = 0x7f0000001000            # 4 KiB aligned, never dereferenced
FAKE_WS = 0x7f0000100000


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:lora|moe_lora)_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = aa.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
        assert n in aa.SIGNATURES, f"binding lacks a signature for {n}"


def test_status_strings():
    for code in range(0, 12):
        assert aa.status_string(code)
    assert aa.status_string(99) == "unknown status"


def _ptrs(n, base=FAKE):
    arr = (C.c_void_p * n)()
    for i in range(n):
        arr[i] = base + 0x100000 * i
    return arr


def _apply(**kw):
    a = dict(y=FAKE, ldy=6144, off=0, x=FAKE, ldx=4096, T=256, K=4096, A=_ptrs(3), B=_ptrs(3),
             N=(C.c_int64 * 3)(4096, 1024, 1024), S=3, L=8, R=16, idx=FAKE, rank=FAKE,
             scale=FAKE, dt=aa.LORA_DT_BF16, path=0, flags=0, ws=FAKE_WS, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return aa.lib().lora_apply_packed(a["y"], a["ldy"], a["off"], a["x"], a["ldx"], a["T"], a["K"],
                                      a["A"], a["B"], a["N"], a["S"], a["L"], a["R"], a["idx"],
                                      a["rank"], a["scale"], a["dt"], a["path"], a["flags"],
                                      a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), aa.LORA_E_SHAPE),
    (dict(L=0), aa.LORA_E_SHAPE),
    (dict(L=1025), aa.LORA_E_SHAPE),
    (dict(R=0), aa.LORA_E_RANK),
    (dict(R=520), aa.LORA_E_RANK),
    (dict(R=12), aa.LORA_E_ALIGN),             # bf16 needs R % 8 == 0
    (dict(S=0), aa.LORA_E_SLICES),
    (dict(S=9), aa.LORA_E_SLICES),
    (dict(dt=7), aa.LORA_E_DTYPE),
    (dict(K=0), aa.LORA_E_SHAPE),
    (dict(K=4100, ldx=4104), aa.LORA_E_ALIGN),
    (dict(ldx=4000), aa.LORA_E_SHAPE),
    (dict(ldx=4100), aa.LORA_E_ALIGN),
    (dict(ldy=6000), aa.LORA_E_SHAPE),
    (dict(off=4, ldy=6144), aa.LORA_E_SHAPE),
    (dict(off=2, ldy=6152), aa.LORA_E_ALIGN),
    (dict(N=(C.c_int64 * 3)(4096, 1022, 1026)), aa.LORA_E_ALIGN),
    (dict(N=(C.c_int64 * 3)(4096, 0, 1024)), aa.LORA_E_SHAPE),
    (dict(N=None), aa.LORA_E_NULL),
    (dict(y=None), aa.LORA_E_NULL),
    (dict(x=None), aa.LORA_E_NULL),
    (dict(idx=None), aa.LORA_E_NULL),
    (dict(scale=None), aa.LORA_E_NULL),
    (dict(A=None), aa.LORA_E_NULL),
    (dict(B=None), aa.LORA_E_NULL),
    (dict(x=FAKE + 8), aa.LORA_E_ALIGN),
    (dict(y=FAKE + 4), aa.LORA_E_ALIGN),
    (dict(A=_ptrs(3, FAKE + 2)), aa.LORA_E_ALIGN),
    # the split decode path needs the workspace (the fused one does not)
    (dict(ws=None, path=aa.LORA_PATH_DECODE), aa.LORA_E_NULL),
    (dict(ws=FAKE_WS + 64, path=aa.LORA_PATH_DECODE), aa.LORA_E_ALIGN),
    (dict(wsb=1024, path=aa.LORA_PATH_DECODE), aa.LORA_E_WORKSPACE),
    (dict(path=aa.LORA_PATH_FUSED, R=128), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_FUSED, T=2048), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_FUSED, dt=aa.LORA_DT_F32), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_PREFILL, dt=aa.LORA_DT_F32), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_PREFILL, R=24), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_GROUPED, R=144), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_GROUPED, T=5000), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_GROUPED, K=8256, ldx=8256), aa.LORA_E_PATH),   # 17 K chunks
    (dict(path=aa.LORA_PATH_GROUPED, K=4104, ldx=4104), aa.LORA_E_PATH),   # K % 64
    (dict(path=aa.LORA_PATH_GROUPED, ldy=6148), aa.LORA_E_PATH),           # ldy % 8
    (dict(path=aa.LORA_PATH_GROUPED, dt=aa.LORA_DT_F32), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_GROUPED, ws=None), aa.LORA_E_NULL),
    (dict(path=aa.LORA_PATH_GROUPED, wsb=1024), aa.LORA_E_WORKSPACE),
    (dict(path=aa.LORA_PATH_FUSED, ldy=6148), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, R=64), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, R=24), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, T=1025), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, L=65), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, K=4104, ldx=4104), aa.LORA_E_PATH),     # K % 256
    (dict(path=aa.LORA_PATH_RELAY, K=8448, ldx=8448), aa.LORA_E_PATH),     # 33 K chunks
    (dict(path=aa.LORA_PATH_RELAY, ldy=6148), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, dt=aa.LORA_DT_F32), aa.LORA_E_PATH),
    (dict(path=aa.LORA_PATH_RELAY, ws=None), aa.LORA_E_NULL),
    (dict(path=aa.LORA_PATH_RELAY, wsb=1024), aa.LORA_E_WORKSPACE),
    # TOKEN takes every shape whose grid one launch holds
    (dict(path=aa.LORA_PATH_TOKEN, S=1, N=(C.c_int64 * 1)(1 << 40), ldy=1 << 40), aa.LORA_E_PATH),
    (dict(path=7), aa.LORA_E_PATH),
    (dict(path=99), aa.LORA_E_PATH),
])
def test_apply_rejects_bad_arguments(kw, code):
    assert _apply(**kw) == code


def test_zero_tokens_is_a_noop_without_launch():
    # T == 0: validation passes and nothing is launched (no GPU here).
    assert _apply(T=0, x=None, y=None, idx=None) == aa.LORA_OK


def test_shrink_expand_validation():
    lib = aa.lib()
    A = _ptrs(2)
    ok_ws = 1 << 40
    assert lib.lora_shrink(None, FAKE, 64, 16, 64, A, 2, 3, 8, FAKE, None, 0, 0, 0, FAKE_WS,
                           ok_ws, None) == aa.LORA_E_NULL
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 8, FAKE, None, 0, 0, 0, FAKE_WS,
                           16, None) == aa.LORA_E_WORKSPACE
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 8, FAKE, None, 1,
                           aa.LORA_PATH_PREFILL, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    # the fused kernel has no separate shrink; the grouped one takes rank <= 64
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 16, FAKE, None, 1,
                           aa.LORA_PATH_FUSED, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 16, FAKE, None, 1,
                           aa.LORA_PATH_RELAY, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 16, FAKE, None, 1,
                           aa.LORA_PATH_TOKEN, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 144, FAKE, None, 1,
                           aa.LORA_PATH_GROUPED, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    # the partial-sum hand-off stops at rank 64 on the grouped path
    assert lib.lora_shrink(FAKE, FAKE, 64, 16, 64, A, 2, 3, 128, FAKE, None, 1,
                           aa.LORA_PATH_GROUPED, aa.LORA_FLAG_PARTIAL, FAKE_WS, ok_ws,
                           None) == aa.LORA_E_PATH
    assert lib.lora_shrink(FAKE, FAKE, 72, 16, 72, A, 2, 3, 16, FAKE, None, 1,
                           aa.LORA_PATH_GROUPED, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    Ng = (C.c_int64 * 2)(64, 68)
    assert lib.lora_expand(FAKE, 136, 0, FAKE, 16, A, Ng, 2, 3, 16, FAKE, None, FAKE, 1,
                           aa.LORA_PATH_GROUPED, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    N = (C.c_int64 * 2)(64, 64)
    assert lib.lora_expand(FAKE, 128, 0, FAKE, 16, A, N, 2, 3, 16, FAKE, None, FAKE, 1,
                           aa.LORA_PATH_TOKEN, 0, FAKE_WS, ok_ws, None) == aa.LORA_E_PATH
    assert lib.lora_expand(FAKE, 128, 0, None, 16, A, N, 2, 3, 8, FAKE, None, FAKE, 0, 0, 0,
                           FAKE_WS, ok_ws, None) == aa.LORA_E_NULL
    assert lib.lora_expand(FAKE, 100, 0, FAKE, 16, A, N, 2, 3, 8, FAKE, None, FAKE, 0, 0, 0,
                           FAKE_WS, ok_ws, None) == aa.LORA_E_SHAPE
    assert lib.lora_build_segments(FAKE, None, -3, 4, 8, FAKE_WS, ok_ws, None) == aa.LORA_E_SHAPE
    assert lib.lora_build_segments(None, None, 5, 4, 8, FAKE_WS, ok_ws, None) == aa.LORA_E_NULL
    assert lib.lora_build_segments(FAKE, None, 5, 4, 8, FAKE_WS, 8, None) == aa.LORA_E_WORKSPACE


def test_workspace_size_and_layout():
    a = aa.lora_workspace_size(256, 4096, 3, 16, 8)
    b = aa.lora_workspace_size(512, 4096, 3, 16, 8)
    c = aa.lora_workspace_size(256, 8192, 3, 16, 8)
    assert 0 < a < b and a < c and a % 256 == 0
    lay = aa.lora_segment_layout(256, 8)
    offs = [lay["header"], lay["slot_start"], lay["perm"], lay["tiles_decode"], lay["tiles_prefill"]]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay["perm"] - lay["slot_start"] >= 4 * 9
    assert lay["tile_decode_tokens"] == 32 and lay["tile_prefill_tokens"] == 64
    with pytest.raises(aa.LoraError):
        aa.lora_workspace_size(256, 4096, 9, 16, 8)


def _moe(**kw):
    a = dict(kind=aa.MOE_LORA_W13, y=FAKE, ldy=3072, rk=0, x=FAKE, ldx=4096, T=2048, k=8, K=4096,
             A=_ptrs(2), Ea=1, B=_ptrs(2), Eb=64, N=(C.c_int64 * 2)(1536, 1536), S=2, E=64, L=8,
             R=16, ids=FAKE, w=None, idx=FAKE, rank=FAKE, scale=FAKE, dt=aa.LORA_DT_BF16, flags=0,
             ws=FAKE_WS, wsb=1 << 40, stream=None)
    a.update(kw)
    return aa.lib().moe_lora_apply(a["kind"], a["y"], a["ldy"], a["rk"], a["x"], a["ldx"], a["T"],
                                   a["k"], a["K"], a["A"], a["Ea"], a["B"], a["Eb"], a["N"], a["S"],
                                   a["E"], a["L"], a["R"], a["ids"], a["w"], a["idx"], a["rank"],
                                   a["scale"], a["dt"], a["flags"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kind=2), aa.LORA_E_SHAPE),
    (dict(dt=aa.LORA_DT_F32), aa.LORA_E_DTYPE),
    (dict(R=24), aa.LORA_E_ALIGN),
    (dict(R=0), aa.LORA_E_RANK),
    (dict(E=200), aa.LORA_E_SHAPE),              # L * E > 1024
    (dict(Ea=3), aa.LORA_E_SHAPE),
    (dict(Eb=2), aa.LORA_E_SHAPE),
    (dict(rk=1), aa.LORA_E_SHAPE),               # k-reduction is a w2 option
    (dict(kind=aa.MOE_LORA_W2, rk=1, Eb=64, S=1), aa.LORA_E_SHAPE),   # needs shared lora_b
    (dict(k=0), aa.LORA_E_SHAPE),
    (dict(T=-1), aa.LORA_E_SHAPE),
    (dict(S=0), aa.LORA_E_SLICES),
    (dict(K=4100, ldx=4104), aa.LORA_E_ALIGN),
    (dict(ldy=3000), aa.LORA_E_SHAPE),
    (dict(N=(C.c_int64 * 2)(1536, 1534)), aa.LORA_E_ALIGN),
    (dict(y=None), aa.LORA_E_NULL),
    (dict(ids=None), aa.LORA_E_NULL),
    (dict(A=_ptrs(2, FAKE + 4)), aa.LORA_E_ALIGN),
    (dict(ws=None), aa.LORA_E_NULL),
    (dict(wsb=4096), aa.LORA_E_WORKSPACE),
])
def test_moe_apply_rejects_bad_arguments(kw, code):
    assert _moe(**kw) == code


def test_moe_sizes_and_align_validation():
    n = aa.moe_lora_workspace_size(2048, 8, 2, 16, 8, 64)
    assert n > 2048 * 8 * 16 * 2 * 4
    assert aa.moe_lora_workspace_size(4096, 8, 2, 16, 8, 64) > n      # more tokens
    assert aa.moe_lora_workspace_size(2048, 8, 2, 32, 8, 64) > n      # higher rank
    assert aa.moe_lora_workspace_size(2048, 8, 3, 16, 8, 64) > n      # more slices
    out = aa.C.c_size_t(0)
    size = aa.lib().moe_lora_workspace_size
    assert size(16, 2, 0, 16, 4, 4, aa.C.byref(out)) == aa.LORA_E_SLICES
    assert size(16, 2, 9, 16, 4, 4, aa.C.byref(out)) == aa.LORA_E_SLICES
    assert size(16, 2, 1, 16, 41, 25, aa.C.byref(out)) == aa.LORA_E_SHAPE   # 1025 slot-expert keys
    assert size(16, 2, 1, 0, 4, 4, aa.C.byref(out)) == aa.LORA_E_RANK
    assert size(-1, 2, 1, 16, 4, 4, aa.C.byref(out)) == aa.LORA_E_SHAPE
    assert size(16, 2, 1, 16, 4, 4, None) == aa.LORA_E_NULL
    assert size(0, 2, 1, 16, 4, 4, aa.C.byref(out)) == aa.LORA_OK
    assert aa.moe_lora_align_capacity(2, 2, 2, 4) == 12
    assert aa.moe_lora_align_capacity(2, 2, 2, 2) == 6
    lib = aa.lib()
    assert lib.moe_lora_align(FAKE, FAKE, FAKE, 16, 2, 4, 3, 16, 0, None, None, None, FAKE_WS,
                              1 << 30, None) == aa.LORA_E_SHAPE
    assert lib.moe_lora_align(FAKE, FAKE, FAKE, 16, 2, 4, 3, 16, 4, FAKE, None, None, FAKE_WS,
                              1 << 30, None) == aa.LORA_E_NULL
    assert lib.moe_lora_align(FAKE, FAKE, FAKE, 16, 2, 4, 3, 16, 4, None, None, None, FAKE_WS,
                              16, None) == aa.LORA_E_WORKSPACE
    assert _moe(T=0, y=None, x=None) == aa.LORA_OK


def test_moe_plan_reports_the_unsorted_rule():
    """moe_lora_plan: at most 1024 (token, k) pairs at rank 16 without the
    k-reduction skip the alignment; anything else builds it."""
    assert aa.moe_lora_plan(128, 8, 16)                  # 1024 pairs
    assert aa.moe_lora_plan(1, 1, 16)
    assert aa.moe_lora_plan(0, 8, 16)
    assert not aa.moe_lora_plan(129, 8, 16)              # 1032 pairs
    assert not aa.moe_lora_plan(4, 8, 32)                # another rank
    assert not aa.moe_lora_plan(4, 8, 16, reduce_k=True)
    assert not aa.moe_lora_plan(1 << 28, 16, 16)         # pair count past int32
    lib = aa.lib()
    out = aa._i32(0)
    assert lib.moe_lora_plan(-1, 8, 16, 0, aa.C.byref(out)) == aa.LORA_E_SHAPE
    assert lib.moe_lora_plan(4, 0, 16, 0, aa.C.byref(out)) == aa.LORA_E_SHAPE
    assert lib.moe_lora_plan(4, 8, 16, 0, None) == aa.LORA_E_NULL


def test_workspace_size_grows_with_every_argument():
    """A workspace shared by calls of several shapes is sized at the largest
    value of each argument; that keeps the single-launch K-split decode's
    region (at the end of the buffer) clear of every other call's regions only
    if the size never shrinks when any one argument grows."""
    rng = np.random.default_rng(11)
    lims = dict(T=(1, 1200), K=(8, 9000), S=(1, 8), R=(8, 512), L=(1, 1024))
    for _ in range(300):
        args = {k: int(rng.integers(lo, hi + 1)) for k, (lo, hi) in lims.items()}
        args["K"] -= args["K"] % 8
        args["R"] -= args["R"] % 8
        args["K"], args["R"] = max(args["K"], 8), max(args["R"], 8)
        base = aa.lora_workspace_size(args["T"], args["K"], args["S"], args["R"], args["L"])
        for k, (lo, hi) in lims.items():
            step = 8 if k in ("K", "R") else 1
            bigger = dict(args)
            bigger[k] = min(hi - (hi % step), args[k] + step * int(rng.integers(1, 64)))
            if bigger[k] <= args[k]:
                continue
            n = aa.lora_workspace_size(bigger["T"], bigger["K"], bigger["S"], bigger["R"], bigger["L"])
            assert n >= base, (args, k, bigger[k], base, n)


def test_workspace_check_rejects_before_any_runtime_call():
    lib = aa.lib()
    assert lib.lora_workspace_check(None, 1 << 20, None) == aa.LORA_E_NULL
    assert lib.lora_workspace_check(FAKE_WS + 16, 1 << 20, None) == aa.LORA_E_ALIGN
    assert lib.lora_workspace_check(FAKE_WS, 255, None) == aa.LORA_E_WORKSPACE


def _plan(**kw):
    a = dict(y=FAKE, ldy=6144, off=0, x=FAKE, ldx=4096, T=256, K=4096, A=_ptrs(3), B=_ptrs(3),
             N=(C.c_int64 * 3)(4096, 1024, 1024), S=3, L=8, R=16, idx=FAKE, rank=FAKE,
             scale=FAKE, dt=aa.LORA_DT_BF16, path=0, flags=0, ws=FAKE_WS, wsb=1 << 40)
    a.update(kw)
    out = C.c_int32(-1)
    st = aa.lib().lora_plan_packed(a["y"], a["ldy"], a["off"], a["x"], a["ldx"], a["T"], a["K"],
                                   a["A"], a["B"], a["N"], a["S"], a["L"], a["R"], a["idx"],
                                   a["rank"], a["scale"], a["dt"], a["path"], a["flags"],
                                   a["ws"], a["wsb"], C.byref(out))
    return st, out.value


def _ws_size(T, K, S, R, L):
    n = C.c_size_t(0)
    assert aa.lib().lora_workspace_size(T, K, S, R, L, C.byref(n)) == 0
    return n.value


@pytest.mark.parametrize("kw,path", [
    # decode QKV with a workspace: the single-launch K-split kernel
    (dict(), aa.LORA_PATH_RELAY),
    # ... with a workspace one byte short of lora_workspace_size(): the other single launch
    (dict(path=aa.LORA_PATH_AUTO, wsb=_ws_size(256, 4096, 3, 16, 8) - 1, ws=None),
     aa.LORA_PATH_FUSED),
    (dict(ws=None, wsb=0), aa.LORA_PATH_FUSED),
    # decode-sized batches of long slot runs: the single launch (8 slots, 512
    # and 1024 tokens); past its 1024 tokens at rank 16, the grouped kernels
    # (narrow outputs, up to 4096 tokens); at higher ranks the tile kernels
    (dict(T=512), aa.LORA_PATH_RELAY),
    (dict(T=1024), aa.LORA_PATH_RELAY),
    (dict(T=2048), aa.LORA_PATH_GROUPED),
    (dict(T=2048, L=16), aa.LORA_PATH_GROUPED),
    (dict(T=8192, L=16), aa.LORA_PATH_PREFILL),
    (dict(T=2048, R=32), aa.LORA_PATH_PREFILL),
    # many slots at rank 32: the tile kernels, not the single launch
    (dict(T=1024, L=128, R=32), aa.LORA_PATH_PREFILL),
    # many slots of a few tokens each: the other single launch
    (dict(T=64, L=64), aa.LORA_PATH_FUSED),
    (dict(T=256, L=64), aa.LORA_PATH_FUSED),
    (dict(T=512, L=32), aa.LORA_PATH_FUSED),
    # a few tokens: one work-group per token and 256 columns while the lora_a
    # its shrinks re-read stays within 44 MB (bf16, narrow, RELAY possible):
    # 12 tokens x 24 chunks x 128 KB = 36 MB; at 16 tokens (48 MB) the K-split
    # single launch; without a workspace for it the bound is 72 MB
    (dict(T=8), aa.LORA_PATH_TOKEN),
    (dict(T=1), aa.LORA_PATH_TOKEN),
    (dict(T=12), aa.LORA_PATH_TOKEN),
    (dict(T=16), aa.LORA_PATH_RELAY),
    (dict(T=32), aa.LORA_PATH_RELAY),
    (dict(T=8, ws=None, wsb=0), aa.LORA_PATH_TOKEN),           # needs no workspace
    (dict(T=16, ws=None, wsb=0), aa.LORA_PATH_TOKEN),
    (dict(T=32, ws=None, wsb=0), aa.LORA_PATH_FUSED),
    # a 32000-column lm_head: 4 tokens (500 work-groups, 66 MB) TOKEN, 16 RELAY
    (dict(T=4, S=1, N=(C.c_int64 * 1)(32000), ldy=32000), aa.LORA_PATH_TOKEN),
    (dict(T=16, S=1, N=(C.c_int64 * 1)(32000), ldy=32000), aa.LORA_PATH_RELAY),
    # rank 64 at one token: 4 passes of 16 rows, one round of work-groups
    (dict(T=1, R=64), aa.LORA_PATH_TOKEN),
    (dict(T=16, R=64), aa.LORA_PATH_GROUPED),                  # 384 x 512 KB past 72 MB
    # fp32 (the split VALU path otherwise): up to 512 MB of lora_a re-reads
    # and 4 rounds x passes; the fp32 workload at hidden 64
    (dict(dt=aa.LORA_DT_F32, R=16, T=64), aa.LORA_PATH_TOKEN),
    (dict(dt=aa.LORA_DT_F32, R=16, T=96), aa.LORA_PATH_DECODE),
    (dict(dt=aa.LORA_DT_F32, R=4, T=16, K=64, ldx=64, L=3, S=1, N=(C.c_int64 * 1)(64), ldy=64),
     aa.LORA_PATH_TOKEN),
    (dict(dt=aa.LORA_DT_F32, R=4, T=4096, K=64, ldx=64, L=3, S=1, N=(C.c_int64 * 1)(64), ldy=64),
     aa.LORA_PATH_TOKEN),
    (dict(dt=aa.LORA_DT_F32, R=4, T=4097, K=64, ldx=64, L=3, S=1, N=(C.c_int64 * 1)(64), ldy=64),
     aa.LORA_PATH_DECODE),                                     # 5 rounds of 1024 work-groups
    (dict(dt=aa.LORA_DT_F32, R=64, T=1, K=8192, ldx=8192, S=1, N=(C.c_int64 * 1)(64), ldy=64),
     aa.LORA_PATH_DECODE),                                     # 2 MB of lora_a per work-group
    # long runs per slot (8192 tokens over 16 slots): the tile kernels
    (dict(T=8192, L=16, R=64, S=2, N=(C.c_int64 * 2)(14336, 14336), ldy=28672), aa.LORA_PATH_PREFILL),
    # 128 slots at rank 128: the tile kernels
    (dict(T=1024, L=128, R=128, S=1, K=8192, ldx=8192, N=(C.c_int64 * 1)(8192), ldy=8192),
     aa.LORA_PATH_PREFILL),
    # rank 64 with few slots and a short batch: the grouped kernels
    (dict(T=64, R=64), aa.LORA_PATH_GROUPED),
    # an lm_head vocabulary: the K-split single launch wherever it runs (up to
    # 1024 tokens and 64 slots, with its workspace); past that the tile kernels
    (dict(S=1, N=(C.c_int64 * 1)(128256), ldy=128256), aa.LORA_PATH_RELAY),
    (dict(T=512, L=64, S=1, N=(C.c_int64 * 1)(128256), ldy=128256), aa.LORA_PATH_RELAY),
    (dict(T=384, S=1, N=(C.c_int64 * 1)(128256), ldy=128256), aa.LORA_PATH_RELAY),
    (dict(T=1024, L=64, S=1, N=(C.c_int64 * 1)(128256), ldy=128256), aa.LORA_PATH_RELAY),
    (dict(T=1025, S=1, N=(C.c_int64 * 1)(128256), ldy=128256), aa.LORA_PATH_PREFILL),
    (dict(T=256, L=65, S=1, N=(C.c_int64 * 1)(128256), ldy=128256), aa.LORA_PATH_PREFILL),
    # a 32000-column vocabulary: the single launch up to 1024 tokens
    (dict(T=1024, L=16, S=1, N=(C.c_int64 * 1)(32000), ldy=32000), aa.LORA_PATH_RELAY),
    # fp32: the VALU path only
    (dict(dt=aa.LORA_DT_F32, R=16), aa.LORA_PATH_DECODE),
    # rows not in 8-column units: the VALU path
    (dict(N=(C.c_int64 * 3)(4096, 1020, 1028)), aa.LORA_PATH_DECODE),
    # forced paths are reported as such
    (dict(path=aa.LORA_PATH_GROUPED), aa.LORA_PATH_GROUPED),
    (dict(path=aa.LORA_PATH_DECODE), aa.LORA_PATH_DECODE),
    (dict(path=aa.LORA_PATH_TOKEN), aa.LORA_PATH_TOKEN),
    (dict(path=aa.LORA_PATH_TOKEN, dt=aa.LORA_DT_F32, R=4, T=8192), aa.LORA_PATH_TOKEN),
])
def test_plan_reports_the_path(kw, path):
    st, got = _plan(**kw)
    assert st == aa.LORA_OK
    assert got == path, (got, path)


@pytest.mark.parametrize("kw", [dict(R=0), dict(N=None), dict(y=FAKE + 4), dict(path=99),
                                dict(path=aa.LORA_PATH_FUSED, R=128), dict(wsb=1024, path=1)])
def test_plan_fails_as_the_call_would(kw):
    st, _ = _plan(**kw)
    ap = {k: v for k, v in kw.items()}
    assert st != aa.LORA_OK
    assert st == _apply(**ap)


def test_noalloc_rejects_sizes_past_its_scratch():
    lib = aa.lib()
    args = [FAKE, 28672, 0, FAKE, 4096, 8192, 4096, _ptrs(2), _ptrs(2), (C.c_int64 * 2)(14336, 14336),
            2, 16, 64, FAKE, FAKE, FAKE, aa.LORA_DT_BF16, 0, 0, None]
    assert lib.lora_apply_packed_noalloc(*args) == aa.LORA_E_SCRATCH
    args[16] = 9                                  # a bad dtype is reported first
    assert lib.lora_apply_packed_noalloc(*args) == aa.LORA_E_DTYPE
