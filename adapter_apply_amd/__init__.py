"""Python binding of the adapter_apply C ABI (include/adapter_apply.h).

Argument marshalling only: every function here derives sizes, strides and
pointers from torch tensors and calls the entry point of the same name in
``libadapter_apply.so``.  All arithmetic runs in the library's HIP kernels on
the GPU; there is no fallback.  PyTorch supplies device memory and the
current stream.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libadapter_apply.so")

LORA_OK = 0
LORA_E_NULL = 1
LORA_E_SHAPE = 2
LORA_E_DTYPE = 3
LORA_E_RANK = 4
LORA_E_SLICES = 5
LORA_E_WORKSPACE = 6
LORA_E_ALIGN = 7
LORA_E_PATH = 8
LORA_E_LAUNCH = 9
LORA_E_TIMEOUT = 10
LORA_E_RUNTIME = 11
LORA_E_SCRATCH = 12
LORA_STATIC_SCRATCH_BYTES = 32 << 20

LORA_DT_F32 = 0
LORA_DT_BF16 = 1

LORA_PATH_AUTO = 0
LORA_PATH_DECODE = 1
LORA_PATH_PREFILL = 2
LORA_PATH_FUSED = 3
LORA_PATH_GROUPED = 4
LORA_PATH_RELAY = 5
LORA_PATH_TOKEN = 6

MOE_LORA_W13 = 0
MOE_LORA_W2 = 1

LORA_FLAG_SEGMENTS_READY = 1
LORA_FLAG_ACTIVE_ONLY = 2
LORA_FLAG_PARTIAL = 4
LORA_FLAG_RELAY_GIVE_UP = 8   # test hook: the RELAY path's waits give up at once

# Every symbol the header declares, with its ctypes signature.
_vp = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_u32 = C.c_uint32
_sz = C.c_size_t


class SegmentLayout(C.Structure):
    _fields_ = [("header", _i64), ("slot_start", _i64), ("perm", _i64),
                ("tiles_decode", _i64), ("tiles_prefill", _i64),
                ("tile_decode_tokens", _i32), ("tile_prefill_tokens", _i32)]


SIGNATURES = {
    "lora_status_string": (C.c_char_p, [_i32]),
    "lora_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, C.POINTER(_sz)]),
    "lora_workspace_init": (_i32, [_vp, _sz, _vp]),
    "lora_workspace_check": (_i32, [_vp, _sz, _vp]),
    "lora_segment_layout": (_i32, [_i32, _i32, C.POINTER(SegmentLayout)]),
    "lora_build_segments": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "lora_shrink": (_i32, [_vp, _vp, _i64, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _i32,
                           _i32, _u32, _vp, _sz, _vp]),
    "lora_expand": (_i32, [_vp, _i64, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                           _vp, _i32, _i32, _u32, _vp, _sz, _vp]),
    "lora_apply_packed": (_i32, [_vp, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _i32,
                                 _i32, _i32, _vp, _vp, _vp, _i32, _i32, _u32, _vp, _sz, _vp]),
    "lora_plan_packed": (_i32, [_vp, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _i32,
                                _i32, _i32, _vp, _vp, _vp, _i32, _i32, _u32, _vp, _sz,
                                C.POINTER(_i32)]),
    "lora_apply_packed_noalloc": (_i32, [_vp, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp,
                                         _i32, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _u32, _vp]),
    "moe_lora_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, C.POINTER(_sz)]),
    "moe_lora_align_capacity": (_i32, [_i32, _i32, _i32, _i32, C.POINTER(_i32)]),
    "moe_lora_plan": (_i32, [_i32, _i32, _i32, _i32, C.POINTER(_i32)]),
    "moe_lora_align": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                              _vp, _sz, _vp]),
    "moe_lora_apply": (_i32, [_i32, _vp, _i64, _i32, _vp, _i64, _i32, _i32, _i32, _vp, _i32, _vp,
                              _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32,
                              _u32, _vp, _sz, _vp]),
}

_lib = None


class LoraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (status {code})")


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python adapter_apply_amd/build.py` "
                "(or __graft_entry__.build()); there is no fallback path")
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(code: int) -> str:
    return lib().lora_status_string(code).decode()


def _check(code: int, where: str):
    if code != LORA_OK:
        raise LoraError(code, where)


# ---------------------------------------------------------------------------
# tensor marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        torch = _torch()
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LORA_DT_BF16
    if t.dtype == torch.float32:
        return LORA_DT_F32
    return -1


def _ptr_array(ts: Sequence):
    arr = (_vp * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")


def _stacked(ts, name, ndim):
    for t in ts:
        if t.dim() != ndim or not t.is_contiguous():
            raise ValueError(f"{name} tensors must be contiguous with {ndim} dims")


# Argument checks of the wrappers.  The C library checks sizes, alignment and
# pointers, but it cannot see a tensor's dtype, device or length: an int64
# idx would be read as pairs of int32, a short idx or y read or written past
# its end.  So every wrapper checks these here and raises ValueError before
# the C call (dtypes and shapes first, then the device).

def _need_dtype(t, dtypes, name):
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected " +
                         " or ".join(str(d) for d in dtypes))


def _need_shape(t, shape, name):
    """shape: a tuple with None for dimensions not checked."""
    if t.dim() != len(shape) or any(e is not None and t.shape[i] != e for i, e in enumerate(shape)):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}; expected {want}")


def _need_vec(t, n, dtype, name):
    _need_dtype(t, (dtype,), name)
    if t.dim() != 1 or t.shape[0] != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous 1-D tensor of {n} elements "
                         f"(got shape {list(t.shape)})")


def _same_list(ts, name, ndim, dtype, shape_fn=None):
    if len(ts) < 1:
        raise ValueError(f"{name} must hold at least one tensor")
    _stacked(ts, name, ndim)
    for i, t in enumerate(ts):
        _need_dtype(t, (dtype,), f"{name}[{i}]")
        if shape_fn is not None:
            _need_shape(t, shape_fn(i), f"{name}[{i}]")


def _need_device(tensors):
    """Every tensor on one GPU."""
    ts = [t for t in tensors if t is not None]
    for t in ts:
        if not t.is_cuda:
            raise ValueError(f"every tensor must be on a GPU; got one on {t.device}")
    devs = {t.device for t in ts}
    if len(devs) > 1:
        raise ValueError(f"tensors are on several devices: {sorted(str(d) for d in devs)}")


def _float_types():
    torch = _torch()
    return (torch.bfloat16, torch.float32)


def _check_meta(idx, slot_rank, scale, T, L):
    torch = _torch()
    _need_vec(idx, T, torch.int32, "idx")
    if slot_rank is not None:
        _need_vec(slot_rank, L, torch.int32, "slot_rank")
    if scale is not None:
        _need_vec(scale, L, torch.float32, "scale")


def _check_ws(ws):
    if ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous 1-D tensor")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def lora_workspace_size(T: int, K: int, S: int, R: int, L: int) -> int:
    n = _sz(0)
    _check(lib().lora_workspace_size(T, K, S, R, L, C.byref(n)), "lora_workspace_size")
    return int(n.value)


def lora_workspace_init(ws, stream=None):
    _check(lib().lora_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lora_workspace_init")


def lora_workspace_check(ws, stream=None):
    """Synchronises the stream and raises LoraError(LORA_E_TIMEOUT) if a
    single-launch K-split decode call on this workspace had a wait give up
    since the last check (the library has then zero-filled the workspace)."""
    _check_ws(ws)
    _check(lib().lora_workspace_check(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lora_workspace_check")


def lora_segment_layout(T: int, L: int) -> dict:
    out = SegmentLayout()
    _check(lib().lora_segment_layout(T, L, C.byref(out)), "lora_segment_layout")
    return {f: getattr(out, f) for f, _ in SegmentLayout._fields_}


def lora_build_segments(idx, slot_rank, L: int, R: int, ws, stream=None):
    _check_meta(idx, slot_rank, None, idx.shape[0] if idx.dim() == 1 else -1, L)
    _check_ws(ws)
    _need_device([idx, slot_rank, ws])
    _check(lib().lora_build_segments(_ptr(idx), _ptr(slot_rank), idx.shape[0], L, R, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "lora_build_segments")


def lora_shrink(buf, x, A: Sequence, idx, slot_rank, ws, path: int = LORA_PATH_AUTO,
                flags: int = 0, stream=None):
    """buf [S, T, R] fp32 (overwritten); x [T, K]; A[s] [L, R, K]."""
    torch = _torch()
    _rowmajor(x, "x")
    _need_dtype(x, _float_types(), "x")
    T, K = x.shape
    _same_list(A, "A", 3, x.dtype)
    L, R, _ = A[0].shape
    _same_list(A, "A", 3, x.dtype, lambda i: (L, R, K))
    _need_dtype(buf, (torch.float32,), "buf")
    _need_shape(buf, (len(A), T, R), "buf")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _check_meta(idx, slot_rank, None, T, L)
    _check_ws(ws)
    _need_device([buf, x, *A, idx, slot_rank, ws])
    _check(lib().lora_shrink(_ptr(buf), _ptr(x), x.stride(0), T, K, _ptr_array(A), len(A), L, R,
                             _ptr(idx), _ptr(slot_rank), _dtype_code(x), path, flags, _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "lora_shrink")


def lora_expand(y, buf, B: Sequence, idx, slot_rank, scale, ws, y_col_offset: int = 0,
                path: int = LORA_PATH_AUTO, flags: int = 0, stream=None):
    """y [T, >= y_col_offset + sum N] updated in place; buf [S, T, R] fp32;
    B[s] [L, N_s, R]; scale [L] fp32."""
    torch = _torch()
    _rowmajor(y, "y")
    _need_dtype(y, _float_types(), "y")
    _need_dtype(buf, (torch.float32,), "buf")
    if buf.dim() != 3 or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous [S, T, R] tensor")
    S, T, R = buf.shape
    _same_list(B, "B", 3, y.dtype)
    L = B[0].shape[0]
    if len(B) != S:
        raise ValueError(f"buf has {S} slices but B holds {len(B)} tensors")
    _same_list(B, "B", 3, y.dtype, lambda i: (L, None, R))
    _need_shape(y, (T, None), "y")
    _check_meta(idx, slot_rank, scale, T, L)
    _check_ws(ws)
    _need_device([y, buf, *B, idx, slot_rank, scale, ws])
    N = (_i64 * S)(*[b.shape[1] for b in B])
    _check(lib().lora_expand(_ptr(y), y.stride(0), y_col_offset, _ptr(buf), T, _ptr_array(B), N,
                             S, L, R, _ptr(idx), _ptr(slot_rank), _ptr(scale), _dtype_code(y),
                             path, flags, _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "lora_expand")


def _check_packed(y, x, A, B, idx, slot_rank, scale, ws):
    _rowmajor(x, "x")
    _rowmajor(y, "y")
    _need_dtype(x, _float_types(), "x")
    _need_dtype(y, (x.dtype,), "y")
    T, K = x.shape
    _same_list(A, "A", 3, x.dtype)
    L, R, _ = A[0].shape
    _same_list(A, "A", 3, x.dtype, lambda i: (L, R, K))
    if len(B) != len(A):
        raise ValueError(f"A holds {len(A)} tensors but B holds {len(B)}")
    _same_list(B, "B", 3, x.dtype, lambda i: (L, None, R))
    _need_shape(y, (T, None), "y")
    _check_meta(idx, slot_rank, scale, T, L)
    if ws is not None:
        _check_ws(ws)
    _need_device([y, x, *A, *B, idx, slot_rank, scale, ws])


def lora_apply_packed(y, x, A: Sequence, B: Sequence, idx, slot_rank, scale, ws,
                      y_col_offset: int = 0, path: int = LORA_PATH_AUTO, flags: int = 0,
                      stream=None, check: bool = False):
    """y += scale * (x A^T) B^T per slice, in place.  check=True then runs
    lora_workspace_check (synchronises; raises if a wait gave up)."""
    _check_packed(y, x, A, B, idx, slot_rank, scale, ws)
    T, K = x.shape
    L, R, _ = A[0].shape
    S = len(A)
    N = (_i64 * S)(*[b.shape[1] for b in B])
    _check(lib().lora_apply_packed(_ptr(y), y.stride(0), y_col_offset, _ptr(x), x.stride(0), T, K,
                                   _ptr_array(A), _ptr_array(B), N, S, L, R, _ptr(idx),
                                   _ptr(slot_rank), _ptr(scale), _dtype_code(x), path, flags,
                                   _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)),
           "lora_apply_packed")
    if check and ws is not None:
        lora_workspace_check(ws, stream)


def lora_plan_packed(y, x, A: Sequence, B: Sequence, idx, slot_rank, scale, ws,
                     y_col_offset: int = 0, path: int = LORA_PATH_AUTO, flags: int = 0) -> int:
    """The LORA_PATH_* that lora_apply_packed takes for these arguments
    (nothing is run)."""
    _check_packed(y, x, A, B, idx, slot_rank, scale, ws)
    T, K = x.shape
    L, R, _ = A[0].shape
    S = len(A)
    N = (_i64 * S)(*[b.shape[1] for b in B])
    out = _i32(-1)
    _check(lib().lora_plan_packed(_ptr(y), y.stride(0), y_col_offset, _ptr(x), x.stride(0), T, K,
                                  _ptr_array(A), _ptr_array(B), N, S, L, R, _ptr(idx),
                                  _ptr(slot_rank), _ptr(scale), _dtype_code(x), path, flags,
                                  _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                  C.byref(out)), "lora_plan_packed")
    return int(out.value)


PATH_NAMES = {LORA_PATH_AUTO: "auto", LORA_PATH_DECODE: "decode", LORA_PATH_PREFILL: "prefill",
              LORA_PATH_FUSED: "fused", LORA_PATH_GROUPED: "grouped", LORA_PATH_RELAY: "relay",
              LORA_PATH_TOKEN: "token"}


def lora_apply_packed_noalloc(y, x, A: Sequence, B: Sequence, idx, slot_rank, scale,
                              y_col_offset: int = 0, path: int = LORA_PATH_AUTO, flags: int = 0,
                              stream=None):
    """lora_apply_packed with the library's static per-GPU scratch instead of
    a workspace: allocates nothing.  Calls overlapping in time on one GPU
    race (they share the array)."""
    _check_packed(y, x, A, B, idx, slot_rank, scale, None)
    T, K = x.shape
    L, R, _ = A[0].shape
    S = len(A)
    N = (_i64 * S)(*[b.shape[1] for b in B])
    _check(lib().lora_apply_packed_noalloc(_ptr(y), y.stride(0), y_col_offset, _ptr(x),
                                           x.stride(0), T, K, _ptr_array(A), _ptr_array(B), N, S,
                                           L, R, _ptr(idx), _ptr(slot_rank), _ptr(scale),
                                           _dtype_code(x), path, flags, _stream(stream)),
           "lora_apply_packed_noalloc")


def lora_static_scratch_check(stream=None):
    """lora_workspace_check on the static scratch of lora_apply_packed_noalloc
    (current device)."""
    _check(lib().lora_workspace_check(None, 0, _stream(stream)), "lora_workspace_check")


def _aligned_ws(n: int, device):
    torch = _torch()
    ws = torch.empty(max(n, 256) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + max(n, 256)]
    lora_workspace_init(ws)
    return ws


def alloc_workspace(T: int, K: int, S: int, R: int, L: int, device="cuda"):
    """A zero-filled workspace tensor (uint8) of the required size.  A
    workspace shared by calls of several shapes must be sized with the
    largest value of each argument (the single-launch K-split decode keeps a
    zero-on-entry region at its end, clear of the other calls' regions only
    then)."""
    return _aligned_ws(lora_workspace_size(T, K, S, R, L), device)


# ---------------------------------------------------------------------------
# fused MoE
# ---------------------------------------------------------------------------

def moe_lora_workspace_size(T: int, top_k: int, S: int, R: int, L: int, E: int) -> int:
    n = _sz(0)
    _check(lib().moe_lora_workspace_size(T, top_k, S, R, L, E, C.byref(n)),
           "moe_lora_workspace_size")
    return int(n.value)


def moe_lora_align_capacity(T: int, top_k: int, E: int, block_m: int) -> int:
    c = _i32(0)
    _check(lib().moe_lora_align_capacity(T, top_k, E, block_m, C.byref(c)),
           "moe_lora_align_capacity")
    return int(c.value)


def moe_lora_plan(T: int, top_k: int, R: int, reduce_k: bool = False) -> bool:
    """True when moe_lora_apply without LORA_FLAG_SEGMENTS_READY skips the
    alignment for these sizes (the library's own rule)."""
    u = _i32(0)
    _check(lib().moe_lora_plan(T, top_k, R, int(bool(reduce_k)), C.byref(u)), "moe_lora_plan")
    return bool(u.value)


def alloc_moe_workspace(T: int, top_k: int, S: int, R: int, L: int, E: int, device="cuda"):
    return _aligned_ws(moe_lora_workspace_size(T, top_k, S, R, L, E), device)


def moe_lora_align(topk_ids, idx, slot_rank, E: int, L: int, R: int, block_m: int, ws,
                   sorted_ids=None, block_expert=None, num_post_padded=None, stream=None):
    """topk_ids [T, top_k] int32; outputs (optional) [L, cap], [L, cap/bm], [L] int32."""
    torch = _torch()
    if topk_ids.dim() != 2 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [T, top_k] tensor")
    _need_dtype(topk_ids, (torch.int32,), "topk_ids")
    T, k = topk_ids.shape
    _check_meta(idx, slot_rank, None, T, L)
    outs = (sorted_ids, block_expert, num_post_padded)
    if any(o is not None for o in outs):
        if any(o is None for o in outs):
            raise ValueError("give all three alignment outputs or none")
        cap = moe_lora_align_capacity(T, k, E, block_m)
        for o, shape, name in ((sorted_ids, (L, cap), "sorted_ids"),
                               (block_expert, (L, cap // block_m), "block_expert"),
                               (num_post_padded, (L,), "num_post_padded")):
            _need_dtype(o, (torch.int32,), name)
            _need_shape(o, shape, name)
            if not o.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
    _check_ws(ws)
    _need_device([topk_ids, idx, slot_rank, ws, *outs])
    _check(lib().moe_lora_align(_ptr(topk_ids), _ptr(idx), _ptr(slot_rank), T, k, E, L, R,
                                block_m, _ptr(sorted_ids), _ptr(block_expert),
                                _ptr(num_post_padded), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_lora_align")


def moe_lora_apply(kind: int, y, x, A: Sequence, B: Sequence, topk_ids, topk_w, idx, slot_rank,
                   scale, E: int, ws, reduce_k: bool = False, flags: int = 0, stream=None):
    """A[s] [L, E_a, R, K]; B[s] [L, E_b, N_s, R]; y updated in place."""
    torch = _torch()
    _rowmajor(x, "x")
    _rowmajor(y, "y")
    _need_dtype(x, _float_types(), "x")
    _need_dtype(y, (x.dtype,), "y")
    if topk_ids.dim() != 2 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [T, top_k] tensor")
    _need_dtype(topk_ids, (torch.int32,), "topk_ids")
    T, k = topk_ids.shape
    _same_list(A, "A", 4, x.dtype)
    L, E_a, R, K = A[0].shape
    _same_list(A, "A", 4, x.dtype, lambda i: (L, E_a, R, K))
    if len(B) != len(A):
        raise ValueError(f"A holds {len(A)} tensors but B holds {len(B)}")
    _same_list(B, "B", 4, x.dtype)
    E_b = B[0].shape[1]
    _same_list(B, "B", 4, x.dtype, lambda i: (L, E_b, None, R))
    if kind == MOE_LORA_W13:
        _need_shape(x, (T, K), "x")
        _need_shape(y, (T * k, None), "y")
    else:
        _need_shape(x, (T * k, K), "x")
        _need_shape(y, (T if reduce_k else T * k, None), "y")
    if topk_w is not None:
        _need_dtype(topk_w, (torch.float32,), "topk_w")
        _need_shape(topk_w, (T, k), "topk_w")
        if not topk_w.is_contiguous():
            raise ValueError("topk_w must be contiguous")
    _check_meta(idx, slot_rank, scale, T, L)
    _check_ws(ws)
    _need_device([y, x, *A, *B, topk_ids, topk_w, idx, slot_rank, scale, ws])
    S = len(A)
    N = (_i64 * S)(*[b.shape[2] for b in B])
    _check(lib().moe_lora_apply(kind, _ptr(y), y.stride(0), int(bool(reduce_k)), _ptr(x),
                                x.stride(0), T, k, K, _ptr_array(A), E_a, _ptr_array(B), E_b, N, S,
                                E, L, R, _ptr(topk_ids), _ptr(topk_w), _ptr(idx), _ptr(slot_rank),
                                _ptr(scale), _dtype_code(x), flags, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_lora_apply")
