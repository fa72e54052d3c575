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

LORA_DT_F32 = 0
LORA_DT_BF16 = 1

LORA_PATH_AUTO = 0
LORA_PATH_DECODE = 1
LORA_PATH_PREFILL = 2
LORA_PATH_FUSED = 3
LORA_PATH_GROUPED = 4
LORA_PATH_RELAY = 5

MOE_LORA_W13 = 0
MOE_LORA_W2 = 1

LORA_FLAG_SEGMENTS_READY = 1
LORA_FLAG_ACTIVE_ONLY = 2
LORA_FLAG_PARTIAL = 4

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
    "lora_segment_layout": (_i32, [_i32, _i32, C.POINTER(SegmentLayout)]),
    "lora_build_segments": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "lora_shrink": (_i32, [_vp, _vp, _i64, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _i32,
                           _i32, _u32, _vp, _sz, _vp]),
    "lora_expand": (_i32, [_vp, _i64, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                           _vp, _i32, _i32, _u32, _vp, _sz, _vp]),
    "lora_apply_packed": (_i32, [_vp, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _i32,
                                 _i32, _i32, _vp, _vp, _vp, _i32, _i32, _u32, _vp, _sz, _vp]),
    "moe_lora_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, C.POINTER(_sz)]),
    "moe_lora_align_capacity": (_i32, [_i32, _i32, _i32, _i32, C.POINTER(_i32)]),
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


def lora_segment_layout(T: int, L: int) -> dict:
    out = SegmentLayout()
    _check(lib().lora_segment_layout(T, L, C.byref(out)), "lora_segment_layout")
    return {f: getattr(out, f) for f, _ in SegmentLayout._fields_}


def lora_build_segments(idx, slot_rank, L: int, R: int, ws, stream=None):
    _check(lib().lora_build_segments(_ptr(idx), _ptr(slot_rank), idx.shape[0], L, R, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "lora_build_segments")


def lora_shrink(buf, x, A: Sequence, idx, slot_rank, ws, path: int = LORA_PATH_AUTO,
                flags: int = 0, stream=None):
    """buf [S, T, R] fp32 (overwritten); x [T, K]; A[s] [L, R, K]."""
    _rowmajor(x, "x")
    _stacked(A, "A", 3)
    T, K = x.shape
    L, R, _ = A[0].shape
    _check(lib().lora_shrink(_ptr(buf), _ptr(x), x.stride(0), T, K, _ptr_array(A), len(A), L, R,
                             _ptr(idx), _ptr(slot_rank), _dtype_code(x), path, flags, _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "lora_shrink")


def lora_expand(y, buf, B: Sequence, idx, slot_rank, scale, ws, y_col_offset: int = 0,
                path: int = LORA_PATH_AUTO, flags: int = 0, stream=None):
    """y [T, >= y_col_offset + sum N] updated in place; buf [S, T, R] fp32;
    B[s] [L, N_s, R]; scale [L] fp32."""
    _rowmajor(y, "y")
    _stacked(B, "B", 3)
    S, T, R = buf.shape
    L = B[0].shape[0]
    N = (_i64 * S)(*[b.shape[1] for b in B])
    _check(lib().lora_expand(_ptr(y), y.stride(0), y_col_offset, _ptr(buf), T, _ptr_array(B), N,
                             S, L, R, _ptr(idx), _ptr(slot_rank), _ptr(scale), _dtype_code(y),
                             path, flags, _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "lora_expand")


def lora_apply_packed(y, x, A: Sequence, B: Sequence, idx, slot_rank, scale, ws,
                      y_col_offset: int = 0, path: int = LORA_PATH_AUTO, flags: int = 0,
                      stream=None):
    """y += scale * (x A^T) B^T per slice, in place."""
    _rowmajor(x, "x")
    _rowmajor(y, "y")
    _stacked(A, "A", 3)
    _stacked(B, "B", 3)
    T, K = x.shape
    L, R, _ = A[0].shape
    S = len(A)
    N = (_i64 * S)(*[b.shape[1] for b in B])
    _check(lib().lora_apply_packed(_ptr(y), y.stride(0), y_col_offset, _ptr(x), x.stride(0), T, K,
                                   _ptr_array(A), _ptr_array(B), N, S, L, R, _ptr(idx),
                                   _ptr(slot_rank), _ptr(scale), _dtype_code(x), path, flags,
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lora_apply_packed")


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


def alloc_moe_workspace(T: int, top_k: int, S: int, R: int, L: int, E: int, device="cuda"):
    return _aligned_ws(moe_lora_workspace_size(T, top_k, S, R, L, E), device)


def moe_lora_align(topk_ids, idx, slot_rank, E: int, L: int, R: int, block_m: int, ws,
                   sorted_ids=None, block_expert=None, num_post_padded=None, stream=None):
    """topk_ids [T, top_k] int32; outputs (optional) [L, cap], [L, cap/bm], [L] int32."""
    T, k = topk_ids.shape
    _check(lib().moe_lora_align(_ptr(topk_ids), _ptr(idx), _ptr(slot_rank), T, k, E, L, R,
                                block_m, _ptr(sorted_ids), _ptr(block_expert),
                                _ptr(num_post_padded), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_lora_align")


def moe_lora_apply(kind: int, y, x, A: Sequence, B: Sequence, topk_ids, topk_w, idx, slot_rank,
                   scale, E: int, ws, reduce_k: bool = False, flags: int = 0, stream=None):
    """A[s] [L, E_a, R, K]; B[s] [L, E_b, N_s, R]; y updated in place."""
    _rowmajor(x, "x")
    _rowmajor(y, "y")
    _stacked(A, "A", 4)
    _stacked(B, "B", 4)
    T, k = topk_ids.shape
    L, E_a, R, K = A[0].shape
    E_b = B[0].shape[1]
    S = len(A)
    N = (_i64 * S)(*[b.shape[2] for b in B])
    _check(lib().moe_lora_apply(kind, _ptr(y), y.stride(0), int(bool(reduce_k)), _ptr(x),
                                x.stride(0), T, k, K, _ptr_array(A), E_a, _ptr_array(B), E_b, N, S,
                                E, L, R, _ptr(topk_ids), _ptr(topk_w), _ptr(idx), _ptr(slot_rank),
                                _ptr(scale), _dtype_code(x), flags, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_lora_apply")
