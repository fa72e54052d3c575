"""CPU oracle for the multi-LoRA delta -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.

The arithmetic lives in ``oracle.c`` (plain fp32 loops over tokens, built with
``-O2 -ffp-contract=off``); this module compiles it with gcc and marshals numpy
arrays through ctypes.  All floating-point arrays are float32 numpy arrays;
bf16 workloads are passed as their exact float32 widening.  Outputs are kept
in fp32 (no rounding to a storage type).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (always, when force)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("ADAPTER_APPLY_ORACLE_LIB")  # mutation tests only
        if alt:
            _lib = C.CDLL(alt)
            return _lib
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = C.CDLL(LIB)
    return _lib


_f = C.POINTER(C.c_float)
_i = C.POINTER(C.c_int32)
_l = C.POINTER(C.c_int64)


def _fp(a):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_f)


def _ip(a):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_i)


def _ptr_array(arrs):
    arr = (_f * len(arrs))()
    for i, a in enumerate(arrs):
        arr[i] = _fp(a)
    return arr


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def lora_shrink(x, A, idx, slot_rank, R=None):
    """buf[S][T][R] = shrink of x by the per-slice stacked lora_a tensors."""
    lib = _load()
    x = _f32(x)
    A = [_f32(a) for a in A]
    T, K = x.shape
    L, Rr, K2 = A[0].shape
    assert K2 == K
    R = Rr if R is None else R
    idx, slot_rank = _i32(idx), _i32(slot_rank)
    buf = np.zeros((len(A), T, R), np.float32)
    lib.oracle_lora_shrink(_fp(buf), _fp(x), C.c_int64(K), C.c_int32(T), C.c_int32(K),
                           _ptr_array(A), C.c_int32(len(A)), C.c_int32(L), C.c_int32(R),
                           _ip(idx), _ip(slot_rank))
    return buf


def lora_expand(y, buf, B, idx, slot_rank, scale, y_col_offset=0):
    """Returns y (fp32 copy) after y[:, off_s + n] += scale * buf . B_s^T."""
    lib = _load()
    y = _f32(y).copy()
    buf = _f32(buf)
    B = [_f32(b) for b in B]
    S, T, R = buf.shape
    L = B[0].shape[0]
    N = (C.c_int64 * S)(*[b.shape[1] for b in B])
    lib.oracle_lora_expand(_fp(y), C.c_int64(y.shape[1]), C.c_int64(y_col_offset), _fp(buf),
                           C.c_int32(T), _ptr_array(B), N, C.c_int32(S), C.c_int32(L),
                           C.c_int32(R), _ip(_i32(idx)), _ip(_i32(slot_rank)),
                           _fp(_f32(scale)))
    return y


def lora_apply(y, x, A, B, idx, slot_rank, scale, y_col_offset=0):
    """Returns (y_out fp32, buf fp32) for the packed shrink + expand."""
    lib = _load()
    y = _f32(y).copy()
    x = _f32(x)
    A = [_f32(a) for a in A]
    B = [_f32(b) for b in B]
    T, K = x.shape
    L, R, _ = A[0].shape
    S = len(A)
    N = (C.c_int64 * S)(*[b.shape[1] for b in B])
    buf = np.zeros((S, T, R), np.float32)
    lib.oracle_lora_apply(_fp(y), C.c_int64(y.shape[1]), C.c_int64(y_col_offset), _fp(x),
                          C.c_int64(K), C.c_int32(T), C.c_int32(K), _ptr_array(A),
                          _ptr_array(B), N, C.c_int32(S), C.c_int32(L), C.c_int32(R),
                          _ip(_i32(idx)), _ip(_i32(slot_rank)), _fp(_f32(scale)), _fp(buf))
    return y, buf


def segments(idx, slot_rank, L, R=1 << 30):
    """(perm[T], slot_start[L+1], n_invalid) of the stable sort by slot."""
    lib = _load()
    idx = _i32(idx)
    slot_rank = _i32(slot_rank)
    T = idx.shape[0]
    perm = np.empty(T, np.int32)
    start = np.empty(L + 1, np.int32)
    ninv = C.c_int32(0)
    lib.oracle_segments(_ip(idx), _ip(slot_rank), C.c_int32(T), C.c_int32(L), C.c_int32(R),
                        _ip(perm), _ip(start), C.byref(ninv))
    return perm, start, int(ninv.value)


def moe_align_capacity(T, k, E, block_m):
    """Entries per slot that always suffice for moe_align's padded output."""
    c = T * k + E * (block_m - 1)
    return (c + block_m - 1) // block_m * block_m


def moe_align(topk_ids, idx, slot_rank, E, L, block_m, R=1 << 30):
    lib = _load()
    topk_ids = _i32(topk_ids)
    T, k = topk_ids.shape
    cap = moe_align_capacity(T, k, E, block_m)
    sorted_ids = np.empty((L, cap), np.int32)
    block_expert = np.empty((L, cap // block_m), np.int32)
    npp = np.empty(L, np.int32)
    lib.oracle_moe_align(_ip(topk_ids), _ip(_i32(idx)), _ip(_i32(slot_rank)), C.c_int32(T),
                         C.c_int32(k), C.c_int32(E), C.c_int32(L), C.c_int32(R),
                         C.c_int32(block_m), C.c_int32(cap), _ip(sorted_ids), _ip(block_expert),
                         _ip(npp))
    return sorted_ids, block_expert, npp


def moe_lora_apply(kind, y, x, A, B, topk_ids, topk_w, idx, slot_rank, scale, E,
                   reduce_k=False):
    """kind 0 = w13 (x [T,K], y [T*k, sum N]); kind 1 = w2 (x [T*k, K],
    y [T*k, N] or [T, N] when reduce_k).  Returns the fp32 result."""
    lib = _load()
    y = _f32(y).copy()
    x = _f32(x)
    A = [_f32(a) for a in A]
    B = [_f32(b) for b in B]
    topk_ids = _i32(topk_ids)
    T, k = topk_ids.shape
    L, E_a, R, K = A[0].shape
    E_b = B[0].shape[1]
    S = len(A)
    N = (C.c_int64 * S)(*[b.shape[2] for b in B])
    w = _fp(_f32(topk_w)) if topk_w is not None else None
    scratch = np.zeros(R, np.float32)
    lib.oracle_moe_lora_apply(C.c_int32(kind), _fp(y), C.c_int64(y.shape[1]),
                              C.c_int32(int(reduce_k)), _fp(x), C.c_int64(x.shape[1]),
                              C.c_int32(T), C.c_int32(k), C.c_int32(K), _ptr_array(A),
                              C.c_int32(E_a), _ptr_array(B), C.c_int32(E_b), N,
                              C.c_int32(S), C.c_int32(E), C.c_int32(L), C.c_int32(R),
                              _ip(topk_ids), w, _ip(_i32(idx)), _ip(_i32(slot_rank)),
                              _fp(_f32(scale)), _fp(scratch))
    return y
