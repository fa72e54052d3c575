"""Seeded synthetic workloads for the multi-LoRA delta.

This module only draws random inputs and lays them out in the stacked-slot
format; it performs none of the delta's arithmetic.  Both the CPU oracle
(through the tests) and the HIP library consume the arrays it returns.

Layouts follow the vLLM ``vllm.lora.layers`` page:
  * lora_a per slice: ``[max_loras, R, K]`` (the page's ``[max_loras, 1, R, K]``
    without the singleton dim), section MergedColumnParallelLinearWithLoRA,
    create_lora_weights;
  * lora_b per slice: ``[max_loras, N_s, R]``, same section;
  * a rank-r adapter fills the first r rows of A and the first r columns of B
    and the rest of the slot is zero (reset_lora then set_lora, same section);
  * MoE: lora_a ``[max_loras, E_a, R, K]``, lora_b ``[max_loras, E_b, N, R]``
    with ``E_a``/``E_b`` equal to 1 for the shared-outer layout (FusedMoEWithLoRA
    section of that page; the vLLM PR #48884 report, item 4 of its change list).

``N(mu, sigma)`` in the workload recipes is read as mean and standard
deviation.  Floating-point draws are made in float32 and, for bf16 workloads,
rounded to the nearest bf16 (ties to even) so that every consumer sees the
same values; the arrays are returned as float32 holding bf16-representable
numbers.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np


# ----------------------------------------------------------------------------
# storage-format helpers (data preparation, not arithmetic of the method)
# ----------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16-representable float32 values."""
    return bf16_widen(bf16_bits(a))


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_bf16(a) if dtype == "bf16" else a


# ----------------------------------------------------------------------------
# linear (packed-slice) workloads
# ----------------------------------------------------------------------------

@dataclass
class LinearCase:
    name: str
    dtype: str                 # "f32" or "bf16"
    T: int
    K: int
    N: List[int]               # per-slice output widths
    R: int                     # max rank (padded)
    L: int                     # max_loras slots
    x: np.ndarray              # [T, K]
    A: List[np.ndarray]        # S x [L, R, K]
    B: List[np.ndarray]        # S x [L, N_s, R]
    y0: np.ndarray             # [T, sum(N)]
    idx: np.ndarray            # [T] int32, -1 = no adapter
    slot_rank: np.ndarray      # [L] int32, 0 = empty slot
    scale: np.ndarray          # [L] float32
    note: str = ""

    @property
    def S(self) -> int:
        return len(self.N)

    @property
    def Ntot(self) -> int:
        return int(sum(self.N))


def _zero_pad(A, B, slot_rank):
    for a, b in zip(A, B):
        for s, r in enumerate(slot_rank):
            a[s, r:, :] = 0.0
            b[s, :, r:] = 0.0


def make_linear(name, T, K, N, R, L, idx, slot_rank, scale, dtype, seed,
                x_std=1.0, w_std=0.02, y_std=1.0, note=""):
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, K), x_std, dtype)
    A = [_normal(rng, (L, R, K), w_std, dtype) for _ in N]
    B = [_normal(rng, (L, n, R), w_std, dtype) for n in N]
    _zero_pad(A, B, slot_rank)
    y0 = _normal(rng, (T, int(sum(N))), y_std, dtype) if y_std > 0 else \
        np.zeros((T, int(sum(N))), np.float32)
    return LinearCase(name, dtype, T, K, list(N), R, L, x, A, B, y0,
                      np.asarray(idx, np.int32), np.asarray(slot_rank, np.int32),
                      np.asarray(scale, np.float32), note)


def config_tiny(seed=1001):
    """16 tokens, hidden 64, one 64-wide slice, rank 4, 3 slots, fp32,
    idx uniform over {-1,0,1,2}, x~N(0,1), A,B~N(0,0.1), scale 2."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, 3, size=16).astype(np.int32)
    return make_linear("tiny", 16, 64, [64], 4, 3, idx, [4, 4, 4], [2.0] * 3,
                       "f32", seed + 1, w_std=0.1)


def config_decode(seed=1002, T=256):
    """Decode: 256 tokens, hidden 4096, QKV slices 4096/1024/1024, rank 16,
    8 slots, 10% idx=-1 else uniform over slots, bf16, A,B~N(0,0.02), scale 2."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, 8, size=T).astype(np.int32)
    idx[rng.random(T) < 0.1] = -1
    return make_linear("decode_qkv", T, 4096, [4096, 1024, 1024], 16, 8, idx,
                       [16] * 8, [2.0] * 8, "bf16", seed + 1)


def config_logits(seed=1006, T=256, vocab=128256):
    """lm_head LoRA at decode: 256 tokens, hidden 4096, one vocab-wide slice
    (128256 columns by default; the pages accept 32000..257024), rank 16,
    8 slots, 10% idx=-1 else uniform over slots, bf16, A,B~N(0,0.02), scale 1
    (the logits call passes 1.0)."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, 8, size=T).astype(np.int32)
    idx[rng.random(T) < 0.1] = -1
    return make_linear("logits", T, 4096, [vocab], 16, 8, idx, [16] * 8, [1.0] * 8, "bf16",
                       seed + 1)


def prefill_lengths(rng, n_seq=32, total=8192, lo=64, hi=512):
    """Sequence lengths drawn uniform on [lo, hi] and then walked to the
    requested total one seeded step of +-1 at a time, staying in [lo, hi]."""
    lens = rng.integers(lo, hi + 1, size=n_seq).astype(np.int64)
    while lens.sum() != total:
        i = int(rng.integers(0, n_seq))
        step = 1 if lens.sum() < total else -1
        if lo <= lens[i] + step <= hi:
            lens[i] += step
    return lens


def config_prefill(seed=1003, n_seq=32, total=8192, K=4096, Nslice=14336, R=64, L=16):
    """Prefill: 8192 tokens in 32 sequences of length ~U[64,512], one adapter
    per sequence from 16 slots, hidden 4096, gate_up slices 2x14336, rank 64,
    bf16, A,B~N(0,0.02), scale 1."""
    rng = np.random.default_rng(seed)
    lens = prefill_lengths(rng, n_seq, total)
    seq_slot = rng.integers(0, L, size=n_seq)
    idx = np.repeat(seq_slot, lens).astype(np.int32)
    return make_linear("prefill_gate_up", total, K, [Nslice, Nslice], R, L, idx,
                       [R] * L, [1.0] * L, "bf16", seed + 1,
                       note="seq_lens=" + ",".join(map(str, lens.tolist())))


def zipf_slots(rng, T, L, s=1.1):
    p = (np.arange(1, L + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    return rng.choice(L, size=T, p=p).astype(np.int32)


def config_many(seed=1004, T=1024, L=128, K=8192, N=8192, R=128, scale_mode="one"):
    """Many-adapter decode: 1024 tokens, 128 slots with Zipf(1.1) popularity,
    true ranks uniform over {8,16,32,64,128} padded to 128, hidden 8192,
    output 8192, bf16, A,B~N(0,0.02).  scale_mode "one" gives scale 1; "alpha"
    gives 16/r per slot."""
    rng = np.random.default_rng(seed)
    idx = zipf_slots(rng, T, L)
    ranks = rng.choice(np.array([8, 16, 32, 64, 128]), size=L).astype(np.int32)
    scale = np.ones(L, np.float32) if scale_mode == "one" else (16.0 / ranks).astype(np.float32)
    return make_linear("many_adapter", T, K, [N], R, L, idx, ranks, scale, "bf16", seed + 1)


LINEAR_CONFIGS = {
    "tiny": config_tiny,
    "decode": config_decode,
    "prefill": config_prefill,
    "many": config_many,
    "logits": config_logits,
}


# ----------------------------------------------------------------------------
# fused-MoE workloads
# ----------------------------------------------------------------------------

@dataclass
class MoECase:
    name: str
    dtype: str
    T: int
    k: int                     # top_k
    E: int                     # experts
    K: int                     # d_model (w13 input, w2 output width)
    I: int                     # d_mlp (per gate/up slice; w2 input width)
    R: int
    L: int
    x: np.ndarray              # [T, K]            w13 input (hidden states)
    h: np.ndarray              # [T*k, I]          w2 input (activation output)
    A13: List[np.ndarray]      # 2 x [L, E_a, R, K]
    B13: List[np.ndarray]      # 2 x [L, E, I, R]
    A2: np.ndarray             # [L, E, R, I]
    B2: np.ndarray             # [L, E_b, K, R]
    gate_up0: np.ndarray       # [T*k, 2I]         base w13 output (pre-activation)
    out0: np.ndarray           # [T*k, K]          base w2 output (per pair)
    topk_ids: np.ndarray       # [T, k] int32
    topk_w: np.ndarray         # [T, k] float32
    idx: np.ndarray            # [T] int32
    slot_rank: np.ndarray      # [L] int32
    scale: np.ndarray          # [L] float32
    shared_outer: bool = True

    @property
    def E_a(self):
        return self.A13[0].shape[1]

    @property
    def E_b(self):
        return self.B2.shape[1]


def route_topk(rng, T, E, k):
    """Softmax of N(0,1) logits, top-k with ties to the lower expert id; the
    weights are the softmax probabilities of the chosen experts, not
    renormalised."""
    logits = rng.standard_normal(size=(T, E)).astype(np.float64)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, order, axis=1)
    return order.astype(np.int32), w.astype(np.float32)


def make_moe(name, T, k, E, K, I, R, L, dtype, seed, shared_outer=True,
             w_std=0.02, idx=None, slot_rank=None, scale=None, base_std=1.0):
    rng = np.random.default_rng(seed)
    topk_ids, topk_w = route_topk(rng, T, E, k)
    if idx is None:
        idx = rng.integers(0, L, size=T).astype(np.int32)
    if slot_rank is None:
        slot_rank = np.full(L, R, np.int32)
    if scale is None:
        scale = np.ones(L, np.float32)
    Ea = 1 if shared_outer else E
    x = _normal(rng, (T, K), 1.0, dtype)
    h = _normal(rng, (T * k, I), 1.0, dtype)
    A13 = [_normal(rng, (L, Ea, R, K), w_std, dtype) for _ in range(2)]
    B13 = [_normal(rng, (L, E, I, R), w_std, dtype) for _ in range(2)]
    A2 = _normal(rng, (L, E, R, I), w_std, dtype)
    B2 = _normal(rng, (L, Ea, K, R), w_std, dtype)
    for s, r in enumerate(slot_rank):
        for a in A13:
            a[s, :, r:, :] = 0.0
        for b in B13:
            b[s, :, :, r:] = 0.0
        A2[s, :, r:, :] = 0.0
        B2[s, :, :, r:] = 0.0
    if base_std > 0:
        gate_up0 = _normal(rng, (T * k, 2 * I), base_std, dtype)
        out0 = _normal(rng, (T * k, K), base_std, dtype)
    else:
        gate_up0 = np.zeros((T * k, 2 * I), np.float32)
        out0 = np.zeros((T * k, K), np.float32)
    return MoECase(name, dtype, T, k, E, K, I, R, L, x, h, A13, B13, A2, B2,
                   gate_up0, out0, topk_ids, topk_w, np.asarray(idx, np.int32),
                   np.asarray(slot_rank, np.int32), np.asarray(scale, np.float32),
                   shared_outer)


def config_moe(seed=1005, T=2048, k=8, E=64, K=4096, I=1536, R=16, L=8, shared_outer=True):
    """Fused-MoE LoRA: 2048 tokens, 64 experts, top-8 from softmax of N(0,1)
    logits, d_model 4096, d_mlp 1536, w13 (2x1536) and w2 rank 16, 8 adapters,
    shared-outer (w13 lora_a and w2 lora_b with expert dim 1), bf16."""
    return make_moe("moe_shared_outer", T, k, E, K, I, R, L, "bf16", seed,
                    shared_outer=shared_outer)


# ----------------------------------------------------------------------------
# integer-exact vectors: every product and partial sum is a small integer, so
# any summation order gives the same bits in fp32 and in bf16 storage.
# ----------------------------------------------------------------------------

def ternary_sparse(rng, shape, nnz_per_row):
    """Rows of {-1,0,+1} with at most nnz_per_row non-zeros (last axis): each
    row's non-zero columns are the nnz_per_row smallest of its uniform keys
    (distinct columns), each with a random sign."""
    n = shape[-1]
    nnz = min(nnz_per_row, n)
    rows = int(np.prod(shape[:-1], dtype=np.int64))
    out = np.zeros((rows, n), np.float32)
    if rows and nnz:
        keys = rng.random((rows, n), dtype=np.float32)
        cols = np.argpartition(keys, nnz - 1, axis=1)[:, :nnz] if nnz < n else \
            np.broadcast_to(np.arange(n), (rows, n))
        signs = rng.choice(np.array([-1.0, 1.0], np.float32), size=(rows, nnz))
        out[np.arange(rows)[:, None], cols] = signs
    return out.reshape(shape)


def make_integer_linear(T, K, N, R, L, seed, dtype="bf16", p_none=0.15, slot_rank=None,
                        idx=None):
    """x, A, B in {-1,0,+1} (<=32 non-zeros per A row, <=2 per B row), y0 an
    integer in [-8,8], scale 2: |partial sums| stay <= 256, exact in bf16/fp32."""
    rng = np.random.default_rng(seed)
    if idx is None:
        idx = rng.integers(0, L, size=T).astype(np.int32)
        idx[rng.random(T) < p_none] = -1
    if slot_rank is None:
        slot_rank = rng.integers(1, R + 1, size=L).astype(np.int32)
    x = rng.integers(-1, 2, size=(T, K)).astype(np.float32)
    A = [ternary_sparse(rng, (L, R, K), 32) for _ in N]
    B = [ternary_sparse(rng, (L, n, R), 2) for n in N]
    _zero_pad(A, B, slot_rank)
    y0 = rng.integers(-8, 9, size=(T, int(sum(N)))).astype(np.float32)
    return LinearCase("integer", dtype, T, K, list(N), R, L, x, A, B, y0,
                      np.asarray(idx, np.int32), np.asarray(slot_rank, np.int32),
                      np.full(L, 2.0, np.float32))
