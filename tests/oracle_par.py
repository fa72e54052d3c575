"""The CPU oracle run over token blocks in host threads.

A token's delta depends on its own x row, its slot and the slot's weights
only (the per-token definition on the [vLLM] "vllm.lora.layers" page,
RowParallelLinearWithShardedLoRA.apply; the (token, k) pairs of a token in
FusedMoEWithLoRA), so the oracle called on disjoint token blocks gives, block
for block, the rows it gives on the whole batch.  ctypes releases the GIL
around the oracle's C calls, so the blocks run on several host cores.  A CPU
test checks the block-wise result against the whole-batch call bit for bit.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np


def host_threads() -> int:
    """Threads to use: the cores this process may run on, capped by
    OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _blocks(T, n_blocks):
    edges = np.linspace(0, T, n_blocks + 1).astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def lora_apply(oracle_mod, y0, x, A, B, idx, slot_rank, scale, threads=None, rows=None):
    """oracle.lora_apply's y over all tokens (or over the token ids `rows`),
    computed in token blocks on `threads` host threads."""
    threads = threads or host_threads()
    if rows is not None:
        rows = np.asarray(rows)
        y0, x, idx = y0[rows], x[rows], np.asarray(idx)[rows]
    T = x.shape[0]
    out = np.empty(y0.shape, np.float32)

    def run(b):
        lo, hi = b
        y, _ = oracle_mod.lora_apply(y0[lo:hi], x[lo:hi], A, B, idx[lo:hi], slot_rank, scale)
        out[lo:hi] = y

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, _blocks(T, 4 * threads)))
    return out


def moe_lora_apply(oracle_mod, kind, y0, x, A, B, topk_ids, topk_w, idx, slot_rank, scale, E,
                   reduce_k=False, threads=None):
    """oracle.moe_lora_apply over all tokens in token blocks.  y0 and x are
    per pair ([T*k, ...]) or per token ([T, ...]) as the oracle takes them."""
    threads = threads or host_threads()
    T, k = topk_ids.shape
    out = np.empty(y0.shape, np.float32)
    x_per_pair = kind == 1
    y_per_pair = not (kind == 1 and reduce_k)

    def run(b):
        lo, hi = b
        xs = x[lo * k:hi * k] if x_per_pair else x[lo:hi]
        ys = y0[lo * k:hi * k] if y_per_pair else y0[lo:hi]
        w = None if topk_w is None else topk_w[lo:hi]
        r = oracle_mod.moe_lora_apply(kind, ys, xs, A, B, topk_ids[lo:hi], w, idx[lo:hi],
                                      slot_rank, scale, E, reduce_k=reduce_k)
        if y_per_pair:
            out[lo * k:hi * k] = r
        else:
            out[lo:hi] = r

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, _blocks(T, 4 * threads)))
    return out
