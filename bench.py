"""Benchmark of the multi-LoRA delta on one MI355X.

One step = one pass of the whole hot path over one batch: segment build (or
the kernels' own token grouping), shrink and expand of every slice
(lora_apply_packed with the segments rebuilt; for the fused-MoE workload the
alignment and the w13 and w2 calls), on synthetic seeded inputs already
resident in HBM.  Steps rotate over distinct copies of the inputs (>= 512 MB
in total, twice the 256 MB Infinity Cache) so the measured bandwidth is HBM
bandwidth.  Launches are captured in HIP graphs (torch.cuda.CUDAGraph on ROCm)
so host launch cost does not hide the GPU time.

Prints one JSON line.  By default the line is the headline decode workload
(256 tokens, QKV) with every other configuration nested under "configs": the
tiny fp32 case, prefill gate_up, many-adapter decode, fused-MoE and the
lm_head delta, each with its own roofline, counter traffic, timed footprint
and CPU baseline.  `--workload NAME` prints one configuration alone
(development runs).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import re
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-delta tokens/sec + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROT_BYTES = 512 << 20
LINEAR = ("decode", "tiny", "prefill", "many", "logits")
NESTED = ("tiny", "prefill", "many", "moe", "logits")

DESC = {
    "decode": "decode QKV: 256 tokens, hidden 4096, slices 4096/1024/1024, rank 16, 8 slots, 10% no-adapter",
    "tiny": "tiny oracle case: 16 tokens, hidden 64, one 64-wide slice, rank 4, 3 slots, fp32",
    "prefill": "prefill gate_up: 8192 tokens in 32 sequences, 16 slots, hidden 4096, slices 2x14336, rank 64",
    "many": "many-adapter decode: 1024 tokens, 128 slots Zipf(1.1), ranks 8..128 padded to 128, 8192x8192",
    "logits": "lm_head LoRA at decode: 256 tokens, hidden 4096, vocab 128256, rank 16, 8 slots, 10% no-adapter",
}
# (timed steps, warmup steps) of a configuration timed alone, and nested
DEFAULTS = {"decode": (4000, 400), "tiny": (2000, 200), "prefill": (200, 20), "many": (1000, 100),
            "moe": (200, 20), "logits": (1000, 100)}
NESTED_STEPS = {"tiny": (2000, 200), "prefill": (200, 20), "many": (200, 20), "moe": (200, 20),
                "logits": (200, 20)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="all", choices=["all", *LINEAR, "moe"],
                   help="all: the headline decode line with every other configuration nested")
    p.add_argument("--path", default="auto", choices=["auto", "fused", "relay", "grouped", "decode", "prefill",
                                                     "token"],
                   help="force a decode path (development runs; the headline uses auto)")
    p.add_argument("--moe-reduce-k", action="store_true",
                   help="fused-MoE: the w2 delta summed over the token's k pairs into [T][d_model]")
    p.add_argument("--moe-tokens", type=int, default=2048,
                   help="tokens of the fused-MoE workload (2048 by default)")
    p.add_argument("--shared-a", action="store_true",
                   help="one lora_a tensor for every slice (the shrink runs once)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=4.0,
                   help="seconds of oracle work per CPU-baseline leg (1 thread, all cores)")
    p.add_argument("--profile", action="store_true",
                   help="few eager steps, no graphs, for rocprofv3 runs")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 256 MiB device copy (counter calibration)")
    return p.parse_args()


def make_case(name):
    import synth
    return {"decode": synth.config_decode, "tiny": synth.config_tiny,
            "prefill": synth.config_prefill, "many": synth.config_many,
            "logits": synth.config_logits}[name]()


# ---------------------------------------------------------------------------
# algorithmic bytes and flops of the realised draws
# ---------------------------------------------------------------------------

def algorithmic_bytes(c, shared_a=False):
    """Bytes each kernel must move (per launch) for the realised draw.
    shrink: x rows of active tokens, the active slots' lora_a rows j < r, and
    the fp32 buffer of those tokens; expand: the active slots' lora_b
    columns j < r, the buffer, and the read-modify-write of the active rows of
    y; segments: idx read, perm written.  The single-launch decode kernels
    keep the buffer on chip ("fused")."""
    el = 2 if c.dtype == "bf16" else 4
    act = [(t, int(s)) for t, s in enumerate(c.idx) if 0 <= s < c.L and c.slot_rank[s] > 0]
    slots = sorted({s for _, s in act})
    ta = len(act)
    rank_tok = sum(int(c.slot_rank[s]) for _, s in act)
    rank_slot = sum(int(c.slot_rank[s]) for s in slots)
    sa = 1 if shared_a else c.S          # one lora_a (and one buffer) for every slice
    shrink = ta * c.K * el + sa * rank_slot * c.K * el + sa * rank_tok * 4
    expand = rank_slot * c.Ntot * el + c.S * rank_tok * 4 + ta * c.Ntot * el * 2
    seg = c.T * 4 * 2
    flops = 2 * sa * rank_tok * c.K + 2 * rank_tok * c.Ntot
    fused = ta * c.K * el + sa * rank_slot * c.K * el + rank_slot * c.Ntot * el + ta * c.Ntot * el * 2
    return dict(shrink=shrink, expand=expand, segments=seg, fused=fused,
                total=shrink + expand + seg, flops=flops, active_tokens=ta,
                active_slots=len(slots))


def moe_algorithmic_bytes(c, reduce_k=False):
    """Bytes the fused-MoE step must move for the realised routing: w13 reads
    the x rows of tokens with an adapter, the shared lora_a of their slots, the
    lora_b of every (slot, expert) pair used, and read-modify-writes their
    gate_up rows; w2 reads the h rows, lora_a of every (slot, expert) pair
    used, the shared lora_b, and read-modify-writes the w2 output rows (one
    per pair, or one per token when the delta is summed over the k pairs)."""
    el = 2
    act = [t for t in range(c.T) if 0 <= c.idx[t] < c.L and c.slot_rank[c.idx[t]] > 0]
    slots = sorted({int(c.idx[t]) for t in act})
    pairs = [(int(c.idx[t]), int(e)) for t in act for e in c.topk_ids[t]]
    used = sorted(set(pairs))
    rk = lambda s: int(c.slot_rank[s])
    n_pairs = len(pairs)
    w13 = (len(act) * c.K * el + 2 * sum(rk(s) for s in slots) * c.K * el
           + 2 * sum(rk(s) for s, _ in used) * c.I * el + n_pairs * 2 * c.I * el * 2)
    w2 = (n_pairs * c.I * el + sum(rk(s) for s, _ in used) * c.I * el
          + sum(rk(s) for s in slots) * c.K * el
          + (len(act) if reduce_k else n_pairs) * c.K * el * 2)
    flops = 2 * (2 * sum(rk(int(c.idx[t])) for t in act) * c.K
                 + sum(rk(s) for s, _ in pairs) * 2 * c.I
                 + sum(rk(s) for s, _ in pairs) * (c.I + c.K))
    return dict(w13=w13, w2=w2, total=w13 + w2, flops=flops, active_tokens=len(act),
                pairs=n_pairs, used_groups=len(used))


# ---------------------------------------------------------------------------
# committed counter summaries (valid only for the kernel sources they were
# taken on)
# ---------------------------------------------------------------------------

def kernel_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "adapter_apply_amd", "csrc"))):
        with open(os.path.join(ROOT, "adapter_apply_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _code_only(src):
    """Source text without comments and with whitespace runs collapsed: edits
    to comments leave the kernels, and so the counters taken on them, valid."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def _load_json(name, khash):
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d if d.get("kernel_hash") == khash else None


def load_traffic(workload, kernel, khash):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed rocprofv3 counter summary of this workload."""
    d = _load_json(f"pmc_{workload}.json", khash)
    k = None if d is None else d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def load_mfma_counters(workload, khash):
    """MFMA flops executed per step (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, summed
    over the step's kernels) from the committed rocprofv3 counter summary."""
    d = _load_json(f"pmc_mfma_{workload}.json", khash)
    return None if d is None else d.get("step_mfma_bf16_flops")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on 1 host thread and on all cores
# ---------------------------------------------------------------------------

def host_threads():
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def oracle_rates(run, T, seconds, what):
    """run(lo, hi) computes the oracle's delta for tokens [lo, hi) of the
    batch (each token depends on its own row only).  Times it for about
    `seconds` on 1 host thread and then on every host core (one token block
    per thread, repeated; ctypes releases the GIL around the oracle's C
    calls).  Returns the cpu_baseline object (all cores) with the 1-thread
    figure nested."""
    t0 = time.perf_counter()
    run(0, 1)
    one = max(time.perf_counter() - t0, 1e-6)
    blk = int(min(T, max(1, 0.5 / one)))          # about half a second per call

    def timed(nthreads):
        stop = time.perf_counter() + seconds
        done = [0] * nthreads
        lock = threading.Lock()

        def worker(i):
            lo = (i * blk) % T
            hi = min(T, lo + blk)
            n = 0
            while time.perf_counter() < stop:
                run(lo, hi)
                n += hi - lo
            with lock:
                done[i] = n
        t = time.perf_counter()
        with cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(worker, range(nthreads)))
        return sum(done) / (time.perf_counter() - t)

    single = timed(1)
    n = host_threads()
    multi = timed(n)
    sample = (f"{what}: token blocks of {blk} of the batch's {T} tokens, repeated for "
              f"about {seconds:.1f} s per leg; fp32 C loops (the oracle, unchanged)")
    return {"value": round(multi, 1), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": sample + f", one block per thread on {n} host threads",
            "single_thread": {"value": round(single, 1), "unit": "tokens/s", "cores": 1}}


def linear_cpu_baseline(c, seconds):
    import oracle
    oracle.build(force=False)
    return oracle_rates(lambda lo, hi: oracle.lora_apply(c.y0[lo:hi], c.x[lo:hi], c.A, c.B,
                                                         c.idx[lo:hi], c.slot_rank, c.scale),
                        c.T, seconds, "the same batch")


def moe_cpu_baseline(c, seconds, reduce_k=False):
    import oracle
    oracle.build(force=False)
    out_red = moe_reduced_out(c) if reduce_k else None

    def run(lo, hi):
        pr = slice(lo * c.k, hi * c.k)
        oracle.moe_lora_apply(0, c.gate_up0[pr], c.x[lo:hi], c.A13, c.B13, c.topk_ids[lo:hi],
                              None, c.idx[lo:hi], c.slot_rank, c.scale, c.E)
        oracle.moe_lora_apply(1, out_red[lo:hi] if reduce_k else c.out0[pr], c.h[pr], [c.A2], [c.B2],
                              c.topk_ids[lo:hi], c.topk_w[lo:hi], c.idx[lo:hi], c.slot_rank, c.scale,
                              c.E, reduce_k=reduce_k)
    return oracle_rates(run, c.T, seconds, "the same batch, w13 per (token, k) pair and w2 " +
                        ("summed over each token's pairs" if reduce_k else "per (token, k) pair"))


def moe_reduced_out(c):
    """The w2 output for the k-reduced form, [T][d_model]: the first pair row
    of each token of the seeded per-pair output."""
    return c.out0.reshape(c.T, c.k, -1)[:, 0, :].copy()


# ---------------------------------------------------------------------------
# GPU timing helpers
# ---------------------------------------------------------------------------

def measure_copy_gbps(torch, dev, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate of a plain 1 GiB copy (read + write bytes
    over time): the practical HBM ceiling beside the 8 TB/s nominal."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbps


def measure_gemm_tflops(torch, dev, n=8192, reps=10):
    """Rate of a large dense bf16 matrix product through torch (hipBLASLt):
    the practical MFMA ceiling of this machine beside the 2.5 PFLOP/s nominal
    (the copy rate above plays the same part for HBM)."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return tflops


# measured once per run by main(); reported in every entry's "mfma"
GEMM_TFLOPS = [None]


def _gemm_fields(achieved):
    g = GEMM_TFLOPS[0]
    return {} if g is None else {"gemm_TFLOPs": round(g, 1), "frac_of_gemm": round(achieved / g, 5)}


class Rotation:
    """Graph capture and timing over n_inst distinct instances."""

    def __init__(self, torch, insts):
        self.torch = torch
        self.insts = insts
        self.n = len(insts)

    def capture(self, fn, count):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(count):          # warm the path outside capture
                fn(self.insts[i % self.n])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(self.insts[i % self.n])
        torch.cuda.synchronize()
        return g

    def time_steps(self, step, steps, warmup):
        """K timed steps (whole rotations, then a tail of the first instances)
        after at least `warmup` untimed ones; returns (ms per step, wall s)."""
        torch = self.torch
        g_full = self.capture(step, self.n)
        tail = steps % self.n
        g_tail = self.capture(step, tail) if tail else None
        for _ in range(max(1, math.ceil(warmup / self.n))):
            g_full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps // self.n):
            g_full.replay()
        if tail:
            g_tail.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    def median_us(self, fn, min_launches=2000, reps=None):
        """Per-launch time of fn: a graph of one launch per instance, replayed
        `reps` times, each replay between its own events on the stream the
        kernels run on; the median replay over n_inst launches."""
        torch = self.torch
        g = self.capture(fn, self.n)
        reps = reps or max(20, min(400, math.ceil(min_launches / self.n)))
        for _ in range(2):
            g.replay()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        del g
        return statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3 / self.n


def n_instances(inst_bytes, profile=False):
    n = max(2, math.ceil(ROT_BYTES / inst_bytes))
    return min(n, 4) if profile else n


# ---------------------------------------------------------------------------
# linear (packed-slice) workloads
# ---------------------------------------------------------------------------

def linear_entry(name, args, steps, warmup, cpu_seconds, copy_gbps):
    import numpy as np
    import torch
    import adapter_apply_amd as aa

    dev = torch.device("cuda:0")
    c = make_case(name)
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    to = lambda a, d=None: (torch.from_numpy(np.ascontiguousarray(a)).to(d) if d is not None
                            else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    base = dict(x=to(c.x, dt), A=[to(a, dt) for a in c.A], B=[to(b, dt) for b in c.B],
                y=to(c.y0, dt), idx=to(c.idx), rank=to(c.slot_rank), scale=to(c.scale))
    inst_bytes = (base["x"].numel() + base["y"].numel() + sum(a.numel() for a in base["A"]) +
                  sum(b.numel() for b in base["B"])) * base["x"].element_size()
    n_inst = n_instances(inst_bytes, args.profile)
    insts = []
    for _ in range(n_inst):
        d = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone()) for k, v in base.items()}
        if args.shared_a:
            d["A"] = [d["A"][0]] * len(d["A"])   # one tensor, one pointer for every slice
        d["ws"] = aa.alloc_workspace(c.T, c.K, c.S, c.R, c.L)
        d["buf"] = torch.zeros((c.S, c.T, c.R), dtype=torch.float32, device=dev)
        insts.append(d)
    del base
    torch.cuda.synchronize()

    step_path = {"auto": aa.LORA_PATH_AUTO, "fused": aa.LORA_PATH_FUSED,
                 "prefill": aa.LORA_PATH_PREFILL, "grouped": aa.LORA_PATH_GROUPED,
                 "decode": aa.LORA_PATH_DECODE, "relay": aa.LORA_PATH_RELAY,
                 "token": aa.LORA_PATH_TOKEN}[args.path]

    def step(d):
        aa.lora_apply_packed(d["y"], d["x"], d["A"], d["B"], d["idx"], d["rank"], d["scale"],
                             d["ws"], path=step_path)

    # The path the step takes, as the library reports it (lora_plan_packed runs
    # the same checks and choice as lora_apply_packed); the kernel-by-kernel
    # calls below launch exactly that path's kernels.
    d0 = insts[0]
    taken = aa.lora_plan_packed(d0["y"], d0["x"], d0["A"], d0["B"], d0["idx"], d0["rank"],
                                d0["scale"], d0["ws"], path=step_path)
    relay, fused = taken == aa.LORA_PATH_RELAY, taken == aa.LORA_PATH_FUSED
    # the paths that are one kernel for the whole step
    single = {aa.LORA_PATH_RELAY: "relay", aa.LORA_PATH_FUSED: "fused",
              aa.LORA_PATH_TOKEN: "token"}.get(taken)
    grouped, prefill = taken == aa.LORA_PATH_GROUPED, taken == aa.LORA_PATH_PREFILL
    # the decode path folds the K-chunk reduction into the expand while
    # ceil(K/256) * R <= 512, else a reduce kernel runs
    fold = not prefill and math.ceil(c.K / 256) * c.R <= 512
    part, ready = aa.LORA_FLAG_PARTIAL, aa.LORA_FLAG_SEGMENTS_READY
    kpath = (aa.LORA_PATH_GROUPED if grouped else aa.LORA_PATH_PREFILL if prefill
             else aa.LORA_PATH_DECODE)
    # grouped path above rank 64: shrink, reduce into the buffer, expand from it
    grouped_buf = grouped and c.R > 64
    # past one-wave discovery the grouped kernels read the segment table
    grouped_tab = grouped and not (c.L <= 64 and c.T <= 1024)

    def shrink_only(d):
        aa.lora_shrink(d["buf"], d["x"], d["A"], d["idx"], d["rank"], d["ws"], path=kpath,
                       flags=ready | aa.LORA_FLAG_ACTIVE_ONLY | part)

    def shrink_reduce(d):
        aa.lora_shrink(d["buf"], d["x"], d["A"], d["idx"], d["rank"], d["ws"], path=kpath,
                       flags=ready | aa.LORA_FLAG_ACTIVE_ONLY)

    def expand_only(d):
        aa.lora_expand(d["y"], d["buf"], d["B"], d["idx"], d["rank"], d["scale"], d["ws"],
                       path=kpath, flags=ready | (part if (fold or grouped) and not grouped_buf else 0))

    def segments_only(d):
        aa.lora_build_segments(d["idx"], d["rank"], c.L, c.R, d["ws"])

    if args.profile:
        for i in range(max(steps, 1)):
            step(insts[i % n_inst])
        if not single:
            for fn in ((segments_only, shrink_reduce, expand_only) if grouped_buf else
                       (segments_only, shrink_reduce, shrink_only, expand_only)):
                for i in range(n_inst):
                    fn(insts[i])
        torch.cuda.synchronize()
        if args.calib_copy:
            a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
        return {"profile_run": name, "steps": steps, "instances": n_inst,
                "path": aa.PATH_NAMES[taken]}

    rot = Rotation(torch, insts)
    ms_per_step, wall = rot.time_steps(step, steps, warmup)

    # ---- per-kernel durations, live: median over replays of one-kernel graphs
    if single:
        kernel_calls = [(single, step)]   # the whole step is one kernel
    elif grouped:
        kernel_calls = [("segments", segments_only)] if grouped_tab else []
        kernel_calls += ([("shrink+reduce", shrink_reduce), ("expand", expand_only)] if grouped_buf
                         else [("shrink", shrink_only), ("expand", expand_only)])
    else:
        kernel_calls = [("segments", segments_only), ("shrink", shrink_only)]
        if not fold and not prefill:
            kernel_calls.append(("shrink+reduce", shrink_reduce))
        kernel_calls.append(("expand", expand_only))
    per_kernel = {k: rot.median_us(fn) for k, fn in kernel_calls}
    if "shrink+reduce" in per_kernel and "shrink" in per_kernel:
        per_kernel["reduce"] = per_kernel.pop("shrink+reduce") - per_kernel["shrink"]
    # the expand calls above must leave every instance's buffers as a step does
    for d in insts:
        step(d)
    torch.cuda.synchronize()

    ab = algorithmic_bytes(c, args.shared_a)
    if single:
        dom, dom_bytes = single, ab["fused"]
    else:
        dom = max((k for k in ("shrink", "shrink+reduce", "expand") if k in per_kernel),
                  key=lambda k: per_kernel[k])
        dom_bytes = ab["shrink" if dom == "shrink+reduce" else dom]
    achieved = dom_bytes / (per_kernel[dom] * 1e-6) / 1e9
    khash = kernel_hash()
    counted = args.path == "auto" and not args.shared_a
    traffic = load_traffic(name, dom, khash) if counted else None
    mfma_exec = load_mfma_counters(name, khash) if counted else None
    step_bytes = (ab["fused"] if single else
                  ab["shrink"] + ab["expand"] if grouped else ab["total"])
    entry = {
        "workload": DESC[name] + (", one lora_a for every slice" if args.shared_a else ""),
        "path": aa.PATH_NAMES[taken],
        "value": round(c.T / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": ms_per_step, "steps": steps, "warmup": warmup, "dtype": c.dtype,
        "tokens": c.T, "hidden": c.K, "slices": c.N, "rank": c.R, "slots": c.L,
        "active_tokens": ab["active_tokens"],
        "rotating_instances": n_inst,
        "rotation_MB": round(n_inst * inst_bytes / 1e6, 1),
        # bytes of the instances the timed steps touch (the untimed warmup
        # replays every instance first, so the timed ones are not cache-resident)
        "timed_footprint_MB": round(min(steps, n_inst) * inst_bytes / 1e6, 1),
        "kernels_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "roofline": {"bound": "launch" if name == "tiny" else "hbm", "kernel": dom,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": dom_bytes, "kernel_us": round(per_kernel[dom], 3),
                     "copy_GBps": round(copy_gbps, 1),
                     "frac_of_copy": round(achieved / copy_gbps, 4)},
        "step_algorithmic_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        # dense MFMA work of the step (2 * rank * (K * slices + N_total) per
        # active token) against the 2.5 PFLOP/s bf16 peak; executed_frac is
        # what the matrix cores ran (padding included) from the counters
        "mfma": {"achieved": round(ab["flops"] / (ms_per_step * 1e-3) / 1e12, 3),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(ab["flops"] / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                 **_gemm_fields(ab["flops"] / (ms_per_step * 1e-3) / 1e12),
                 "executed_frac": (None if mfma_exec is None else
                                   round(mfma_exec / (ms_per_step * 1e-3) / 1e12 /
                                         MFMA_BF16_PEAK_TFLOPS, 5))},
        "cpu_baseline": None if args.no_cpu_baseline else linear_cpu_baseline(c, cpu_seconds),
        "wall_s": round(wall, 3),
    }
    del insts, rot
    torch.cuda.empty_cache()
    return entry


# ---------------------------------------------------------------------------
# fused-MoE workload
# ---------------------------------------------------------------------------

def moe_entry(args, steps, warmup, cpu_seconds, copy_gbps):
    """Fused-MoE LoRA step: alignment, then the w13 and w2 deltas (per pair)."""
    import numpy as np
    import torch
    import adapter_apply_amd as aa
    import synth
    dev = torch.device("cuda:0")
    c = synth.config_moe(T=args.moe_tokens)
    red = getattr(args, "moe_reduce_k", False)   # w2 delta summed over each token's pairs
    bf = torch.bfloat16
    to = lambda a, d=None: (torch.from_numpy(np.ascontiguousarray(a)).to(d) if d is not None
                            else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    base = dict(x=to(c.x, bf), h=to(c.h, bf), A13=[to(a, bf) for a in c.A13],
                B13=[to(b, bf) for b in c.B13], A2=[to(c.A2, bf)], B2=[to(c.B2, bf)],
                g=to(c.gate_up0, bf), o=to(moe_reduced_out(c) if red else c.out0, bf),
                ids=to(c.topk_ids), w=to(c.topk_w),
                idx=to(c.idx), rank=to(c.slot_rank), scale=to(c.scale))
    inst_bytes = sum((t.numel() * t.element_size()) for k, v in base.items()
                     for t in (v if isinstance(v, list) else [v]))
    n_inst = n_instances(inst_bytes, args.profile)
    insts = []
    for _ in range(n_inst):
        d = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone()) for k, v in base.items()}
        d["ws"] = aa.alloc_moe_workspace(c.T, c.k, 2, c.R, c.L, c.E)
        insts.append(d)
    del base
    torch.cuda.synchronize()
    ready = aa.LORA_FLAG_SEGMENTS_READY
    # whether the calls of this size skip the alignment (the library's own rule)
    small = aa.moe_lora_plan(c.T, c.k, c.R) and aa.moe_lora_plan(c.T, c.k, c.R, red)

    def align(d):
        aa.moe_lora_align(d["ids"], d["idx"], d["rank"], c.E, c.L, c.R, 16, d["ws"])

    def w13(d):
        aa.moe_lora_apply(aa.MOE_LORA_W13, d["g"], d["x"], d["A13"], d["B13"], d["ids"], None,
                          d["idx"], d["rank"], d["scale"], c.E, d["ws"], flags=0 if small else ready)

    def w2(d):
        aa.moe_lora_apply(aa.MOE_LORA_W2, d["o"], d["h"], d["A2"], d["B2"], d["ids"], d["w"],
                          d["idx"], d["rank"], d["scale"], c.E, d["ws"], reduce_k=red,
                          flags=0 if small else ready)

    calls = (("w13", w13), ("w2", w2)) if small else (("align", align), ("w13", w13), ("w2", w2))

    def step(d):
        for _, fn in calls:
            fn(d)

    if args.profile:
        for i in range(max(steps, 1)):
            step(insts[i % n_inst])
        torch.cuda.synchronize()
        if args.calib_copy:
            a_ = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            b_ = torch.empty_like(a_)
            b_.copy_(a_)
            torch.cuda.synchronize()
        return {"profile_run": "moe", "steps": steps, "instances": n_inst}

    rot = Rotation(torch, insts)
    ms_per_step, wall = rot.time_steps(step, steps, warmup)
    per_call = {k: rot.median_us(fn, min_launches=200) for k, fn in calls}
    ab = moe_algorithmic_bytes(c, red)
    dom = max(("w13", "w2"), key=lambda k: per_call[k])
    achieved = ab[dom] / (per_call[dom] * 1e-6) / 1e9
    khash = kernel_hash()
    entry = {
        "workload": (f"fused-MoE LoRA: {c.T} tokens, 64 experts top-8, d_model 4096, d_mlp 1536, "
                     "rank 16, 8 adapters, shared-outer; " +
                     ("w13 + w2 per (token, k), no alignment (few pairs)" if small else
                      "align + w13 per (token, k) + w2 summed over each token's k pairs" if red else
                      "align + w13 + w2 per (token, k)")),
        "value": round(c.T / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": ms_per_step, "steps": steps, "warmup": warmup, "dtype": "bf16",
        "tokens": c.T, "pairs": ab["pairs"], "used_slot_expert_groups": ab["used_groups"],
        "rotating_instances": n_inst,
        "rotation_MB": round(n_inst * inst_bytes / 1e6, 1),
        "timed_footprint_MB": round(min(steps, n_inst) * inst_bytes / 1e6, 1),
        "calls_us": {k: round(v, 3) for k, v in per_call.items()},
        "roofline": {"bound": "hbm", "kernel": dom + " (shrink + expand launches)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if red else load_traffic("moe", dom, khash),
                     "algorithmic_bytes": ab[dom], "kernel_us": round(per_call[dom], 3),
                     "copy_GBps": round(copy_gbps, 1),
                     "frac_of_copy": round(achieved / copy_gbps, 4)},
        "step_algorithmic_GBps": round(ab["total"] / (ms_per_step * 1e-3) / 1e9, 1),
        "mfma": {"achieved": round(ab["flops"] / (ms_per_step * 1e-3) / 1e12, 3),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(ab["flops"] / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                 **_gemm_fields(ab["flops"] / (ms_per_step * 1e-3) / 1e12)},
        "cpu_baseline": None if args.no_cpu_baseline else moe_cpu_baseline(c, cpu_seconds, red),
        "wall_s": round(wall, 3),
    }
    del insts, rot
    torch.cuda.empty_cache()
    return entry


# ---------------------------------------------------------------------------

def headline_line(entry, name, steps, warmup, copy_gbps, khash):
    """The contract's JSON line around one configuration's entry."""
    e = dict(entry)
    cfg = {"workload": e.pop("workload")}
    for k in ("tokens", "hidden", "slices", "rank", "slots", "active_tokens", "pairs",
              "used_slot_expert_groups", "rotating_instances", "rotation_MB",
              "timed_footprint_MB", "path"):
        if k in e:
            cfg[k] = e.pop(k)
    out = {"metric": METRIC, "value": e.pop("value"), "unit": e.pop("unit"), "n_gpus": 1,
           "steps": steps, "warmup": warmup, "ms_per_step": e.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": e.pop("dtype"), "data": "synthetic (seeded)", "config": cfg}
    e.pop("steps", None)
    e.pop("warmup", None)
    out.update(e)
    out["copy_GBps"] = round(copy_gbps, 1)
    if GEMM_TFLOPS[0] is not None:
        out["gemm_TFLOPs"] = round(GEMM_TFLOPS[0], 1)
    out["kernel_hash"] = khash
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    name = "decode" if args.workload == "all" else args.workload
    steps, warmup = DEFAULTS[name]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    if args.profile:
        run = moe_entry if name == "moe" else (lambda *a: linear_entry(name, *a))
        print(json.dumps(run(args, steps, warmup, 0.0, 1.0)))
        return
    t0 = time.perf_counter()
    copy_gbps = measure_copy_gbps(torch, torch.device("cuda:0"))
    GEMM_TFLOPS[0] = measure_gemm_tflops(torch, torch.device("cuda:0"))
    khash = kernel_hash()
    if name == "moe":
        entry = moe_entry(args, steps, warmup, args.cpu_seconds, copy_gbps)
    else:
        entry = linear_entry(name, args, steps, warmup, args.cpu_seconds, copy_gbps)
    out = headline_line(entry, name, steps, warmup, copy_gbps, khash)
    if args.workload == "all":
        # every other configuration, each timed on its own rotation
        nested = {}
        for other in NESTED:
            s, w = NESTED_STEPS[other]
            secs = min(args.cpu_seconds, 3.0)
            nested[other] = (moe_entry(args, s, w, secs, copy_gbps) if other == "moe" else
                             linear_entry(other, args, s, w, secs, copy_gbps))
        out["configs"] = nested
    out["bench_wall_s"] = round(time.perf_counter() - t0, 1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
