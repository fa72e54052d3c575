"""Benchmark of the multi-LoRA delta on one MI355X.

One step = one pass of the whole hot path over one batch: segment build,
shrink and expand of every slice (lora_apply_packed with the segments
rebuilt), on synthetic seeded inputs already resident in HBM.  Steps rotate
over distinct copies of the inputs (>= 512 MB in total, twice the 256 MB
Infinity Cache) so the measured bandwidth is HBM bandwidth.  Launches are
captured in HIP graphs (torch.cuda.CUDAGraph on ROCm) so host launch cost
does not hide the GPU time.

Prints one JSON line.  `--workload` picks another configuration for
development runs; the default is the headline decode workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROT_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode", choices=["decode", "prefill", "many", "moe", "logits"])
    p.add_argument("--path", default="auto", choices=["auto", "fused", "relay", "grouped", "decode", "prefill"],
                   help="force a decode path (development runs; the headline uses auto)")
    p.add_argument("--moe-tokens", type=int, default=2048,
                   help="tokens of the fused-MoE workload (2048 by default)")
    p.add_argument("--shared-a", action="store_true",
                   help="one lora_a tensor for every slice (the shrink runs once on the tile path)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--profile", action="store_true",
                   help="few eager steps, no graphs, for rocprofv3 runs")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 256 MiB device copy (counter calibration)")
    return p.parse_args()


DEFAULTS = {"decode": (4000, 400), "prefill": (200, 20), "many": (1000, 100), "moe": (200, 20),
            "logits": (1000, 100)}


def make_case(name):
    import synth
    if name == "decode":
        return synth.config_decode()
    if name == "prefill":
        return synth.config_prefill()
    if name == "logits":
        return synth.config_logits()
    return synth.config_many()


def algorithmic_bytes(c, shared_a=False):
    """Bytes each kernel must move (per launch) for the realised draw.
    shrink: x rows of active tokens, the active slots' lora_a rows j < r, and
    the fp32 buffer of those tokens; expand: the active slots' lora_b
    columns j < r, the buffer, and the read-modify-write of the active rows of
    y; segments: idx read, perm written."""
    import numpy as np
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
    flops_shrink = 2 * c.S * rank_tok * c.K
    flops_expand = 2 * rank_tok * c.Ntot
    # the single-launch decode kernel keeps the buffer on chip
    fused = ta * c.K * el + c.S * rank_slot * c.K * el + rank_slot * c.Ntot * el + ta * c.Ntot * el * 2
    return dict(shrink=shrink, expand=expand, segments=seg, fused=fused,
                total=shrink + expand + seg,
                flops=flops_shrink + flops_expand, active_tokens=ta, active_slots=len(slots))


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


def load_traffic(workload, kernel, khash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != khash:
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def load_mfma_counters(workload, khash):
    """MFMA flops executed per step (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, summed
    over the step's kernels) from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_mfma_{workload}.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != khash:
        return None
    return d.get("step_mfma_bf16_flops")


def cpu_baseline(c, seconds):
    """The CPU oracle, single-threaded, on a bounded sample of the same
    workload: whole batches (or a token prefix of one) repeated for about
    `seconds`; tokens/s."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    n = c.T
    t0 = time.perf_counter()
    oracle.lora_apply(c.y0[:1], c.x[:1], c.A, c.B, c.idx[:1], c.slot_rank, c.scale)
    one = max(time.perf_counter() - t0, 1e-6)
    # choose a token prefix that takes about a second, then repeat it
    n = int(min(c.T, max(1, 1.0 / one)))
    done, t0 = 0, time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < seconds:
        oracle.lora_apply(c.y0[:n], c.x[:n], c.A, c.B, c.idx[:n], c.slot_rank, c.scale)
        done += n
        reps += 1
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of the {c.T} tokens of the same batch, {reps} repetitions, "
                      f"{el:.1f} s, fp32 C loops on 1 host thread"}


def moe_cpu_baseline(c, seconds):
    """The CPU oracle, single-threaded, on a token prefix of the same MoE batch
    (w13 then w2 per (token, k) pair), repeated for about `seconds`; tokens/s."""
    import oracle
    oracle.build(force=False)

    def run(n):
        pr = slice(0, n * c.k)
        oracle.moe_lora_apply(0, c.gate_up0[pr], c.x[:n], c.A13, c.B13, c.topk_ids[:n], None,
                              c.idx[:n], c.slot_rank, c.scale, c.E)
        oracle.moe_lora_apply(1, c.out0[pr], c.h[pr], [c.A2], [c.B2], c.topk_ids[:n],
                              c.topk_w[:n], c.idx[:n], c.slot_rank, c.scale, c.E)
    t0 = time.perf_counter()
    run(1)
    one = max(time.perf_counter() - t0, 1e-6)
    n = int(min(c.T, max(1, 1.0 / one)))
    done, reps, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run(n)
        done += n
        reps += 1
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of the {c.T} tokens of the same batch (w13 and w2 per pair), "
                      f"{reps} repetitions, {el:.1f} s, fp32 C loops on 1 host thread"}


def moe_algorithmic_bytes(c):
    """Bytes the fused-MoE step must move for the realised routing: w13 reads
    the x rows of tokens with an adapter, the shared lora_a of their slots, the
    lora_b of every (slot, expert) pair used, and read-modify-writes their
    gate_up rows; w2 reads the h rows, lora_a of every (slot, expert) pair
    used, the shared lora_b, and read-modify-writes the w2 output rows."""
    import numpy as np
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
          + sum(rk(s) for s in slots) * c.K * el + n_pairs * c.K * el * 2)
    flops = 2 * (2 * sum(rk(int(c.idx[t])) for t in act) * c.K
                 + sum(rk(s) for s, _ in pairs) * 2 * c.I
                 + sum(rk(s) for s, _ in pairs) * (c.I + c.K))
    return dict(w13=w13, w2=w2, total=w13 + w2, flops=flops, active_tokens=len(act),
                pairs=n_pairs, used_groups=len(used))


def run_moe(args, steps, warmup):
    """Fused-MoE LoRA step: alignment, then the w13 and w2 deltas (per pair)."""
    import numpy as np
    import torch
    import adapter_apply_amd as aa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = synth.config_moe(T=args.moe_tokens)
    bf = torch.bfloat16
    to = lambda a, d=None: (torch.from_numpy(np.ascontiguousarray(a)).to(d) if d is not None
                            else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    base = dict(x=to(c.x, bf), h=to(c.h, bf), A13=[to(a, bf) for a in c.A13],
                B13=[to(b, bf) for b in c.B13], A2=[to(c.A2, bf)], B2=[to(c.B2, bf)],
                g=to(c.gate_up0, bf), o=to(c.out0, bf), ids=to(c.topk_ids), w=to(c.topk_w),
                idx=to(c.idx), rank=to(c.slot_rank), scale=to(c.scale))
    inst_bytes = sum((t.numel() * t.element_size()) for k, v in base.items()
                     for t in (v if isinstance(v, list) else [v]))
    n_inst = max(2, math.ceil(ROT_BYTES / inst_bytes))
    insts = []
    for i in range(n_inst):
        d = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone()) for k, v in base.items()}
        d["ws"] = aa.alloc_moe_workspace(c.T, c.k, 2, c.R, c.L, c.E)
        insts.append(d)
    del base
    torch.cuda.synchronize()
    ready = aa.LORA_FLAG_SEGMENTS_READY

    def align(d):
        aa.moe_lora_align(d["ids"], d["idx"], d["rank"], c.E, c.L, c.R, 16, d["ws"])

    def w13(d):
        aa.moe_lora_apply(aa.MOE_LORA_W13, d["g"], d["x"], d["A13"], d["B13"], d["ids"], None,
                          d["idx"], d["rank"], d["scale"], c.E, d["ws"], flags=ready)

    def w2(d):
        aa.moe_lora_apply(aa.MOE_LORA_W2, d["o"], d["h"], d["A2"], d["B2"], d["ids"], d["w"],
                          d["idx"], d["rank"], d["scale"], c.E, d["ws"], flags=ready)

    # a call of at most 256 pairs (rank 16) skips the alignment (the library's rule)
    small = c.T * c.k <= 256 and c.R == 16

    def w13_small(d):
        aa.moe_lora_apply(aa.MOE_LORA_W13, d["g"], d["x"], d["A13"], d["B13"], d["ids"], None,
                          d["idx"], d["rank"], d["scale"], c.E, d["ws"])

    def w2_small(d):
        aa.moe_lora_apply(aa.MOE_LORA_W2, d["o"], d["h"], d["A2"], d["B2"], d["ids"], d["w"],
                          d["idx"], d["rank"], d["scale"], c.E, d["ws"])

    if small:
        align, w13, w2 = None, w13_small, w2_small

    def step(d):
        if align:
            align(d)
        w13(d)
        w2(d)

    if args.profile:
        for i in range(max(steps, 1)):
            step(insts[i % n_inst])
        torch.cuda.synchronize()
        if args.calib_copy:
            a_ = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            b_ = torch.empty_like(a_)
            b_.copy_(a_)
            torch.cuda.synchronize()
        print(json.dumps({"profile_run": "moe", "steps": steps, "instances": n_inst}))
        return

    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for i in range(count):
                fn(insts[i % n_inst])
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(insts[i % n_inst])
        torch.cuda.synchronize()
        return g

    g_full = capture(step, n_inst)
    reps = max(1, math.ceil(steps / n_inst))
    for _ in range(max(1, math.ceil(warmup / n_inst))):
        g_full.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g_full.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_steps = reps * n_inst
    ms_per_step = e0.elapsed_time(e1) / n_steps
    per_call = {}
    for name, fn in (("align", align), ("w13", w13), ("w2", w2)):
        if fn is None:
            continue
        g = capture(fn, n_inst)
        r = max(1, 200 // n_inst)
        g.replay()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(r):
            g.replay()
        a1.record()
        torch.cuda.synchronize()
        per_call[name] = a0.elapsed_time(a1) * 1e3 / (r * n_inst)
        del g
    ab = moe_algorithmic_bytes(c)
    dom = max(("w13", "w2"), key=lambda k: per_call[k])
    achieved = ab[dom] / (per_call[dom] * 1e-6) / 1e9
    out = {
        "metric": "LoRA-delta tokens/sec + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU",
        "value": round(c.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": f"fused-MoE LoRA: {c.T} tokens, 64 experts top-8, d_model 4096, d_mlp 1536, "
                               "rank 16, 8 adapters, shared-outer; " +
                               ("w13 + w2 per (token, k), no alignment (few pairs)" if small else
                                "align + w13 + w2 per (token, k)"),
                   "tokens": c.T, "pairs": ab["pairs"], "used_slot_expert_groups": ab["used_groups"],
                   "rotating_instances": n_inst},
        "roofline": {"bound": "hbm", "kernel": dom + " (shrink + expand launches)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes": ab[dom], "kernel_us": round(per_call[dom], 3)},
        "calls_us": {k: round(v, 3) for k, v in per_call.items()},
        "step_algorithmic_GBps": round(ab["total"] / (ms_per_step * 1e-3) / 1e9, 1),
        "cpu_baseline": None if args.no_cpu_baseline else moe_cpu_baseline(c, args.cpu_seconds),
        "wall_s": round(wall, 3),
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    steps, warmup = DEFAULTS[args.workload]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    if args.workload == "moe":
        run_moe(args, steps, warmup)
        return

    import numpy as np
    import torch
    import adapter_apply_amd as aa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = make_case(args.workload)
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    to = lambda a, d=None: (torch.from_numpy(np.ascontiguousarray(a)).to(d) if d is not None
                            else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    base = dict(x=to(c.x, dt), A=[to(a, dt) for a in c.A], B=[to(b, dt) for b in c.B],
                y=to(c.y0, dt), idx=to(c.idx), rank=to(c.slot_rank), scale=to(c.scale))
    inst_bytes = (base["x"].numel() + base["y"].numel() + sum(a.numel() for a in base["A"]) +
                  sum(b.numel() for b in base["B"])) * base["x"].element_size()
    n_inst = max(2, math.ceil(ROT_BYTES / inst_bytes))
    if args.profile:
        n_inst = min(n_inst, 4)
    insts = []
    for i in range(n_inst):
        d = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone()) for k, v in base.items()}
        if args.shared_a:
            d["A"] = [d["A"][0]] * len(d["A"])   # one tensor, one pointer for every slice
        d["ws"] = aa.alloc_workspace(c.T, c.K, c.S, c.R, c.L)
        d["buf"] = torch.zeros((c.S, c.T, c.R), dtype=torch.float32, device=dev)
        insts.append(d)
    del base
    torch.cuda.synchronize()

    step_path = {"auto": aa.LORA_PATH_AUTO, "fused": aa.LORA_PATH_FUSED, "prefill": aa.LORA_PATH_PREFILL,
                 "grouped": aa.LORA_PATH_GROUPED, "decode": aa.LORA_PATH_DECODE,
                 "relay": aa.LORA_PATH_RELAY}[args.path]

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
    grouped, prefill = taken == aa.LORA_PATH_GROUPED, taken == aa.LORA_PATH_PREFILL
    # the decode path folds the K-chunk reduction into the expand while
    # ceil(K/256) * R <= 512, else a reduce kernel runs
    fold = not prefill and math.ceil(c.K / 256) * c.R <= 512
    part = aa.LORA_FLAG_PARTIAL
    ready = aa.LORA_FLAG_SEGMENTS_READY
    # the kernel-by-kernel calls use the step's path explicitly
    kpath = (aa.LORA_PATH_GROUPED if grouped else aa.LORA_PATH_PREFILL if prefill
             else aa.LORA_PATH_DECODE if args.path == "decode" else aa.LORA_PATH_AUTO)

    def shrink_only(d):
        aa.lora_shrink(d["buf"], d["x"], d["A"], d["idx"], d["rank"], d["ws"], path=kpath,
                       flags=ready | aa.LORA_FLAG_ACTIVE_ONLY | part)

    def shrink_reduce(d):
        aa.lora_shrink(d["buf"], d["x"], d["A"], d["idx"], d["rank"], d["ws"], path=kpath,
                       flags=ready | aa.LORA_FLAG_ACTIVE_ONLY)

    # grouped path above rank 64: shrink, reduce into the buffer, expand from it
    grouped_buf = grouped and c.R > 64
    # past one-wave discovery the grouped kernels read the segment table
    grouped_tab = grouped and not (c.L <= 64 and c.T <= 1024)

    def expand_only(d):
        aa.lora_expand(d["y"], d["buf"], d["B"], d["idx"], d["rank"], d["scale"], d["ws"],
                       path=kpath, flags=ready | (part if (fold or grouped) and not grouped_buf else 0))

    def segments_only(d):
        aa.lora_build_segments(d["idx"], d["rank"], c.L, c.R, d["ws"])

    if args.profile:
        for i in range(max(steps, 1)):
            step(insts[i % n_inst])
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
        print(json.dumps({"profile_run": args.workload, "steps": steps, "instances": n_inst}))
        return

    # ---- graphs: one replay = one step on each instance, in order ----------
    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(count):          # warm the path outside capture
                fn(insts[i % n_inst])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(insts[i % n_inst])
        torch.cuda.synchronize()
        return g

    g_full = capture(step, n_inst)
    tail = steps % n_inst
    g_tail = capture(step, tail) if tail else None

    def run_steps(k):
        full, rem = divmod(k, n_inst)
        assert rem in (0, tail)
        for _ in range(full):
            g_full.replay()
        if rem:
            g_tail.replay()

    # warmup (untimed): at least `warmup` steps, in whole replays
    for _ in range(max(1, math.ceil(warmup / n_inst))):
        g_full.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(steps)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / steps

    # ---- per-kernel durations, live, with events around graphs of one kernel
    per_kernel = {}
    if fused or relay:
        # the whole step is one kernel
        kernel_calls = [("relay" if relay else "fused", step)]
    elif grouped:
        kernel_calls = [("segments", segments_only)] if grouped_tab else []
        if grouped_buf:
            kernel_calls += [("shrink+reduce", shrink_reduce), ("expand", expand_only)]
        else:
            kernel_calls += [("shrink", shrink_only), ("expand", expand_only)]
    else:
        kernel_calls = [("segments", segments_only), ("shrink", shrink_only)]
        if not fold and not prefill:
            kernel_calls.append(("shrink+reduce", shrink_reduce))
        kernel_calls.append(("expand", expand_only))
    for name, fn in kernel_calls:
        g = capture(fn, n_inst)
        reps = max(1, 2000 // n_inst)
        for _ in range(2):
            g.replay()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(reps):
            g.replay()
        a1.record()
        torch.cuda.synchronize()
        per_kernel[name] = a0.elapsed_time(a1) * 1e3 / (reps * n_inst)   # us per launch
        del g
    if "shrink+reduce" in per_kernel and "shrink" in per_kernel:
        per_kernel["reduce"] = per_kernel.pop("shrink+reduce") - per_kernel["shrink"]
    # the expand above must leave every instance's buffer state as a step does
    for i in range(n_inst):
        step(insts[i])
    torch.cuda.synchronize()

    ab = algorithmic_bytes(c, args.shared_a)
    if fused or relay:
        dom, dom_bytes = ("relay" if relay else "fused"), ab["fused"]
    else:
        dom = max((k for k in ("shrink", "shrink+reduce", "expand") if k in per_kernel),
                  key=lambda k: per_kernel[k])
        dom_bytes = ab["shrink" if dom == "shrink+reduce" else dom]
    achieved = dom_bytes / (per_kernel[dom] * 1e-6) / 1e9
    khash = kernel_hash()
    traffic = load_traffic(args.workload, dom, khash)
    mfma_exec = (load_mfma_counters(args.workload, khash)
                 if args.path == "auto" and not args.shared_a else None)
    tokens_per_s = c.T / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c, args.cpu_seconds)

    workload_desc = {
        "decode": "decode QKV: 256 tokens, hidden 4096, slices 4096/1024/1024, rank 16, 8 slots, 10% no-adapter",
        "prefill": "prefill gate_up: 8192 tokens in 32 sequences, 16 slots, hidden 4096, slices 2x14336, rank 64",
        "many": "many-adapter decode: 1024 tokens, 128 slots Zipf(1.1), ranks 8..128 padded to 128, 8192x8192",
        "logits": "lm_head LoRA at decode: 256 tokens, hidden 4096, vocab 128256, rank 16, 8 slots, 10% no-adapter",
    }[args.workload]
    out = {
        "metric": "LoRA-delta tokens/sec + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic (seeded)",
        "config": {"workload": workload_desc + (", one lora_a for every slice" if args.shared_a else ""),
                   "tokens": c.T, "hidden": c.K, "slices": c.N,
                   "rank": c.R, "slots": c.L, "rotating_instances": n_inst,
                   "active_tokens": ab["active_tokens"]},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": dom_bytes,
                     "kernel_us": round(per_kernel[dom], 3)},
        "kernels_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "step_algorithmic_GBps": round((ab["fused"] if fused or relay else
                                        ab["shrink"] + ab["expand"] if grouped else ab["total"]) /
                                       (ms_per_step * 1e-3) / 1e9, 1),
        # dense bf16 MFMA work of the step (2 * rank * (K * slices + N_total)
        # per active token) against the 2.5 PFLOP/s bf16 peak
        "mfma": {"achieved": round(ab["flops"] / (ms_per_step * 1e-3) / 1e12, 3),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(ab["flops"] / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                 # what the MFMA units executed (padding rows included), from
                 # the counters, over this run's step time; null without them
                 "executed_frac": (None if mfma_exec is None else
                                   round(mfma_exec / (ms_per_step * 1e-3) / 1e12 /
                                         MFMA_BF16_PEAK_TFLOPS, 5))},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
        "kernel_hash": khash,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
