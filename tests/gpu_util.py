"""Helpers of the GPU tests: move seeded workloads to the device, read results
back, and guard output buffers with canary bands."""
import sys

import numpy as np
import torch

import adapter_apply_amd as aa

CANARY = 4096   # elements of guard band on each side of an output


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tdt(case_dtype):
    return torch.bfloat16 if case_dtype == "bf16" else torch.float32


def dev(a, dtype=None, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def host_f32(t):
    return t.detach().float().cpu().numpy()


def guarded(arr_f32, dtype, fill=7.0):
    """Device copy of a 2-D array inside a flat allocation with canary bands;
    returns (full, view)."""
    rows, cols = arr_f32.shape
    full = torch.full((rows * cols + 2 * CANARY,), fill, dtype=dtype, device="cuda")
    view = full[CANARY:CANARY + rows * cols].view(rows, cols)
    view.copy_(dev(arr_f32, dtype))
    return full, view


def canaries_intact(full, fill=7.0):
    head = full[:CANARY].float()
    tail = full[-CANARY:].float()
    return bool(torch.all(head == fill)) and bool(torch.all(tail == fill))


class LinearOnDevice:
    """A LinearCase's tensors on the GPU."""

    def __init__(self, c, guard=True):
        self.c = c
        dt = tdt(c.dtype)
        self.dt = dt
        self.x = dev(c.x, dt)
        self.A = [dev(a, dt) for a in c.A]
        self.B = [dev(b, dt) for b in c.B]
        self.idx = dev(c.idx)
        self.rank = dev(c.slot_rank)
        self.scale = dev(c.scale)
        if guard:
            self.yfull, self.y = guarded(c.y0, dt)
        else:
            self.yfull, self.y = None, dev(c.y0, dt)
        self.ws = aa.alloc_workspace(c.T, c.K, c.S, c.R, c.L)

    def apply(self, path=aa.LORA_PATH_AUTO, flags=0):
        aa.lora_apply_packed(self.y, self.x, self.A, self.B, self.idx, self.rank, self.scale,
                             self.ws, path=path, flags=flags)

    def y_host(self):
        torch.cuda.synchronize()
        return host_f32(self.y)

    def reset_y(self):
        self.y.copy_(dev(self.c.y0, self.dt))
