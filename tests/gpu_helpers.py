"""Helpers for the GPU parity tests: numpy -> device tensors, guard bands."""
import sys

import numpy as np

SENTINEL = 0x7EEEEEEE
GUARD = 64


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_logits(a, dtype, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint64:
        a = a.view(np.int64)
    return torch.from_numpy(a).to(device)


def guarded_i32(shape, device="cuda"):
    """An int32 output view followed by a guard band of sentinels; returns (view, full)."""
    import torch
    n = int(np.prod(shape))
    full = torch.full((n + GUARD,), SENTINEL, dtype=torch.int32, device=device)
    return full[:n].view(shape), full


def guard_intact(full, n):
    return bool((full[n:] == SENTINEL).all().item())


def np_i(t):
    return t.detach().cpu().numpy().astype(np.int64)
