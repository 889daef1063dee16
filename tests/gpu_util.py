"""Helpers for the GPU parity tests: move seeded inputs to the device and
measure the max-over-heads relative Frobenius error."""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def dev(x, dtype="f32"):
    """float64 numpy array holding dtype-representable values -> device tensor (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(torch_dtype(dtype)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, ref, lead=2):
    """max over the leading `lead` axes of ||x - ref||_F / ||ref||_F."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ax = tuple(range(lead, ref.ndim))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=ax))
    den = np.sqrt(np.sum(ref ** 2, axis=ax))
    return float(np.max(num / np.maximum(den, 1e-300)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
