"""Shared test helpers: device upload and the relative-L2 parity metric."""
import numpy as np
import torch

TOL = {"fp32": 1e-5, "bf16": 1e-2}   # relative L2 bound per output tensor


def dev(x, dtype):
    """numpy float32 array -> device tensor of `dtype` (exact for bf16-representable values)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32
