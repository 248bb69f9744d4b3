"""Helpers for the GPU tests: device tensors from numpy, comparison metrics.
The metrics follow the parity bar: fp32 mode compares loss relative error and
per-tensor max relative error (max |g - o| / max |o|); bf16 mode compares loss
relative error, per-tensor cosine and relative L2 error."""
from __future__ import annotations

import numpy as np


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(a64):
    """float64 numpy -> bf16 device tensor (round to nearest even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).to(torch.bfloat16).cuda()


def host64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def max_rel(g, o):
    g, o = np.asarray(g, np.float64).ravel(), np.asarray(o, np.float64).ravel()
    return float(np.abs(g - o).max() / max(np.abs(o).max(), 1e-300))


def cosine(g, o):
    g, o = np.asarray(g, np.float64).ravel(), np.asarray(o, np.float64).ravel()
    return float(g @ o / max(np.linalg.norm(g) * np.linalg.norm(o), 1e-300))


def rel_l2(g, o):
    g, o = np.asarray(g, np.float64).ravel(), np.asarray(o, np.float64).ravel()
    return float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))


def check_bf16(g, o, name, cos_min=0.999, l2_max=3e-2):
    c, r = cosine(g, o), rel_l2(g, o)
    assert c >= cos_min and r <= l2_max, f"{name}: cosine {c:.6f}, rel L2 {r:.3e}"
    return c, r
