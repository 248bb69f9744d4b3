"""Count-sketch of a whole gradient tensor, for comparing tensors too large to
store in the repository.

Every coordinate i of a tensor (its flat index in the parameter buffer) goes
to bucket h1(i) mod K with sign s(i) = +-1, and the sketch is
    S[b] = sum over i with h1(i) mod K = b of s(i) * g[i].
h1 and h2 are Carter-Wegman hashes (a * i + c) mod (2^31 - 1) with fixed odd
multipliers; every product stays below 2^62, so numpy int64 and torch int64
(CPU or GPU) give the same buckets and signs bit for bit.

The sketch is linear, so S(g) - S(o) = S(g - o). Over random hash choices
<S(x), S(y)> estimates <x, y> without bias, with a variance of about
(|x|^2 |y|^2 + <x, y>^2) / K: with K = 2048 a squared norm of a vector whose
mass is spread over many coordinates comes out within a relative standard
deviation of about sqrt(2 / K) = 3.1 %, i.e. about 1.6 % on the norm itself.
Cosine and relative L2 computed from two sketches therefore estimate the
whole-tensor values to that accuracy (tests/test_sketch.py checks it for the
fixed hashes used here). Every coordinate of the tensor contributes, which
sampled coordinates alone cannot give.
"""
from __future__ import annotations

import numpy as np

K = 2048
P31 = (1 << 31) - 1
A1, C1 = 1_103_515_245 | 1, 12_345
A2, C2 = 1_664_525 * 1021 | 1, 1_013_904_223 % P31
CHUNK = 1 << 24


def _buckets_signs_np(idx: np.ndarray):
    idx = idx.astype(np.int64)
    h1 = (A1 * idx + C1) % P31
    h2 = (A2 % P31 * idx + C2) % P31
    return (h1 % K).astype(np.int64), (1 - 2 * (h2 & 1)).astype(np.float64)


def sketch_np(values: np.ndarray, first: int) -> np.ndarray:
    """Sketch of values[j] living at flat index first + j (float64 result)."""
    values = np.asarray(values).ravel()
    out = np.zeros(K, dtype=np.float64)
    for s in range(0, values.size, CHUNK):
        v = values[s:s + CHUNK].astype(np.float64)
        b, sg = _buckets_signs_np(np.arange(first + s, first + s + v.size, dtype=np.int64))
        out += np.bincount(b, weights=sg * v, minlength=K)
    return out


def sketch_torch(values, first: int):
    """The same sketch of a torch tensor (any device), accumulated in float64."""
    import torch
    values = values.reshape(-1)
    dev = values.device
    out = torch.zeros(K, dtype=torch.float64, device=dev)
    for s in range(0, values.numel(), CHUNK):
        v = values[s:s + CHUNK].to(torch.float64)
        idx = torch.arange(first + s, first + s + v.numel(), dtype=torch.int64, device=dev)
        h1 = (A1 * idx + C1) % P31
        h2 = ((A2 % P31) * idx + C2) % P31
        out.index_add_(0, h1 % K, (1 - 2 * (h2 & 1)).to(torch.float64) * v)
    return out


def cosine_rel_l2(sg: np.ndarray, so: np.ndarray):
    """Estimated (cosine, relative L2) of g against o from their sketches."""
    sg, so = np.asarray(sg, np.float64), np.asarray(so, np.float64)
    cos = float(sg @ so / max(np.linalg.norm(sg) * np.linalg.norm(so), 1e-300))
    rl2 = float(np.linalg.norm(sg - so) / max(np.linalg.norm(so), 1e-300))
    return cos, rl2
