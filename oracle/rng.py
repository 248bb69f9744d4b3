"""The oracle's own implementation of the parameter-initialisation rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages do not say how weights are initialised; the rule used here (and,
written independently, by the library's init kernel) is:

  * every element i of the flat parameter buffer gets
        std(tensor) * N_i,   N_i ~ N(0, 1)
    with std = init_std (0.02 as the float32 the config carries, widened to
    float64), divided by sqrt(2 * depth) for the attention output
    projection Wo and the MLP output projection Wpr; padding elements are 0;
  * N_i comes from a counter-based stream: SplitMix64 (Steele, Lea and Flood,
    "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014) seeded with
    the user seed, whose outputs 2i and 2i+1 feed the Box-Muller transform
    (Box and Muller, 1958) in float64:
        u1 = ((z_{2i} >> 11) + 1) * 2^-53         in (0, 1]
        u2 =  (z_{2i+1} >> 11)     * 2^-53         in [0, 1)
        N_i = sqrt(-2 ln u1) * cos(2 pi u2)
  * the float64 value is rounded to float32 (round to nearest even), and in
    bf16 mode once more from float32 to bf16 (round to nearest even).
"""
from __future__ import annotations

import numpy as np

from .model import OracleConfig, layout, param_count

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64_stream(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of SplitMix64 begun in state ``seed``.
    Output n is the mix of seed + (n + 1) * golden-gamma (mod 2^64)."""
    with np.errstate(over="ignore"):
        n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed) + n * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _normals(seed: int, start: int, count: int) -> np.ndarray:
    z = splitmix64_stream(seed, 2 * start, 2 * count)
    u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def init_params(cfg: OracleConfig, seed: int, dtype: str, init_std: float = 0.02) -> np.ndarray:
    """The whole flat buffer under the rule above. Returns float32 values
    (dtype 'f32') or uint16 bf16 bit patterns (dtype 'bf16')."""
    n = param_count(cfg, padded=True)
    out = np.zeros(n, dtype=np.float32)
    base = float(np.float32(init_std))
    proj_scale = 1.0 / np.sqrt(2.0 * cfg.depth)
    for name, off, r, c in layout(cfg):
        std = base * (proj_scale if name.endswith(".Wo") or name.endswith(".Wpr") else 1.0)
        out[off:off + r * c] = (std * _normals(seed, off, r * c)).astype(np.float32)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        return f32_to_bf16_bits(out)
    raise ValueError(dtype)
