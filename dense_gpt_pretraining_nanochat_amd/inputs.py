"""Seeded synthetic inputs shared by the tests, the oracle timing and the bench.

This module holds none of the model's arithmetic: it only draws numbers.
The pages train on FineWeb-EDU text through a 65,536-id BPE tokenizer (the
wmrh.cn tutorial, section 2.1; the hsin-life.com post "你不知道的nanochat",
section "先進的Rust BPE tokenizer架構"); neither is available offline, so
seeded tokens with the same shape and id range stand in:

  * uniform ids in [0, V) for the tiny fp32 config;
  * Zipf(s = 1.1) ids otherwise: P(id = k - 1) proportional to k^-1.1 for
    k = 1..V (id 0 is the most frequent), drawn by inverse-CDF sampling.

Each row is one sequence of T + 1 draws; tokens are its first T entries and
targets its last T (next-token targets).

Token byte lengths (the tokenizer's table, for bits-per-byte evaluation) are
synthetic too: ids 0..255 one byte each (the byte-level base of a BPE
vocabulary), the last 8 ids zero (special tokens), the rest 1 + a geometric
draw (at least 1, mean 3.8), so that a typical token spans about 4.8 bytes, the
compression the tutorial quotes for the pages' tokenizer (section 2.1).

Parameters for parity runs are N(0, std^2) per tensor, drawn with numpy's
``default_rng(seed)`` in float64 and rounded to float32, then to bf16 in bf16
mode. (The library's own initialiser uses a different, counter-based
generator; it is tested on its own.)
"""
from __future__ import annotations

import numpy as np


def zipf_ids(rng: np.random.Generator, vocab: int, n: int, s: float = 1.1) -> np.ndarray:
    k = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(k ** -s)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def make_tokens(vocab: int, seq_len: int, batch: int, seed: int, law: str = "zipf"):
    """Returns (tokens, targets), int32 [batch, seq_len]."""
    rng = np.random.default_rng(seed)
    n = batch * (seq_len + 1)
    if law == "uniform":
        seq = rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)
    elif law == "zipf":
        seq = zipf_ids(rng, vocab, n)
    else:
        raise ValueError(law)
    seq = seq.reshape(batch, seq_len + 1)
    return np.ascontiguousarray(seq[:, :-1]), np.ascontiguousarray(seq[:, 1:])


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_params(entries, total: int, seed: int, dtype: str, depth: int,
                std: float = 0.02):
    """Flat parameter buffer for a layout given as (name, offset, rows, cols).

    Output projections (names ending in '.Wo' and '.Wpr') use
    std / sqrt(2 * depth). Returns float32 values for dtype 'f32' or uint16
    bf16 bit patterns for 'bf16'. Padding between tensors is 0."""
    rng = np.random.default_rng(seed)
    out = np.zeros(total, dtype=np.float32)
    scale = 1.0 / np.sqrt(2.0 * depth)
    for name, off, r, c in entries:
        s = std * (scale if (name.endswith(".Wo") or name.endswith(".Wpr")) else 1.0)
        out[off:off + r * c] = (s * rng.standard_normal(r * c)).astype(np.float32)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        return f32_to_bf16_bits(out)
    raise ValueError(dtype)


def as_float64(flat: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a parameter buffer (float32 values or bf16 bits)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(flat).astype(np.float64)
    return np.asarray(flat, dtype=np.float32).astype(np.float64)


def make_token_bytes(vocab: int, seed: int) -> np.ndarray:
    """Synthetic byte length of every vocabulary id, int32 [vocab]."""
    rng = np.random.default_rng(seed)
    b = (1 + rng.geometric(1.0 / 3.8, size=vocab)).astype(np.int32)
    b[:min(256, vocab)] = 1
    b[max(0, vocab - 8):] = 0
    return b
