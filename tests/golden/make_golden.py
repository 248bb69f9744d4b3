"""Writes the stored expected values for the large-workload parity tests.

Calls only the oracle (and the seeded input generators); the sketch helper
post-processes the oracle's own gradient. For each of the mid (depth 12),
depth-20 and depth-26 workloads it runs the fp64 oracle forward and backward
on batch row 0 (all T = 2048 tokens) and stores, per workload, in
tests/golden/oracle_<name>_row0.npz:
  loss               mean loss over row 0's tokens
  token_losses       [T] per-token losses of row 0
  touched            the distinct token ids of row 0 (the only rows of E with a
                     nonzero gradient; every other row must be exactly 0)
  <tensor>.idx       4096 seeded flat indices into the gradient buffer (int32):
                     for E drawn from the touched rows only, for U half from
                     the rows of row 0's targets (which carry the one-hot
                     term) and half from all rows, uniform for the blocks
  <tensor>.val       the oracle gradient at those indices (float32)
  <tensor>.norm      the L2 norm of the oracle's whole gradient tensor
  <tensor>.sk        the count-sketch (tests/sketch.py) of the whole tensor

Run from the repo root:  python tests/golden/make_golden.py [C3 C4 C5]
(about 1, 2 and 4 minutes of CPU on 8 cores).
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from dense_gpt_pretraining_nanochat_amd import inputs  # noqa: E402
from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW  # noqa: E402
from tests import sketch  # noqa: E402

SAMPLES = 4096


def _rows_sample(rng, rows, d, n):
    """n distinct flat offsets (within a [*, d] tensor) from the given rows."""
    cells = rows.size * d
    pick = rng.choice(cells, size=min(n, cells), replace=False)
    return rows[pick // d].astype(np.int64) * d + pick % d


def make(name):
    c = PRESETS[name]
    pseed, dseed = SEEDS[name]
    cfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=1)
    t0 = time.time()
    flat = inputs.make_params(oracle.layout(cfg), oracle.param_count(cfg, padded=True), pseed,
                              c.dtype, c.depth)
    p64 = inputs.as_float64(flat, c.dtype)
    del flat
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[name])
    loss, g, per_tok = oracle.forward_backward(cfg, p64, tok[:1], tgt[:1])
    del p64
    rng = np.random.default_rng(4242)
    touched = np.unique(tok[0]).astype(np.int32)
    targets = np.unique(tgt[0]).astype(np.int64)
    out = {"loss": np.float64(loss), "token_losses": per_tok[0], "touched": touched}
    for tname, off, r, cc in oracle.layout(cfg):
        n = r * cc
        if tname == "E":
            local = _rows_sample(rng, touched.astype(np.int64), cc, SAMPLES)
        elif tname == "U":
            a = _rows_sample(rng, targets, cc, SAMPLES // 2)
            b = rng.choice(n, size=SAMPLES - a.size, replace=False)
            local = np.unique(np.concatenate([a, b]))
        else:
            local = rng.choice(n, size=min(SAMPLES, n), replace=False)
        idx = off + np.sort(local)
        assert idx.max() < 2 ** 31
        out[f"{tname}.idx"] = idx.astype(np.int32)
        out[f"{tname}.val"] = g[idx].astype(np.float32)
        out[f"{tname}.norm"] = np.float64(np.linalg.norm(g[off:off + n]))
        out[f"{tname}.sk"] = sketch.sketch_np(g[off:off + n], off).astype(np.float32)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"oracle_{name}_row0.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: loss {loss:.6f}  ({time.time() - t0:.0f} s) -> {path}", flush=True)


if __name__ == "__main__":
    for name in (sys.argv[1:] or ["C3", "C4", "C5"]):
        make(name)
