"""Writes the stored expected values for the large-workload parity tests.

Calls only the oracle (and the seeded input generators): for each of the mid
(depth 12), depth-20 and depth-26 workloads it runs the fp64 oracle forward
and backward on batch row 0 (all T = 2048 tokens) and stores, per workload,
in tests/golden/oracle_<name>_row0.npz:
  loss             mean loss over row 0's tokens
  token_losses     [T] per-token losses of row 0
  <tensor>.idx     256 seeded flat indices into the gradient buffer (per tensor)
  <tensor>.val     the oracle gradient at those indices (mean over row 0)
  <tensor>.norm    the L2 norm of the oracle's whole gradient tensor

Run from the repo root:  python tests/golden/make_golden.py [C3 C4 C5]
(about 1, 3 and 6 minutes of CPU on 8 cores).
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

SAMPLES = 256


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
    rng = np.random.default_rng(4242)
    out = {"loss": np.float64(loss), "token_losses": per_tok[0]}
    for tname, off, r, cc in oracle.layout(cfg):
        n = r * cc
        idx = off + np.sort(rng.choice(n, size=min(SAMPLES, n), replace=False))
        out[f"{tname}.idx"] = idx.astype(np.int64)
        out[f"{tname}.val"] = g[idx]
        out[f"{tname}.norm"] = np.float64(np.linalg.norm(g[off:off + n]))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"oracle_{name}_row0.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: loss {loss:.6f}  ({time.time() - t0:.0f} s) -> {path}", flush=True)


if __name__ == "__main__":
    for name in (sys.argv[1:] or ["C3", "C4", "C5"]):
        make(name)
