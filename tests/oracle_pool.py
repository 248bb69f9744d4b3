"""Runs the fp64 oracle over the rows of a whole batch in several processes.

Test infrastructure: each worker (a fresh spawned interpreter that never
touches the GPU) rebuilds the seeded parameters and tokens of a preset itself,
runs ``oracle.forward_backward`` on its contiguous share of the rows with the
batch's 1/M weighting, and returns its partial loss sum, gradient and
per-token losses. The parent adds the partial gradients in row-group order, so
the result does not depend on which worker finishes first. The oracle's own
arithmetic is untouched; this only spreads its per-row loop over the host's
cores (most of a row's time is single-threaded numpy elementwise work).
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np


def _host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    # a GPU machine's share is 16 host cores whatever the machine shows
    return max(1, min(n, 16))


def _worker(args):
    name, rows, batch, threads = args
    from threadpoolctl import threadpool_limits

    import oracle
    from dense_gpt_pretraining_nanochat_amd import inputs
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW
    with threadpool_limits(threads):
        c = PRESETS[name]
        pseed, dseed = SEEDS[name]
        cfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=batch)
        flat = inputs.make_params(oracle.layout(cfg), oracle.param_count(cfg, padded=True), pseed,
                                  c.dtype, c.depth)
        p64 = inputs.as_float64(flat, c.dtype)
        del flat
        tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[name])
        loss, g, per_tok = oracle.forward_backward(cfg, p64, tok[:batch], tgt[:batch], rows=rows,
                                                   M=batch * c.seq_len)
    return float(loss) * batch * c.seq_len, g, per_tok


def forward_backward_batch(name: str, batch: int, workers: int | None = None):
    """Oracle loss, flat fp64 gradient and [batch, T] token losses for rows
    0..batch-1 of preset ``name`` (seeded as the tests seed it)."""
    cores = _host_cores()
    workers = max(1, min(workers or max(1, cores // 4), batch))
    threads = max(1, cores // workers)
    groups = [list(r) for r in np.array_split(np.arange(batch), workers) if len(r)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(len(groups)) as pool:
        parts = pool.map(_worker, [(name, g, batch, threads) for g in groups])
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS
    T = PRESETS[name].seq_len
    total = 0.0
    grads = None
    per_tok = []
    for s, g, pt in parts:
        total += s
        grads = g if grads is None else grads + g
        per_tok.append(pt)
    return total / (batch * T), grads, np.concatenate(per_tok, axis=0)
