"""The process-pool runner of the oracle gives what one process gives: the
same loss, per-token losses and gradient (up to the order of fp64 sums) for
the small workload's whole batch, with its rows split over several workers."""
import numpy as np

import oracle
from dense_gpt_pretraining_nanochat_amd import inputs
from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW
from tests import oracle_pool


def test_pool_equals_serial_oracle():
    name = "C2"
    c = PRESETS[name]
    pseed, dseed = SEEDS[name]
    cfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=c.batch)
    flat = inputs.make_params(oracle.layout(cfg), oracle.param_count(cfg, padded=True), pseed,
                              c.dtype, c.depth)
    p64 = inputs.as_float64(flat, c.dtype)
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[name])
    loss, g, pt = oracle.forward_backward(cfg, p64, tok, tgt)
    ploss, pg, ppt = oracle_pool.forward_backward_batch(name, c.batch, workers=3)
    assert abs(ploss - loss) <= 1e-12 * loss
    assert np.abs(ppt - pt).max() <= 1e-10
    assert np.abs(pg - g).max() <= 1e-12 * np.abs(g).max()
