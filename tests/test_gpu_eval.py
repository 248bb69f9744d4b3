"""Bits-per-byte evaluation on the GPU (nc_eval_bpb) against the fp64 oracle
(oracle/eval.py) on the same seeded parameters, tokens and synthetic byte
table.

Bars: the summed byte length is exact (integer work); the summed loss and the
ratio meet the loss bar of the mode (relative error <= 1e-4 fp32, <= 5e-3
bf16). At depth 20 row 0 is checked against the oracle's stored per-token
losses (tests/golden/make_golden.py)."""
import math
import os

import numpy as np
import pytest

import oracle
from dense_gpt_pretraining_nanochat_amd import inputs
from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_gpt_pretraining_nanochat_amd as nc  # noqa: E402

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _setup(name, batch=None):
    c = PRESETS[name]
    B = batch or c.batch
    pseed, dseed = SEEDS[name]
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, B, c.dtype)
    ocfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=B)
    flat = inputs.make_params(oracle.layout(ocfg), oracle.param_count(ocfg, padded=True), pseed,
                              c.dtype, c.depth)
    step = nc.Step(cfg, with_backward=False)
    if c.dtype == "bf16":
        step.params.copy_(torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda())
    else:
        step.params.copy_(torch.from_numpy(flat).cuda())
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[name])
    return c, ocfg, step, flat, tok[:B], tgt[:B]


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_bpb_matches_oracle(name):
    c, ocfg, step, flat, tok, tgt = _setup(name)
    tb = inputs.make_token_bytes(c.vocab_size, 31)
    tb[np.unique(tgt)[:3]] = 0                     # some targets count as special tokens
    got = step.eval_bpb(dev(tok), dev(tgt), dev(tb)).cpu().numpy()
    loss = float(step.loss.item())
    assert step.status() == 0
    nats, nbytes, bpb = oracle.bits_per_byte(ocfg, inputs.as_float64(flat, c.dtype), tok, tgt, tb)
    bar = 1e-4 if c.dtype == "f32" else 5e-3
    assert got[1] == nbytes
    assert abs(got[0] - nats) <= bar * nats
    assert abs(got[2] - bpb) <= bar * bpb
    assert abs(loss - oracle.forward_loss(ocfg, inputs.as_float64(flat, c.dtype), tok, tgt)) <= bar * loss


def test_bpb_zero_lm_head():
    """Every logit 0: each counted position costs log2(V) bits exactly."""
    c, ocfg, step, flat, tok, tgt = _setup("C1")
    for n, off, r, cc in step.layout:
        if n == "U":
            step.params[off:off + r * cc].zero_()
    tb = inputs.make_token_bytes(c.vocab_size, 2)
    got = step.eval_bpb(dev(tok), dev(tgt), dev(tb)).cpu().numpy()
    counted = tb[tgt] > 0
    assert got[1] == tb[tgt][counted].sum()
    assert abs(got[2] - math.log2(c.vocab_size) * counted.sum() / got[1]) <= 1e-6 * got[2]


def test_bpb_no_counted_position():
    c, ocfg, step, flat, tok, tgt = _setup("C1")
    got = step.eval_bpb(dev(tok), dev(tgt), dev(np.zeros(c.vocab_size, np.int32))).cpu().numpy()
    assert got[0] == 0.0 and got[1] == 0.0 and math.isnan(got[2])


def test_bpb_depth20_row0_against_stored_oracle():
    c, ocfg, step, flat, tok, tgt = _setup("C4", batch=1)
    del flat
    gold = np.load(os.path.join(GOLD, "oracle_C4_row0.npz"))
    tb = inputs.make_token_bytes(c.vocab_size, 77)
    got = step.eval_bpb(dev(tok), dev(tgt), dev(tb)).cpu().numpy()
    assert step.status() == 0
    nats, nbytes, bpb = oracle.bits_per_byte_from_losses(gold["token_losses"], tgt[0], tb)
    assert got[1] == nbytes
    assert abs(got[2] - bpb) <= 5e-3 * bpb, (got, bpb)
