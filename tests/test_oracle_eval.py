"""Pins of the bits-per-byte oracle (oracle/eval.py) against closed forms:
with a zero lm_head every logit is 0, so every position's loss is ln V
exactly and the ratio is log2(V) times positions over bytes whatever the
blocks compute; with one byte length b for every id it is the mean loss
over ln 2 * b; it scales as 1/k when every length is multiplied by k;
zero-length (special) targets leave both sums."""
import math

import numpy as np

from dense_gpt_pretraining_nanochat_amd import inputs
from oracle import bits_per_byte, forward_loss
from oracle.model import OracleConfig, layout, param_count

CFG = OracleConfig(depth=2, vocab=64, seq_len=16, batch=2, head_dim=16, d_model=32)


def _params(seed, zero_u=False):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(param_count(CFG, padded=True)) * 0.3
    if zero_u:
        for name, off, r, c in layout(CFG):
            if name == "U":
                p[off:off + r * c] = 0.0
    return p


def _batch(seed):
    tok, tgt = inputs.make_tokens(CFG.vocab, CFG.seq_len, CFG.batch, seed, "uniform")
    return tok, tgt


def test_zero_lm_head_gives_log2_vocab_per_token():
    tok, tgt = _batch(1)
    tb = inputs.make_token_bytes(CFG.vocab, 3)
    tb[:4] = 0                                    # a few more zero-length ids
    nats, nbytes, bpb = bits_per_byte(CFG, _params(2, zero_u=True), tok, tgt, tb)
    counted = tb[tgt] > 0
    assert counted.sum() < tgt.size               # some positions drop out
    assert abs(nats - math.log(CFG.vocab) * counted.sum()) <= 1e-12 * nats
    assert nbytes == int(tb[tgt][counted].sum())
    assert abs(bpb - math.log2(CFG.vocab) * counted.sum() / nbytes) <= 1e-12 * bpb


def test_constant_lengths_give_mean_loss_in_bits():
    tok, tgt = _batch(4)
    p = _params(5)
    for b in (1, 3, 7):
        nats, nbytes, bpb = bits_per_byte(CFG, p, tok, tgt, np.full(CFG.vocab, b))
        loss = forward_loss(CFG, p, tok, tgt)
        assert nbytes == b * tgt.size
        assert abs(bpb - loss / (math.log(2.0) * b)) <= 1e-12 * bpb
        assert abs(nats - loss * tgt.size) <= 1e-12 * nats


def test_scaling_lengths_scales_bits_per_byte():
    tok, tgt = _batch(6)
    p = _params(7)
    tb = inputs.make_token_bytes(CFG.vocab, 8)
    _, _, a = bits_per_byte(CFG, p, tok, tgt, tb)
    _, _, b = bits_per_byte(CFG, p, tok, tgt, 5 * tb)
    assert abs(b - a / 5) <= 1e-12 * a


def test_no_counted_position():
    tok, tgt = _batch(9)
    nats, nbytes, bpb = bits_per_byte(CFG, _params(10), tok, tgt, np.zeros(CFG.vocab, np.int32))
    assert nats == 0.0 and nbytes == 0 and math.isnan(bpb)


def test_synthetic_byte_table():
    tb = inputs.make_token_bytes(65536, 11)
    assert tb.dtype == np.int32 and tb.shape == (65536,)
    assert np.all(tb[:256] == 1) and np.all(tb[-8:] == 0) and np.all(tb[256:-8] >= 2)
    assert 4.5 < tb[256:-8].mean() < 5.1
