"""What rounding the lm_head output to bf16 before the softcap changes.

The HIP path in bf16 mode stores each chunk's raw logits l = n(x) U^T as bf16
(one rounding of an fp32 accumulator) and applies the softcap c*tanh(l/c) and
the cross-entropy to those values (followin.io release article, architecture
list: logit softcap; wmrh.cn tutorial, section 2.3: next-token objective). The
oracle keeps l in fp64. This test measures the difference with the oracle's own
functions, on the first 256 positions of row 0 of the mid workload (depth 12,
V = 65,536, the bench's parameter recipe), and checks it against a bound that
holds at any size:

  one bf16 rounding (8 significant bits) moves l by at most 2^-8 |l| (the
  fp32 accumulator's own rounding before it adds 2^-24 |l| at most); tanh's
  derivative is <= 1, and log-sum-exp minus one entry changes by at most
  2 max_v |dz_v|, so each token's loss moves by at most 2^-7 max_v |l_v|
  (with the same small fp32 allowance).

Measured here (random init, logits of RMS ~0.55): mean loss relative change
~3e-6, gradients (dlogits, dU, d n(x)) relative L2 ~1e-5 - three orders below
the bf16 bar (3e-2).
"""
import numpy as np

import oracle
from dense_gpt_pretraining_nanochat_amd import inputs
from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW

TP = 256


def _cos_rel(a, b):
    a, b = a.ravel(), b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))), float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_bf16_logits_before_softcap_within_bound():
    c = PRESETS["C3"]
    pseed, dseed = SEEDS["C3"]
    ocfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=1)
    flat = inputs.make_params(oracle.layout(ocfg), oracle.param_count(ocfg, padded=True), pseed,
                              c.dtype, c.depth)
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW["C3"])
    P = oracle.unpack(ocfg, inputs.as_float64(flat, c.dtype))
    del flat
    # causal: the first TP positions of the row see only the first TP tokens
    _, cache = oracle.row_forward(ocfg, P, tok[0, :TP], keep=True)
    xf, U = cache["xf"], P["U"]
    l = xf @ U.T
    lb = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(l.astype(np.float32))).astype(np.float64)
    assert np.all(np.abs(lb - l) <= (2.0 ** -8 + 2.0 ** -24) * np.abs(l))
    w = 1.0 / TP
    le, de = oracle.softcap_ce_rows(l, tgt[0, :TP], c.softcap, w)
    lr, dr = oracle.softcap_ce_rows(lb, tgt[0, :TP], c.softcap, w)
    bound = 2 * (2.0 ** -8 + 2.0 ** -24) * np.abs(l).max(axis=1)
    assert np.all(np.abs(lr - le) <= bound)
    assert abs(lr.mean() - le.mean()) / le.mean() <= 1e-4
    for name, got, ref in (("dlogits", dr, de), ("dU", dr.T @ xf, de.T @ xf), ("dxf", dr @ U, de @ U)):
        cos, rl2 = _cos_rel(got, ref)
        assert cos >= 1 - 1e-6 and rl2 <= 1e-3, (name, cos, rl2)
