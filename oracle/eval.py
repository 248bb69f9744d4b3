"""fp64 oracle of the bits-per-byte evaluation of a batch.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The harness page lists a loss-evaluation module that reports bits per byte
([harness] section "Cấu trúc thư mục và module chính"); the tutorial quotes
tokenizers in the same unit ([tutorial] section 2.1). The pages do not spell
the formula out; the reading here is the usual definition of the unit: the
cross-entropy of the next-token predictions, in bits, per byte of the text
the predicted tokens stand for,

    bpb = sum_t loss_t / (ln 2 * sum_t bytes(target_t)),

summed over the positions whose target has a nonzero byte length (special
tokens have none and drop out of both sums). ``token_bytes[v]`` is the byte
length of vocabulary id v (the tokenizer's table; not available offline,
so the tests draw a synthetic one).

``parity unpinned`` does not apply: the tests pin the function to closed
forms (a zero lm_head gives every position the loss ln V exactly), to the
mean loss when every length is equal, and to its scaling in the lengths.
"""
from __future__ import annotations

import math

import numpy as np

from .model import OracleConfig, forward_loss


def bits_per_byte(cfg: OracleConfig, params: np.ndarray, tokens: np.ndarray, targets: np.ndarray,
                  token_bytes: np.ndarray):
    """Returns (nats, bytes, bpb) over the batch: the summed loss of the
    counted positions, their summed byte lengths and the ratio in bits per
    byte (nan when no position counts)."""
    _, per_tok = forward_loss(cfg, params, tokens, targets, return_token_losses=True)
    return bits_per_byte_from_losses(per_tok, targets, token_bytes)


def bits_per_byte_from_losses(per_tok: np.ndarray, targets: np.ndarray, token_bytes: np.ndarray):
    """The same ratio from per-position losses already computed (in nats)."""
    per_tok = np.asarray(per_tok, dtype=np.float64)
    nbytes = np.asarray(token_bytes, dtype=np.int64)[np.asarray(targets).reshape(per_tok.shape)]
    counted = nbytes > 0
    nats = float(per_tok[counted].sum())
    total = int(nbytes[counted].sum())
    bpb = nats / (math.log(2.0) * total) if total > 0 else float("nan")
    return nats, total, bpb
