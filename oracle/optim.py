"""fp64 numpy oracle of one optimizer step: global-norm gradient clipping,
AdamW for the embedding E and the lm_head U, Muon for the block matrices.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix, and what is read from elsewhere:
  * the optimizer pairs Muon with AdamW, after modded-nanoGPT
      [release] the paragraph after the architecture list (optimizer)
  * the optimizer module implements AdamW together with Muon
      [harness] section "Cấu trúc thư mục và module chính"
  * gradient clipping by global norm (max_grad_norm 1.0 as the remedy for
    NaN losses) and gradient accumulation
      [tutorial] sections 4.1 (gradient accumulation), 5.1 (clipping)

The pages do not define either update rule; they are taken from their public
descriptions and written out here step by step:
  * AdamW: Loshchilov & Hutter, "Decoupled Weight Decay Regularization"
    (ICLR 2019), with Adam's bias correction (Kingma & Ba, 2015):
        m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
        mh = m / (1 - b1^t);     vh = v / (1 - b2^t)
        theta <- theta (1 - lr wd) - lr mh / (sqrt(vh) + eps)
  * Muon: K. Jordan et al., "Muon: An optimizer for hidden layers in neural
    networks" (2024): SGD momentum with Nesterov look-ahead, whose update
    matrix is replaced by an approximate orthogonalisation from a quintic
    Newton-Schulz iteration:
        buf <- mu buf + g;       u = g + mu buf
        X0 = u / (||u||_F + 1e-7), transposed when rows > cols
        X_{k+1} = a X_k + (b A + c A^2) X_k,  A = X_k X_k^T,
                  (a, b, c) = (3.4445, -4.7750, 2.0315)
        theta <- theta (1 - lr wd) - lr max(1, rows/cols)^(1/2) X_ns
    Each iteration maps every singular value s of X to a s + b s^3 + c s^5
    and leaves the singular vectors alone; the coefficients push singular
    values in (0, 1] towards roughly [0.7, 1.2] in five steps.
  * global-norm clipping: every gradient is multiplied by
    min(1, max_norm / (||g||_2 + 1e-6)) before the updates, the norm taken
    over all parameters at once; max_norm <= 0 disables it.

Everything is float64. ``parity unpinned`` does not apply: the tests pin the
Newton-Schulz step to the scalar quintic applied to an SVD's singular values,
AdamW's first step to its closed form, and Muon's scale invariance.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .model import OracleConfig, layout

NS_COEFFS = (3.4445, -4.7750, 2.0315)


@dataclass(frozen=True)
class OptimConfig:
    lr_adamw: float
    beta1: float
    beta2: float
    eps: float
    wd_adamw: float
    lr_muon: float
    momentum: float
    wd_muon: float
    max_grad_norm: float
    ns_steps: int = 5


def global_norm(grads: list) -> float:
    """sqrt of the sum of squares of every gradient entry."""
    return float(np.sqrt(sum(float(np.sum(np.square(g))) for g in grads)))


def clip_scale(norm: float, max_norm: float) -> float:
    if max_norm <= 0.0:
        return 1.0
    return min(1.0, max_norm / (norm + 1e-6))


def adamw(theta, g, m, v, step: int, lr, beta1, beta2, eps, wd):
    """One AdamW step; returns the new (theta, m, v)."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    theta = theta * (1.0 - lr * wd) - lr * mh / (np.sqrt(vh) + eps)
    return theta, m, v


def newton_schulz(u: np.ndarray, steps: int) -> np.ndarray:
    """Quintic Newton-Schulz orthogonalisation of a matrix, in the orientation
    of ``u`` (the iteration itself runs on the wide orientation)."""
    a, b, c = NS_COEFFS
    x = u / (np.linalg.norm(u) + 1e-7)
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = x.T
    for _ in range(steps):
        A = x @ x.T
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    return x.T if tall else x


def muon(theta, g, buf, lr, momentum, wd, steps: int):
    """One Muon step on a [rows, cols] matrix; returns the new (theta, buf)."""
    buf = momentum * buf + g
    u = g + momentum * buf
    x = newton_schulz(u, steps)
    rows, cols = theta.shape
    scale = max(1.0, rows / cols) ** 0.5
    theta = theta * (1.0 - lr * wd) - lr * scale * x
    return theta, buf


def is_adamw_tensor(name: str) -> bool:
    return name in ("E", "U")


def optimizer_step(cfg: OracleConfig, oc: OptimConfig, params: np.ndarray, grads: np.ndarray,
                   state1: np.ndarray, state2: np.ndarray, step: int):
    """One step over the flat parameter buffer (fp64 copies). state1 holds
    AdamW's first moment (E, U) or Muon's momentum (matrices), state2 AdamW's
    second moment (E, U only), both in the parameter layout. Returns
    (params, state1, state2, grad_norm) as new arrays."""
    lay = layout(cfg)
    p, s1, s2 = params.copy(), state1.copy(), state2.copy()
    views = [(name, off, r, c) for name, off, r, c in lay]
    norm = global_norm([grads[off:off + r * c] for _, off, r, c in views])
    sc = clip_scale(norm, oc.max_grad_norm)
    for name, off, r, c in views:
        sl = slice(off, off + r * c)
        g = grads[sl].reshape(r, c) * sc
        if is_adamw_tensor(name):
            th, m, v = adamw(p[sl].reshape(r, c), g, s1[sl].reshape(r, c), s2[sl].reshape(r, c), step,
                             oc.lr_adamw, oc.beta1, oc.beta2, oc.eps, oc.wd_adamw)
            p[sl], s1[sl], s2[sl] = th.ravel(), m.ravel(), v.ravel()
        else:
            th, b = muon(p[sl].reshape(r, c), g, s1[sl].reshape(r, c), oc.lr_muon, oc.momentum,
                         oc.wd_muon, oc.ns_steps)
            p[sl], s1[sl] = th.ravel(), b.ravel()
    return p, s1, s2, norm
