"""Pins of the optimizer oracle (oracle/optim.py) against closed forms and
invariants that do not restate its code: the Newton-Schulz iteration acts on
singular values only (checked through numpy's SVD), AdamW's first step from a
zero state has a closed form, and Muon's update is invariant to the gradient's
scale and, for a constant gradient, the same at every step."""
import numpy as np
import pytest

from oracle import optim
from oracle.model import OracleConfig, layout, param_count



def _quintic_singular(s, steps):
    a, b, c = optim.NS_COEFFS
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (16, 16), (5, 40)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_newton_schulz_acts_on_singular_values(shape, steps):
    rng = np.random.default_rng(shape[0] * 100 + shape[1] + steps)
    u = rng.standard_normal(shape)
    U, S, Vt = np.linalg.svd(u, full_matrices=False)
    s0 = S / (np.linalg.norm(u) + 1e-7)
    expect = (U * _quintic_singular(s0, steps)) @ Vt
    got = optim.newton_schulz(u, steps)
    assert got.shape == u.shape
    assert np.abs(got - expect).max() <= 1e-12 * max(1.0, np.abs(expect).max())


def test_newton_schulz_pushes_singular_values_into_band():
    # the published coefficients move every singular value in (0, 1] to
    # roughly [0.7, 1.2] within five steps
    rng = np.random.default_rng(7)
    u = rng.standard_normal((64, 128)) @ np.diag(np.logspace(-3, 0, 128))
    s = np.linalg.svd(optim.newton_schulz(u, 5), compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.25


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(3)
    th = rng.standard_normal((7, 5))
    g = rng.standard_normal((7, 5))
    lr, b1, b2, eps, wd = 0.01, 0.8, 0.95, 1e-10, 0.1
    new, m, v = optim.adamw(th, g, np.zeros_like(g), np.zeros_like(g), 1, lr, b1, b2, eps, wd)
    # bias correction makes the first moments exactly g and g^2
    assert np.allclose(m, (1 - b1) * g, rtol=0, atol=1e-15)
    assert np.allclose(v, (1 - b2) * g * g, rtol=0, atol=1e-15)
    expect = th * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.abs(new - expect).max() <= 1e-14


def test_muon_first_step_scale_invariant():
    rng = np.random.default_rng(4)
    th = rng.standard_normal((12, 20))
    g = rng.standard_normal((12, 20))
    a, _ = optim.muon(th, g, np.zeros_like(g), 0.02, 0.95, 0.0, 5)
    b, _ = optim.muon(th, 37.0 * g, np.zeros_like(g), 0.02, 0.95, 0.0, 5)
    assert np.abs(a - b).max() <= 1e-9


@pytest.mark.parametrize("shape", [(12, 20), (20, 12)])
def test_muon_constant_gradient_repeats_update(shape):
    # with the same gradient every step the momentum stays parallel to it, so
    # the orthogonalised update (scale invariant) repeats exactly; a wrong
    # sign in the momentum mix flips or shrinks it
    rng = np.random.default_rng(5)
    th0 = rng.standard_normal(shape)
    g = rng.standard_normal(shape)
    buf = np.zeros_like(g)
    th1, buf = optim.muon(th0, g, buf, 0.02, 0.95, 0.0, 5)
    th2, buf = optim.muon(th1, g, buf, 0.02, 0.95, 0.0, 5)
    d1, d2 = th1 - th0, th2 - th1
    # (equal up to the 1e-7 guard in the normalisation, ~1e-8 relative here)
    assert np.abs(d1 - d2).max() <= 1e-7 * np.abs(d1).max()
    # and it is the lr-scaled orthogonalisation of g itself, with the
    # max(1, rows/cols)^(1/2) factor for tall matrices
    scale = max(1.0, shape[0] / shape[1]) ** 0.5
    assert np.abs(d1 + 0.02 * scale * optim.newton_schulz(g, 5)).max() <= 1e-7 * np.abs(d1).max()


def test_clip_scale():
    assert optim.clip_scale(3.0, 5.0) == 1.0
    assert optim.clip_scale(3.0, 0.0) == 1.0
    assert abs(optim.clip_scale(4.0, 2.0) - 2.0 / (4.0 + 1e-6)) < 1e-15


def test_optimizer_step_routes_tensors_and_clips():
    cfg = OracleConfig(depth=2, vocab=64, seq_len=16, batch=1, head_dim=16, d_model=32)
    n = param_count(cfg, padded=True)
    rng = np.random.default_rng(6)
    p = rng.standard_normal(n) * 0.02
    g = rng.standard_normal(n)
    z = np.zeros(n)
    norm = np.linalg.norm(np.concatenate([g[o:o + r * c] for _, o, r, c in layout(cfg)]))
    oc = optim.OptimConfig(lr_adamw=0.01, beta1=0.8, beta2=0.95, eps=1e-10, wd_adamw=0.0,
                           lr_muon=0.02, momentum=0.95, wd_muon=0.0, max_grad_norm=norm / 4)
    newp, s1, s2, gn = optim.optimizer_step(cfg, oc, p, g, z, z, 1)
    assert abs(gn - norm) <= 1e-12 * norm
    for name, off, r, c in layout(cfg):
        sl = slice(off, off + r * c)
        d = (newp[sl] - p[sl]).reshape(r, c)
        if name in ("E", "U"):
            # first AdamW step: -lr gc / (|gc| + eps) (about -lr sign(g)) with gc
            # the clipped gradient
            gc = g[sl].reshape(r, c) / 4 * (norm / (norm + 1e-6))
            assert np.abs(d + 0.01 * gc / (np.abs(gc) + 1e-10)).max() <= 1e-15
            assert np.any(s2[sl] != 0)
        else:
            # Muon's momentum holds the clipped gradient; the update does not
            # depend on the clip
            assert np.abs(s1[sl] - g[sl] / 4 * (norm / (norm + 1e-6))).max() <= 1e-9
            scale = max(1.0, r / c) ** 0.5
            assert np.abs(d + 0.02 * scale * optim.newton_schulz(g[sl].reshape(r, c), 5)).max() \
                <= 1e-6 * np.abs(d).max()
            assert np.all(s2[sl] == 0)


def test_muon_nesterov_cancellation_leaves_only_decay():
    # buf2 = mu g1 + g2 and u2 = g2 + mu buf2 = (1 + mu) g2 + mu^2 g1, which
    # vanishes for g2 = -mu^2 / (1 + mu) g1: the second step is then pure
    # weight decay (plain momentum, u2 = buf2, would still move theta)
    rng = np.random.default_rng(8)
    mu, lr, wd = 0.95, 0.02, 0.1
    th0 = rng.standard_normal((10, 14))
    g1 = rng.standard_normal((10, 14))
    th1, buf = optim.muon(th0, g1, np.zeros_like(g1), lr, mu, wd, 5)
    th2, _ = optim.muon(th1, -mu * mu / (1 + mu) * g1, buf, lr, mu, wd, 5)
    # (u2 is rounding residue, ~1e-15; normalised against the 1e-7 guard and
    # amplified by the quintic steps it moves theta by ~1e-8, against ~lr for
    # plain momentum)
    assert np.abs(th2 - th1 * (1 - lr * wd)).max() <= 1e-6 * np.abs(th1).max()
