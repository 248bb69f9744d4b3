"""Gradient accumulation and the optimizer step on the GPU, against the fp64
oracle (oracle/model.py for the gradients, oracle/optim.py for the step).

Inputs are seeded and synthetic on both sides: parameters and tokens from the
shared input generators, gradients for the optimizer test from a seeded
normal draw (so no oracle input comes from the GPU path).

Bars: fp32 mode - per-tensor max relative error (R15) of the parameter
change and of the optimizer state <= 1e-4; bf16 mode (Newton-Schulz on bf16
operands, parameters rounded to bf16) - per-tensor cosine >= 0.999 and
relative L2 <= 3e-2 of the parameter change, state <= 1e-4."""
import numpy as np
import pytest

import oracle
from oracle import optim as ooptim
from dense_gpt_pretraining_nanochat_amd import inputs
from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW
from tests.gpu_util import check_bf16, dev, host64, max_rel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_gpt_pretraining_nanochat_amd as nc  # noqa: E402


def _setup(name):
    c = PRESETS[name]
    pseed, dseed = SEEDS[name]
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    ocfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=c.batch)
    flat = inputs.make_params(oracle.layout(ocfg), oracle.param_count(ocfg, padded=True), pseed,
                              c.dtype, c.depth)
    step = nc.Step(cfg)
    if c.dtype == "bf16":
        step.params.copy_(torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda())
    else:
        step.params.copy_(torch.from_numpy(flat).cuda())
    return c, cfg, ocfg, step, inputs.as_float64(flat, c.dtype), dseed


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_grad_accumulation(name):
    c, cfg, ocfg, step, p64, dseed = _setup(name)
    law = TOKEN_LAW[name]
    tA, gA = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, law)
    tB, gB = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed + 17, law)
    step.forward_backward(dev(tA), dev(gA))
    ga = host64(step.grads)
    step.forward_backward(dev(tB), dev(gB))
    gb = host64(step.grads)
    step.grads.fill_(0)
    step.forward_backward_accumulate(dev(tA), dev(gA))
    step.forward_backward_accumulate(dev(tB), dev(gB))
    torch.cuda.synchronize()
    acc = host64(step.grads)
    assert step.status() == 0
    # accumulation adds each batch's gradient in fp32: the sum of the two
    # separate results up to fp32 rounding of the additions
    for tname, off, r, cc in oracle.layout(ocfg):
        sl = slice(off, off + r * cc)
        assert max_rel(acc[sl], ga[sl] + gb[sl]) <= 1e-6, tname
    # and it meets the step's parity bar against the oracle's summed gradient
    _, oa, _ = oracle.forward_backward(ocfg, p64, tA, gA)
    _, ob, _ = oracle.forward_backward(ocfg, p64, tB, gB)
    for tname, off, r, cc in oracle.layout(ocfg):
        sl = slice(off, off + r * cc)
        if c.dtype == "f32":
            assert max_rel(acc[sl], oa[sl] + ob[sl]) <= 1e-3, tname
        else:
            check_bf16(acc[sl], oa[sl] + ob[sl], tname)


def _grads(ocfg, n, seed):
    """Seeded synthetic gradients: normal, scaled per tensor like a real
    gradient (the embedding sparse in rows, as with a Zipf batch)."""
    rng = np.random.default_rng(seed)
    g = np.zeros(n)
    for tname, off, r, c in oracle.layout(ocfg):
        x = rng.standard_normal((r, c)) * (1e-3 if tname in ("E", "U") else 3e-3)
        if tname == "E":
            x[rng.random(r) < 0.7] = 0.0        # ids absent from the batch
        g[off:off + r * c] = x.ravel()
    return g


def _run_steps(name, oc_kw, nsteps=2, seed=900):
    c, cfg, ocfg, step, p64, _ = _setup(name)
    n = oracle.param_count(ocfg, padded=True)
    gs = [_grads(ocfg, n, seed + k) for k in range(nsteps)]
    norm0 = ooptim.global_norm([gs[0][o:o + r * cc] for _, o, r, cc in oracle.layout(ocfg)])
    kw = dict(oc_kw)
    if kw.get("max_grad_norm") == "half":
        kw["max_grad_norm"] = 0.5 * norm0
    # oracle
    oc = ooptim.OptimConfig(**kw)
    po, s1, s2 = p64.copy(), np.zeros(n), np.zeros(n)
    onorms, ops = [], []
    for k in range(nsteps):
        po, s1, s2, gn = ooptim.optimizer_step(ocfg, oc, po, gs[k], s1, s2, k + 1)
        onorms.append(gn)
        ops.append(po.copy())
    # GPU
    gnorms, gps = [], []
    for k in range(nsteps):
        step.grads.copy_(torch.from_numpy(gs[k].astype(np.float32)).cuda())
        o = nc.nc_optim_config(kw["lr_adamw"], kw["beta1"], kw["beta2"], kw["eps"], kw["wd_adamw"],
                               kw["lr_muon"], kw["momentum"], kw["wd_muon"], kw["max_grad_norm"],
                               kw.get("ns_steps", 5), k + 1)
        gn = step.optimizer_step(o)
        torch.cuda.synchronize()
        gnorms.append(float(gn.item()))
        gps.append(host64(step.params))
    state = host64(step.opt_state)
    return c, ocfg, p64, ops, gps, onorms, gnorms, (s1, s2), state


OC = dict(lr_adamw=0.01, beta1=0.8, beta2=0.95, eps=1e-10, wd_adamw=0.05, lr_muon=0.1,
          momentum=0.95, wd_muon=0.02, max_grad_norm="half")


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_optimizer_steps_match_oracle(name):
    c, ocfg, p0, ops, gps, onorms, gnorms, (s1, s2), state = _run_steps(name, OC)
    for on, gn in zip(onorms, gnorms):
        assert abs(gn - on) <= 1e-5 * on
    n = len(p0)
    for k, (po, pg) in enumerate(zip(ops, gps)):
        for tname, off, r, cc in oracle.layout(ocfg):
            sl = slice(off, off + r * cc)
            dg, do = pg[sl] - p0[sl], po[sl] - p0[sl]
            if c.dtype == "f32":
                assert max_rel(dg, do) <= 1e-4, (k, tname, max_rel(dg, do))
            else:
                check_bf16(dg, do, f"step {k + 1} {tname}")
    for tname, off, r, cc in oracle.layout(ocfg):
        sl = slice(off, off + r * cc)
        assert max_rel(state[sl], s1[sl]) <= 1e-4, tname
        if tname in ("E", "U"):
            assert max_rel(state[n:][sl], s2[sl]) <= 1e-4, tname


def test_optimizer_without_newton_schulz():
    kw = dict(OC, ns_steps=0)
    c, ocfg, p0, ops, gps, onorms, gnorms, _, _ = _run_steps("C1", kw, nsteps=1)
    for tname, off, r, cc in oracle.layout(ocfg):
        sl = slice(off, off + r * cc)
        assert max_rel(gps[0][sl] - p0[sl], ops[0][sl] - p0[sl]) <= 1e-4, tname


def test_optimizer_is_deterministic():
    a = _run_steps("C2", OC, nsteps=1)
    b = _run_steps("C2", OC, nsteps=1)
    assert np.array_equal(a[4][0], b[4][0])
    assert a[6] == b[6]


def test_optimizer_step_depth12_bf16():
    """d = 768 with 12 layers: the batched Newton-Schulz products B X
    (768 x 3072 per layer, 12 layers) take the 256-tile kernel."""
    depth, V = 12, 1024
    cfg = nc.nc_config_from_depth(depth, V, 64, 1, "bf16")
    ocfg = oracle.OracleConfig(depth=depth, vocab=V, seq_len=64, batch=1)
    n = oracle.param_count(ocfg, padded=True)
    flat = inputs.make_params(oracle.layout(ocfg), n, 4242, "bf16", depth)
    p0 = inputs.as_float64(flat, "bf16")
    step = nc.Step(cfg)
    step.params.copy_(torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda())
    g = _grads(ocfg, n, 77)
    kw = dict(OC, max_grad_norm=0.0)            # clipping disabled
    po, _, _, onorm = ooptim.optimizer_step(ocfg, ooptim.OptimConfig(**kw), p0, g, np.zeros(n),
                                            np.zeros(n), 1)
    step.grads.copy_(torch.from_numpy(g.astype(np.float32)).cuda())
    o = nc.nc_optim_config(kw["lr_adamw"], kw["beta1"], kw["beta2"], kw["eps"], kw["wd_adamw"],
                           kw["lr_muon"], kw["momentum"], kw["wd_muon"], kw["max_grad_norm"], 5, 1)
    gn = float(step.optimizer_step(o).item())
    pg = host64(step.params)
    assert abs(gn - onorm) <= 1e-5 * onorm
    for tname, off, r, cc in oracle.layout(ocfg):
        sl = slice(off, off + r * cc)
        check_bf16(pg[sl] - p0[sl], po[sl] - p0[sl], tname)


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_three_training_iterations_match_oracle(name):
    """Forward + backward + optimizer step, three times in a row on one
    seeded batch, against the oracle doing the same: the parameters after
    the third step (the whole training loop's state) and the loss of every
    iteration. In bf16 mode each update carries the one-step bar (rel L2
    3e-2) and the parameter differences feed the next gradients, so the sum
    of three updates is held to three times it (rel L2 <= 0.1, cosine >=
    0.995); fp32 mode keeps max-rel 1e-3."""
    c, cfg, ocfg, step, p64, dseed = _setup(name)
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[name])
    kw = dict(OC, max_grad_norm=1.0)
    oc = ooptim.OptimConfig(**kw)
    n = oracle.param_count(ocfg, padded=True)
    po, s1, s2 = p64.copy(), np.zeros(n), np.zeros(n)
    olosses = []
    for k in range(3):
        loss, g, _ = oracle.forward_backward(ocfg, po, tok, tgt)
        olosses.append(loss)
        po, s1, s2, _ = ooptim.optimizer_step(ocfg, oc, po, g, s1, s2, k + 1)
        if c.dtype == "bf16":                     # bf16 parameters: rounded once per step
            po = inputs.as_float64(inputs.f32_to_bf16_bits(po.astype(np.float32)), "bf16")
    glosses = []
    for k in range(3):
        step.grads.fill_(0)
        glosses.append(float(step.forward_backward(dev(tok), dev(tgt)).item()))
        o = nc.nc_optim_config(kw["lr_adamw"], kw["beta1"], kw["beta2"], kw["eps"], kw["wd_adamw"],
                               kw["lr_muon"], kw["momentum"], kw["wd_muon"], kw["max_grad_norm"], 5,
                               k + 1)
        step.optimizer_step(o)
    torch.cuda.synchronize()
    assert step.status() == 0
    bar = 1e-4 if c.dtype == "f32" else 5e-3
    for gl, ol in zip(glosses, olosses):
        assert abs(gl - ol) <= bar * ol, (glosses, olosses)
    assert glosses[2] < glosses[0]                 # the loop learns the batch
    pg = host64(step.params)
    for tname, off, r, cc in oracle.layout(ocfg):
        sl = slice(off, off + r * cc)
        if c.dtype == "f32":
            assert max_rel(pg[sl] - p64[sl], po[sl] - p64[sl]) <= 1e-3, tname
        else:
            check_bf16(pg[sl] - p64[sl], po[sl] - p64[sl], tname, cos_min=0.995, l2_max=0.1)
