"""KV-cache inference on the GPU (nc_prefill, nc_decode_step) against the fp64
oracle's full-sequence forward.

The mask is causal, so the logits the oracle gives at position p of the whole
sequence are what a prefill of positions 0..p-1 followed by decoding steps up
to p must return. Inputs are seeded and synthetic (the shared input
generators); the oracle sees the same parameters and tokens.

Bars: fp32 mode - max |z - z_oracle| / max |z_oracle| <= 1e-4 per position;
bf16 mode - per position cosine >= 0.999 and relative L2 <= 3e-2 of the
logits. At depth 20 (the training shape, cache of 2048 positions) the
per-token losses of row 0 are checked against the oracle values stored by
tests/golden/make_golden.py with the training step's bf16 token bar."""
import os

import numpy as np
import pytest

import oracle
from dense_gpt_pretraining_nanochat_amd import inputs
from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS
from tests.gpu_util import check_bf16, dev, max_rel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_gpt_pretraining_nanochat_amd as nc  # noqa: E402

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _model(depth, V, T, B, dtype, pseed):
    cfg = nc.nc_config_from_depth(depth, V, T, B, dtype)
    ocfg = oracle.OracleConfig(depth=depth, vocab=V, seq_len=T, batch=1)
    flat = inputs.make_params(oracle.layout(ocfg), oracle.param_count(ocfg, padded=True), pseed,
                              dtype, depth)
    if dtype == "bf16":
        params = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        params = torch.from_numpy(flat).cuda()
    P = oracle.unpack(ocfg, inputs.as_float64(flat, dtype))
    return cfg, ocfg, params, P


def _oracle_logits(ocfg, P, seq):
    return np.stack([oracle.row_forward(ocfg, P, row, keep=False)[0] for row in seq])


def _check(got, want, dtype, what):
    if dtype == "f32":
        assert max_rel(got, want) <= 1e-4, (what, max_rel(got, want))
    else:
        check_bf16(got, want, what)


def _run(cfg, params, seq, T0, max_seq, positions):
    """Prefill seq[:, :T0] (T0 = 0: no prefill), then decode every position
    up to the last one asked for; returns {position: logits [B, V]}."""
    dec = nc.Decoder(cfg, params, max_seq)
    out = {}
    if T0:
        out[T0 - 1] = dec.prefill(dev(seq[:, :T0])).double().cpu().numpy()
    for p in range(T0, max(positions) + 1):
        lg = dec.step(dev(np.ascontiguousarray(seq[:, p])))
        if p in positions:
            out[p] = lg.double().cpu().numpy()
    torch.cuda.synchronize()
    assert dec.status() == 0
    return out


@pytest.mark.parametrize("dtype,depth,V,B", [("f32", 2, 512, 3), ("bf16", 4, 8192, 5)])
def test_prefill_then_decode_matches_full_forward(dtype, depth, V, B):
    T0, n = 64, 140                          # decoding crosses the 64- and 128-key chunk edges
    cfg, ocfg, params, P = _model(depth, V, 128, B, dtype, 31 + depth)
    seq, _ = inputs.make_tokens(V, n, B, 77, "zipf")
    want = _oracle_logits(ocfg, P, seq)
    positions = {T0 - 1, T0, T0 + 1, 127, 128, 129, n - 1}
    got = _run(cfg, params, seq, T0, n, positions)
    for p in sorted(positions):
        _check(got[p], want[:, p], dtype, f"position {p}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_from_empty_cache(dtype):
    """No prefill: position 0 attends to itself only; 63/64 is the first chunk
    edge."""
    B, n = 17, 70
    cfg, ocfg, params, P = _model(2, 1024, 64, B, dtype, 5)
    seq, _ = inputs.make_tokens(1024, n, B, 8, "uniform")
    want = _oracle_logits(ocfg, P, seq)
    positions = {0, 1, 62, 63, 64, 69}
    got = _run(cfg, params, seq, 0, 96, positions)
    for p in sorted(positions):
        _check(got[p], want[:, p], dtype, f"position {p}")


def test_wide_batch_takes_the_tiled_path():
    """40 sequences in bf16: more rows than the few-row kernels take, so the
    decoding step pads to 48 rows and runs the tiled GEMM, the separate norm
    kernels and the gathered lm_head; same bar against the oracle."""
    B, n = 40, 72
    cfg, ocfg, params, P = _model(2, 1024, 64, B, "bf16", 21)
    seq, _ = inputs.make_tokens(1024, n, B, 22, "zipf")
    want = _oracle_logits(ocfg, P, seq)
    positions = {63, 64, 71}
    got = _run(cfg, params, seq, 64, 96, positions)
    for p in sorted(positions):
        _check(got[p], want[:, p], "bf16", f"position {p}")


def test_prefill_longest_prompt():
    """A prompt of cfg.seq_len tokens (several attention tiles) into a cache
    of exactly that many positions."""
    B, T = 2, 192
    cfg, ocfg, params, P = _model(2, 512, T, B, "f32", 9)
    seq, _ = inputs.make_tokens(512, T, B, 10, "zipf")
    want = _oracle_logits(ocfg, P, seq)
    got = _run(cfg, params, seq, T, T, {T - 1})
    _check(got[T - 1], want[:, T - 1], "f32", "last prompt position")


def test_decode_is_deterministic():
    B, n = 4, 80
    cfg, ocfg, params, _ = _model(4, 8192, 64, B, "bf16", 12)
    seq, _ = inputs.make_tokens(8192, n, B, 13, "zipf")
    a = _run(cfg, params, seq, 64, 128, {79})
    b = _run(cfg, params, seq, 64, 128, {79})
    assert np.array_equal(a[79], b[79])


def test_depth20_cache_against_stored_oracle():
    """Depth 20, vocab 65,536, 32 sequences, cache of 2048 positions: prefill
    1984 tokens, decode the last 64. Row 0's per-token losses at the decoded
    positions (computed here from the returned logits) match the stored
    oracle values; every row's decoded logits are finite."""
    c = PRESETS["C4"]
    pseed, dseed = SEEDS["C4"]
    gold = np.load(os.path.join(GOLD, "oracle_C4_row0.npz"))
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    ocfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=1)
    flat = inputs.make_params(oracle.layout(ocfg), oracle.param_count(ocfg, padded=True), pseed,
                              c.dtype, c.depth)
    params = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
    del flat
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, "zipf")
    T0 = c.seq_len - 64
    dec = nc.Decoder(cfg, params, c.seq_len)
    losses = {}

    def row0_loss(lg, p):
        z = lg[0].double().cpu().numpy()
        m = z.max()
        return m + np.log(np.exp(z - m).sum()) - z[tgt[0, p]]

    losses[T0 - 1] = row0_loss(dec.prefill(dev(tok[:, :T0])), T0 - 1)
    for p in range(T0, c.seq_len):
        lg = dec.step(dev(np.ascontiguousarray(tok[:, p])))
        losses[p] = row0_loss(lg, p)
        assert bool(torch.isfinite(lg).all())
    torch.cuda.synchronize()
    assert dec.status() == 0
    ref = gold["token_losses"]
    for p, l in losses.items():
        assert abs(l - ref[p]) <= 5e-2 * max(1.0, abs(ref[p])), (p, l, ref[p])
    got = np.array([losses[p] for p in sorted(losses)])
    want = ref[sorted(losses)]
    assert abs(got.mean() - want.mean()) <= 5e-3 * want.mean()


# ------------------------------------------------- decoding kernels, one by one

def _bf16_exact(rng, shape):
    t = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return t.cuda(), t.double().numpy()


@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("M", [1, 5, 16, 17, 32])
@pytest.mark.parametrize("N,K", [(48, 96), (1280, 1280), (208, 5120), (4096, 256)])
@pytest.mark.parametrize("splits,ntile", [(0, 0), (5, 1), (0, 2), (5, 4)])
def test_few_rows_gemm(epi, M, N, K, splits, ntile):
    """Against an fp64 product of the same bf16 values; rows past M and the
    padding columns of C stay untouched. Covers one k slice and several
    (0: the count decoding picks, which gives 3 slices at K = 5120) and 1, 2
    or 4 column tiles per workgroup (0: decoding's choice)."""
    splits = min(splits, K // 32)
    while ntile > 1 and N % (16 * ntile):
        ntile //= 2
    rng = np.random.default_rng(M * 1000 + N + K + epi)
    W, W64 = _bf16_exact(rng, (N, K))
    X, X64 = _bf16_exact(rng, (M, K))
    ref = X64 @ W64.T
    ldc = N + 16
    f32_out = epi in (1, 3)
    sentinel = 7.0
    C = torch.full((M + 3, ldc), sentinel, dtype=torch.float32 if f32_out else torch.bfloat16,
                   device="cuda")
    if epi == 1:
        base = rng.standard_normal((M, N)).astype(np.float32)
        C[:M, :N] = torch.from_numpy(base).cuda()
        ref = ref + base
    if epi == 2:
        ref = np.maximum(ref, 0.0) ** 2
    cap = 0.0
    if epi == 3:
        cap = 0.5 * float(np.abs(ref).max())      # so the cap bends the large values
        ref = cap * np.tanh(ref / cap)
    scratch = torch.zeros(nc.nc_op_few_rows_scratch_bytes(M, N, K, splits), dtype=torch.uint8,
                          device="cuda")
    nc.nc_op_few_rows_gemm(epi, W, K, X, K, C, ldc, M, N, K, scratch, cap=cap, splits=splits, ntile=ntile)
    torch.cuda.synchronize()
    out = C.double().cpu().numpy()
    got = out[:M, :N]
    scale = np.abs(ref).max()
    if f32_out:
        assert max_rel(got, ref) <= 1e-5, max_rel(got, ref)
    else:
        assert np.all(np.abs(got - ref) <= 2 ** -7 * np.abs(ref) + 1e-5 * scale)
    assert np.all(out[M:] == sentinel) and np.all(out[:, N:] == sentinel)
    # the arrival counters are left zero for the next call
    assert int(scratch[:4 * (N // 16)].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("M", [3, 32])
@pytest.mark.parametrize("N,K", [(1536, 1280), (1280, 1280), (5120, 2048)])
@pytest.mark.parametrize("ntile", [1, 4])
def test_few_rows_gemm_norm_and_residual_outputs(M, N, K, ntile):
    """The RMS factor comes from per-16-column sums of squares; the residual
    epilogue also leaves a bf16 copy of the new rows and their sums of
    squares (what the next product folds its norm from)."""
    rng = np.random.default_rng(M + N + K)
    W, W64 = _bf16_exact(rng, (N, K))
    X, X64 = _bf16_exact(rng, (M, K))
    resid = rng.standard_normal((M, K)) * 3.0
    ss = np.zeros((K // 16, 32))
    ss[:, :M] = (resid ** 2).reshape(M, K // 16, 16).sum(axis=-1).T
    eps = 1e-6
    r = 1.0 / np.sqrt(ss[:, :M].sum(axis=0) / K + eps)
    scratch = torch.zeros(nc.nc_op_few_rows_scratch_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    ssq_in = torch.from_numpy(ss.astype(np.float32)).cuda()
    nc.nc_op_few_rows_gemm(0, W, K, X, K, C, N, M, N, K, scratch, ssq_in=ssq_in, eps=eps, ntile=ntile)
    ref = r[:, None] * (X64 @ W64.T)
    torch.cuda.synchronize()
    got = C.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= 2 ** -7 * np.abs(ref) + 1e-5 * np.abs(ref).max())
    # residual add with the bf16 copy and the sums of squares
    base = rng.standard_normal((M, N)).astype(np.float32)
    Cf = torch.from_numpy(base).cuda()
    xb = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    ssq_out = torch.full(((N // 16), 32), -1.0, dtype=torch.float32, device="cuda")
    nc.nc_op_few_rows_gemm(1, W, K, X, K, Cf, N, M, N, K, scratch, xb=xb, ssq_out=ssq_out, ntile=ntile)
    torch.cuda.synchronize()
    new = Cf.double().cpu().numpy()
    assert max_rel(new, base + X64 @ W64.T) <= 1e-5
    assert torch.equal(xb, Cf.to(torch.bfloat16))
    so = ssq_out.double().cpu().numpy()
    want = (new ** 2).reshape(M, N // 16, 16).sum(axis=-1).T
    assert max_rel(so[:, :M], want) <= 1e-5
    assert np.all(so[:, M:] == -1.0)


def _unit_rms(a):
    return a / np.sqrt(np.mean(a ** 2, axis=-1, keepdims=True))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,pos", [(1, 1, 0), (3, 10, 63), (2, 16, 64), (5, 3, 100), (32, 10, 1000),
                                     (4, 10, 2047)])
def test_decode_attention(dtype, B, H, pos):
    """One query row per sequence over cache positions 0..pos against the
    fp64 softmax; cache rows past pos hold NaN and must not reach the result."""
    max_seq = 2048
    rng = np.random.default_rng(B * 100 + H * 7 + pos)
    et = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = 128 * H
    ldq = d + 256
    q = _unit_rms(rng.standard_normal((B, H, 128)))
    kh = _unit_rms(rng.standard_normal((B, max_seq, 128)))
    v = rng.standard_normal((B, max_seq, 128))
    qkv = np.zeros((B, ldq))
    qkv[:, :d] = q.reshape(B, d)
    cache = np.concatenate([kh, v], axis=-1)
    cache[:, pos + 1:] = np.nan
    qkv_d = torch.from_numpy(qkv).to(et).cuda()
    cache_d = torch.from_numpy(cache).to(et).cuda()
    q64 = qkv_d.double().cpu().numpy()[:, :d].reshape(B, H, 128)
    c64 = cache_d.double().cpu().numpy()
    nch = pos // 64 + 1
    part = torch.empty(B * nch * H * 129, dtype=torch.float32, device="cuda")
    o = torch.full((B, d + 8), 3.0, dtype=et, device="cuda")
    nc.nc_op_decode_attn(dtype, qkv_d, ldq, B, H, cache_d, max_seq, pos, part, o, d + 8)
    torch.cuda.synchronize()
    got = o.double().cpu().numpy()
    assert np.all(got[:, d:] == 3.0)
    s = np.einsum("bhc,buc->bhu", q64, c64[:, :pos + 1, :128]) / np.sqrt(128.0)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    ref = np.einsum("bhu,buc->bhc", p, c64[:, :pos + 1, 128:]).reshape(B, d)
    got = got[:, :d]
    assert np.all(np.isfinite(got))
    if dtype == "f32":
        assert max_rel(got, ref) <= 1e-5, max_rel(got, ref)
    else:
        # P is rounded to bf16 before the P V product, the output once more
        assert np.abs(got - ref).max() <= 2e-2 * np.abs(ref).max(), np.abs(got - ref).max()
        check_bf16(got, ref, "o")
