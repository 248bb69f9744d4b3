"""nc_op_attn_bwd_noalloc (attention backward with the library's fixed
per-device scratch, for callers that cannot allocate) against the existing
nc_op_attn_bwd with caller scratch: two calls in a row, the second smaller,
each bitwise equal to the reference call (the same kernels); the first also
against the fp64 oracle to the per-kernel bar; a size beyond the fixed array
is refused before anything runs."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import bf16_dev, check_bf16, dev, host64, max_rel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_gpt_pretraining_nanochat_amd as nc  # noqa: E402


def _inputs(rng, B, T, H, dtype):
    """qkv with unit-RMS query / key heads (as rotary + QK-norm leave them),
    the forward's o and lse, and a seeded upstream gradient."""
    d = 128 * H
    Q = d + 256
    M = B * T
    z = rng.standard_normal((M, H + 2, 128))
    z[:, :H + 1] /= np.sqrt(np.mean(z[:, :H + 1] ** 2, axis=-1, keepdims=True))
    et = torch.bfloat16 if dtype == "bf16" else torch.float32
    qkv = (bf16_dev(z.reshape(M, Q)) if dtype == "bf16" else dev(z.reshape(M, Q).astype(np.float32)))
    o = torch.zeros((M, d), dtype=et, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    nc.nc_op_attn_fwd(dtype, qkv, B, T, H, o, lse)
    g = rng.standard_normal((M, d))
    do = bf16_dev(g) if dtype == "bf16" else dev(g.astype(np.float32))
    return qkv, o, lse, do


def _reference(dtype, qkv, o, do, lse, B, T, H):
    d = 128 * H
    dq = torch.zeros((B * T, d + 256), dtype=qkv.dtype, device="cuda")
    delta = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    scratch = torch.empty(nc.nc_op_attn_bwd_scratch_bytes(B, T), dtype=torch.uint8, device="cuda")
    nc.nc_op_attn_bwd(dtype, qkv, o, do, lse, delta, B, T, H, dq, scratch)
    return dq


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_attn_bwd_matches_scratch_version(dtype):
    rng = np.random.default_rng(7 if dtype == "bf16" else 8)
    first = (1, 2560, 2)             # 2560 tokens: two 2048-query chunks for the first key blocks
    second = (1, 192, 3)             # smaller, dK/dV written directly; the array keeps old contents
    outs = []
    for (B, T, H) in (first, second):
        qkv, o, lse, do = _inputs(rng, B, T, H, dtype)
        dq_ref = _reference(dtype, qkv, o, do, lse, B, T, H)
        dq = torch.full_like(dq_ref, float("nan"))
        nc.nc_op_attn_bwd_noalloc(dtype, qkv, o, do, lse, B, T, H, dq)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq_ref), (dtype, B, T, H)
        outs.append((B, T, H, qkv, o, do, dq))
    # the first call's result against the fp64 oracle, per kernel bar
    B, T, H, qkv, o, do, dq = outs[0]
    d = 128 * H
    z = host64(qkv).reshape(B, T, d + 256)
    og = host64(o).reshape(B, T, H, 128)
    g = host64(dq).reshape(B, T, d + 256)
    for b in range(B):
        rq, rk, rv = oracle.causal_mqa_bwd(z[b, :, :d].reshape(T, H, 128), z[b, :, d:d + 128],
                                           z[b, :, d + 128:], og[b],
                                           host64(do).reshape(B, T, H, 128)[b])
        for got, ref, name in ((g[b, :, :d].reshape(T, H, 128), rq, "dq"),
                               (g[b, :, d:d + 128], rk, "dk"), (g[b, :, d + 128:], rv, "dv")):
            if dtype == "f32":
                assert max_rel(got, ref) <= 1e-4, name
            else:
                check_bf16(got, ref, name, cos_min=0.9999, l2_max=1.5e-2)


def test_noalloc_attn_bwd_refuses_sizes_beyond_the_array():
    """B = 4 sequences of 4096 tokens at 10 heads need 34.2 MB of scratch
    (delta and two query chunks of dK/dV partials; > 32 MiB): refused on the
    host, nothing enqueued. B = 3 (25.7 MB) runs and matches the scratch
    version bitwise."""
    B, T, H = 4, 4096, 10
    M, Q = B * T, 128 * H + 256
    qkv = torch.zeros((M, Q), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((M, 128 * H), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    dq = torch.zeros_like(qkv)
    with pytest.raises(nc.NcError) as e:
        nc.nc_op_attn_bwd_noalloc("bf16", qkv, o, o, lse, B, T, H, dq)
    assert e.value.code == -5
    assert int(torch.count_nonzero(dq).item()) == 0
    rng = np.random.default_rng(9)
    B = 3
    qkv, o, lse, do = _inputs(rng, B, T, H, "bf16")
    dq_ref = _reference("bf16", qkv, o, do, lse, B, T, H)
    dq = torch.zeros_like(dq_ref)
    nc.nc_op_attn_bwd_noalloc("bf16", qkv, o, do, lse, B, T, H, dq)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_ref)
