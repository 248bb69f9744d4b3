"""The persistent schedule of the 256x256 bf16 contraction kernel: for
whole-tile products that are not split over K and have more tiles than the
device has compute units, one workgroup per compute unit walks its XCD's
tiles and requests each next tile's first operand slabs before it runs the
current tile's epilogue. The tiles, their order and the arithmetic are those
of the one-workgroup-per-tile launch, so the two launches must agree bitwise;
sampled output rows are also checked against float64 products (the
one-workgroup-per-tile launch itself meets the float64 products element by
element in test_gpu_ops.py). Shapes: 2 tiles per workgroup at K of 2, 4 and
10 slabs of 32 (the shortest main loop, one as deep as the ring, one that
refills it), 1-2 tiles per workgroup over five column tiles, 4 per workgroup
over 64 column tiles, 257 tiles in one column (0-2 per workgroup: part of
the last XCD's workgroups find no tile and return), and a batched
alpha*AB^T + beta*C2 product."""
import numpy as np
import pytest

from tests.gpu_util import bf16_dev, host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dense_gpt_pretraining_nanochat_amd as nc  # noqa: E402

EPIS = [nc.EPI_STORE_T, nc.EPI_STORE_F32, nc.EPI_ADD_F32, nc.EPI_RELU2, nc.EPI_RELU2_BWD]
SHAPES = [(8192, 4096, 64), (8192, 4096, 128), (8192, 4096, 320), (16384, 1280, 256),
          (4096, 16384, 192), (65792, 256, 128)]
ROWS = 24


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    nc.nc_set_gemm_persistent(True)


def _run(persistent, dtype_out_f32, ak, bk, epi, A, B, C0, C2, M, N, K):
    nc.nc_set_gemm_persistent(persistent)
    C = C0.clone()
    nc.nc_op_gemm("bf16", ak, bk, epi, A, B, C, C2, M, N, K, K if ak else M, K if bk else N, N)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("ak,bk", [(1, 1), (1, 0), (0, 0), (0, 1)])
@pytest.mark.parametrize("epi", EPIS)
def test_persistent_matches_per_tile_launch(M, N, K, ak, bk, epi):
    rng = np.random.default_rng(M + N + K + 10 * ak + 20 * bk + 100 * epi)
    A = bf16_dev(rng.standard_normal((M, K) if ak else (K, M)))
    B = bf16_dev(rng.standard_normal((N, K) if bk else (K, N)))
    out_f32 = epi in (nc.EPI_STORE_F32, nc.EPI_ADD_F32)
    g = torch.Generator(device="cuda")
    g.manual_seed(M * 3 + K)
    if out_f32:
        C0 = (torch.randn((M, N), generator=g, device="cuda") if epi == nc.EPI_ADD_F32
              else torch.zeros((M, N), dtype=torch.float32, device="cuda"))
    else:
        C0 = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    C2 = None
    if epi == nc.EPI_RELU2_BWD:
        C2 = torch.relu(torch.randn((M, N), generator=g, device="cuda")).square().to(torch.bfloat16)
    per_tile = _run(False, out_f32, ak, bk, epi, A, B, C0, C2, M, N, K)
    persistent = _run(True, out_f32, ak, bk, epi, A, B, C0, C2, M, N, K)
    assert torch.equal(persistent, per_tile), (M, N, K, ak, bk, epi)
    # sampled rows against float64 (first and last tile rows among them)
    rows = np.unique(np.concatenate([[0, 255, M - 1], rng.integers(0, M, ROWS)]))
    ri = torch.from_numpy(rows).cuda()
    A64, B64 = host64(A), host64(B)
    Am = A64[rows] if ak else A64[:, rows].T
    Bm = B64 if bk else B64.T
    ref = Am @ Bm.T
    if epi == nc.EPI_ADD_F32:
        ref = ref + host64(C0[ri])
    if epi == nc.EPI_RELU2:
        ref = np.maximum(ref, 0.0) ** 2
    if epi == nc.EPI_RELU2_BWD:
        ref = ref * 2.0 * np.sqrt(host64(C2[ri]))
    got = host64(persistent[ri])
    if out_f32:
        assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref).max())
    else:
        assert np.all(np.abs(got - ref) <= 2 ** -7 * np.abs(ref) + 1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("out_f32", [0, 1])
def test_persistent_batched_axpby(out_f32):
    """12 items of 1280 x 1280 (300 tiles over the batch), K = 256, both output
    types: persistent and per-tile launches agree bitwise, sampled rows of
    items 0 and 11 match float64."""
    batch, M, N, K = 12, 1280, 1280, 256
    rng = np.random.default_rng(77 + out_f32)
    A = bf16_dev(rng.standard_normal((batch, M, K)))
    B = bf16_dev(rng.standard_normal((batch, N, K)))
    C2 = bf16_dev(rng.standard_normal((batch, M, N)))
    alpha, beta = 2.0315, 3.4445
    outs = []
    for persistent in (False, True):
        nc.nc_set_gemm_persistent(persistent)
        C = torch.zeros((batch, M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        nc.nc_op_gemm_axpby("bf16", 1, 1, out_f32, A, B, C, C2, M, N, K, K, K, N, alpha, beta,
                            batch=batch, sa=M * K, sb=N * K, sc=M * N, tile=256)
        torch.cuda.synchronize()
        outs.append(C)
    assert torch.equal(outs[0], outs[1])
    rows = np.array([0, 1, 255, 256, 700, M - 1])
    for b in (0, batch - 1):
        A64, B64, C264 = host64(A[b]), host64(B[b]), host64(C2[b])
        ref = alpha * (A64[rows] @ B64.T) + beta * C264[rows]
        got = host64(outs[1][b])[rows]
        if out_f32:
            assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref).max())
        else:
            assert np.all(np.abs(got - ref) <= 2 ** -7 * np.abs(ref) + 1e-5 * np.abs(ref).max())

