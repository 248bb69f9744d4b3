"""The count-sketch used by the large-workload parity tests: numpy and torch
give the same sketch, it is linear, and its cosine / relative-L2 estimates
match the exact whole-vector values on gradient-like vectors."""
import numpy as np
import pytest

from tests import sketch


def test_numpy_torch_agree_and_linear():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    g = rng.standard_normal(300_001)
    first = 123_456_789
    a = sketch.sketch_np(g, first)
    b = sketch.sketch_torch(torch.from_numpy(g), first).numpy()
    assert np.allclose(a, b, rtol=0, atol=1e-9)
    h = rng.standard_normal(g.size)
    assert np.allclose(sketch.sketch_np(g - 2 * h, first),
                       a - 2 * sketch.sketch_np(h, first), atol=1e-9)
    # the chunked loop covers a tensor larger than one chunk
    big = rng.standard_normal(sketch.CHUNK + 17).astype(np.float32)
    c = sketch.sketch_np(big, 7)
    d = sketch.sketch_torch(torch.from_numpy(big), 7).numpy()
    assert np.allclose(c, d, rtol=0, atol=1e-6)


@pytest.mark.parametrize("shape,seed", [((1536, 1280), 1), ((5000, 768), 2), ((65536, 64), 3)])
def test_estimates_match_exact(shape, seed):
    rng = np.random.default_rng(seed)
    n = shape[0] * shape[1]
    # heavy-ish rows (like a gradient whose rows differ in scale) plus a small error
    o = (rng.standard_normal(shape) * rng.gamma(1.0, 1.0, (shape[0], 1))).ravel()
    for rel in (1e-3, 1e-2, 3e-2):
        g = o + rel * np.linalg.norm(o) / np.sqrt(n) * rng.standard_normal(n)
        first = int(rng.integers(0, 1 << 29))
        cos_e, rl2_e = sketch.cosine_rel_l2(sketch.sketch_np(g, first), sketch.sketch_np(o, first))
        rl2 = np.linalg.norm(g - o) / np.linalg.norm(o)
        cos = g @ o / (np.linalg.norm(g) * np.linalg.norm(o))
        assert abs(rl2_e - rl2) <= 0.08 * rl2, (rel, rl2_e, rl2)
        assert abs((1 - cos_e) - (1 - cos)) <= 0.16 * (1 - cos) + 1e-9, (rel, cos_e, cos)
