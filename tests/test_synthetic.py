"""Seeded input generators: determinism, shapes and the distributions the
workloads call for."""
import numpy as np

from ternary_weight_linear_fwd_amd import synthetic as S


def test_c1_deterministic_and_shaped():
    W, x = S.c1_inputs()
    W2, x2 = S.c1_inputs()
    assert W.shape == (2048, 2048) and x.shape == (1, 2048)
    assert W.dtype == np.float32 and x.dtype == np.float32
    assert np.array_equal(W, W2) and np.array_equal(x, x2)
    assert abs(float(W.std()) - 0.02) < 2e-4


def test_block_shapes():
    assert [(p.K, p.N) for p in S.C2_PROJS] == [(3200, 3200)] * 4 + [(3200, 8640)] * 2 + [(8640, 3200)]
    assert [(p.K, p.N) for p in S.C4_PROJS] == [(8192, 8192), (8192, 1024), (8192, 1024), (8192, 8192),
                                                (8192, 28672), (8192, 28672), (28672, 8192)]
    total = S.C4_LAYERS * sum(p.N * p.K for p in S.C4_PROJS)
    assert total == 68_451_041_280
    assert total // 4 == 17_112_760_320


def test_c5_ternary_distribution():
    p = S.C5_PROJS[0]
    Wt, g = S.c5_ternary(p)
    assert Wt.shape == (4096, 4096) and 0.01 <= float(g) <= 0.05
    n = Wt.size
    for v, prob in ((0, 0.6), (1, 0.2), (-1, 0.2)):
        se = (prob * (1 - prob) / n) ** 0.5
        assert abs(float((Wt == v).mean()) - prob) < 5 * se


def test_c5_outliers():
    p = S.C5_PROJS[6]
    ch = S.c5_outlier_channels(p)
    assert len(ch) == 110 and len(set(ch.tolist())) == 110
    x = S.c5_x(p, 32)
    base = S.activations_normal(5, 0, p.index, 32, p.K)
    assert np.array_equal(x[:, ch], base[:, ch] * np.float32(20))
    mask = np.ones(p.K, bool)
    mask[ch] = False
    assert np.array_equal(x[:, mask], base[:, mask])


def test_c3_student_t():
    W, x = S.c3_inputs(0)
    assert W.shape == (8640, 3200) and x.shape == (2048, 3200)
    # heavy tails: kurtosis of t(3) is infinite; the sample max is far beyond a normal's
    assert float(np.abs(x).max()) > 20
