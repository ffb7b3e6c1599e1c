"""GPU parity: per-token absmax INT8 activation quantization, bit-exact against
the oracle (xq, eta and the row sums)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import near_tie_rows, quantize, say
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def check(x):
    say(f"quantize M={x.shape[0]} K={x.shape[1]}")
    xq, eta, xsum = quantize(x)
    rq, reta = oracle.quantize_act(x)
    assert np.array_equal(eta.view(np.uint32), reta.view(np.uint32))
    assert np.array_equal(xq, rq), np.argwhere(xq != rq)[:5]
    assert np.array_equal(xsum, rq.astype(np.int64).sum(axis=1))


@pytest.mark.parametrize("M,K", [(1, 16), (1, 48), (3, 80), (2, 1024), (5, 1040), (1, 2048),
                                 (7, 4096), (2, 8192), (3, 8208), (1, 16384), (2, 28672),
                                 (1, 32784)])
def test_shapes(M, K):
    check(S.random_x(M * 100003 + K, M, K))


def test_config_shapes():
    _, x = S.c1_inputs()
    check(x)
    for M in (1, 8):
        check(S.c2_x(S.C2_PROJS[0], M))
        check(S.c2_x(S.C2_PROJS[6], M))
    for p in (0, 1):
        _, x = S.c3_inputs(p)
        check(x)
    for M in (1, 16):
        check(S.c4_x(0, S.C4_PROJS[0], M))
        check(S.c4_x(0, S.C4_PROJS[6], M))
    for M in (32, 128):
        check(S.c5_x(S.C5_PROJS[0], M))
        check(S.c5_x(S.C5_PROJS[6], M))


def test_edge_values():
    x = np.zeros((4, 64), np.float32)
    x[1, :8] = [127, 62.5, 63.5, -0.5, 0.5, 1.5, 2.5, -2.5]   # ties to even
    x[2, :4] = [5e-6, -2.5e-6, 1e-7, 0.0]                     # below the 1e-5 floor
    x[3] = np.float32(2.0) ** np.arange(-32, 32).astype(np.float32)  # wide range
    x[3, ::2] *= -1
    check(x)
    check(np.full((2, 32), -3.0, np.float32))                  # argmax negative
    check(np.array([[2.0 ** -140] * 16], np.float32))          # subnormals


def test_op_order_cases():
    # inputs where dividing first would round differently (see the oracle pins)
    rows = [(5.2772126, -4.466932), (7.6121526, 4.2855816), (2.7765708, 2.1316192),
            (1.1328796, 0.084742956), (3.7839653, -3.5307078)]
    x = np.zeros((len(rows), 16), np.float32)
    for i, (e, v) in enumerate(rows):
        x[i, 0], x[i, 1] = e, v
    check(x)


def test_empty_rows():
    from gpu_helpers import bl, torch_cuda
    torch = torch_cuda()
    x = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    xq = torch.full((1, 64), 7, dtype=torch.int8, device="cuda")
    eta = torch.full((1,), 3.0, dtype=torch.float32, device="cuda")
    bl().bitlinear_quantize_act(x, 0, 64, xq, eta)   # M = 0: nothing written
    torch.cuda.synchronize()
    assert int(xq[0, 0]) == 7 and float(eta[0]) == 3.0


def test_near_ties():
    # the stand-alone quantizer
    x = near_tie_rows()
    check(x)
    check(-x)


def test_near_ties_fused_forward():
    # the fused decode quantizes inside each workgroup: same rows, one and two
    # tokens at a time, y compared bit for bit with the oracle's forward
    from gpu_helpers import forward_f32, pack_weights
    x = near_tie_rows()
    M_all, K = x.shape
    N = 192
    W = S.random_latent(77, N, K)
    packed, g = pack_weights(W)
    Wt, g_ref = oracle.quantize_weights(W)
    assert g == g_ref
    for m0, m in ((0, 1), (1, 2), (3, 2), (5, 1)):
        xs = x[m0:m0 + m]
        say(f"near-tie fused forward rows {m0}..{m0 + m - 1} K={K}")
        y = forward_f32(xs, packed, g, N)
        y_ref, _, _, _ = oracle.forward(xs, Wt, g_ref)
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))
