"""GPU parity: the absmedian weight scale (radix select of the two middle
magnitudes) and the packing that uses it, bit-exact against the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import bl, empty, say, to_dev, torch_cuda, unpack
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def pack_absmedian(W: np.ndarray):
    torch_cuda()
    L = bl()
    N, K = W.shape
    packed = empty(L.bitlinear_packed_bytes(N, K))
    ws_bytes = L.bitlinear_workspace_bytes(0, N, K)
    ws = empty(ws_bytes)
    g = ctypes.c_float()
    L.bitlinear_pack_weights_absmedian(to_dev(W.astype(np.float32)), N, K, packed, None, g, ws,
                                       ws_bytes)
    return packed, np.float32(g.value)


def check(W: np.ndarray):
    N, K = W.shape
    say(f"absmedian N={N} K={K}")
    packed, g = pack_absmedian(W)
    Wt_ref, g_ref = oracle.quantize_weights_absmedian(W)
    assert g.view(np.uint32) == g_ref.view(np.uint32), (g, g_ref)
    back, bad = unpack(packed, N, K)
    assert bad == 0 and np.array_equal(back, Wt_ref)


@pytest.mark.parametrize("N,K", [(1, 16), (3, 16), (5, 48), (64, 64), (100, 320), (333, 1040)])
def test_shapes(N, K):
    check(S.random_latent(N * 7 + K, N, K))


def test_structured_inputs():
    rng = np.random.default_rng(8)
    W = (rng.standard_t(2, (50, 96))).astype(np.float32)        # heavy tails
    check(W)
    W = rng.choice(np.array([0.0, 0.25, -0.25, 1.0], np.float32), size=(40, 64))
    check(W)                                                      # many ties
    W[:, :40] = 0
    check(W)                                                      # mostly zeros
    check(np.full((8, 32), -0.375, np.float32))                   # constant
    check(np.zeros((4, 16), np.float32))                          # clamp
    W = (rng.standard_normal((30, 80)) * np.exp2(rng.integers(-60, 60, (30, 80)))).astype(np.float32)
    check(W)                                                      # wide exponent range
    # middle pair whose mean is a float32 tie
    W = np.array([[1.0] * 8 + [1 + 2.0 ** -23] * 8] + [[0.25] * 8 + [4.0] * 8], np.float32)
    check(W)


def test_config_shapes():
    W, _ = S.c1_inputs()
    check(W)
    W, _ = S.c3_inputs(0)
    check(W)
