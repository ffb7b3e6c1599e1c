"""GPU parity: the compact base-3 weight format (device layout, packing,
unpacking) and the lookup-table contraction over both weight formats,
bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
from gpu_helpers import bl, empty, pack_ternary, pack_weights, say, to_dev, torch_cuda
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def device_layout3(canon: np.ndarray, N: int, K: int) -> np.ndarray:
    """The documented base-3 device layout, built on the host from the oracle's
    canonical bytes: block (g, b) holds 16 bytes per row, byte p of row r being
    canonical byte 16b + p of row 64g + r; everything else is weight 0."""
    G, Kb3 = -(-N // 64), -(-K // 80)
    out = np.full((G * 64, Kb3 * 16), 121, np.uint8)
    out[:N, :canon.shape[1]] = canon
    return out.reshape(G, 64, Kb3, 16).transpose(0, 2, 1, 3).ravel()


def pack3_ternary(Wt: np.ndarray):
    torch = torch_cuda()
    L = bl()
    N, K = Wt.shape
    packed = empty(L.bitlinear_packed3_bytes(N, K))
    bad = torch.full((1,), 7, dtype=torch.int32, device="cuda")   # the call sets it
    L.bitlinear_pack_ternary3(to_dev(Wt.astype(np.int8)), N, K, packed, bad)
    torch.cuda.synchronize()
    return packed, int(bad.cpu()[0])


def unpack3(packed, N: int, K: int):
    torch = torch_cuda()
    Wt = torch.empty((N, K), dtype=torch.int8, device="cuda")
    bad = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    bl().bitlinear_unpack_weights3(packed, N, K, Wt, bad)
    torch.cuda.synchronize()
    return Wt.cpu().numpy(), int(bad.cpu()[0])


@pytest.mark.parametrize("N,K", [(1, 16), (5, 80), (63, 96), (64, 160), (65, 1040), (200, 3200),
                                 (129, 8208)])
def test_base3_layout_and_roundtrip(N, K):
    say(f"base-3 pack N={N} K={K}")
    Wt = S.random_ternary(31 * N + K, N, K)
    packed, bad = pack3_ternary(Wt)
    assert bad == 0
    L = bl()
    assert L.bitlinear_packed3_bytes(N, K) == packed.numel() or packed.numel() == 256
    dev = packed.cpu().numpy()[:L.bitlinear_packed3_bytes(N, K)]
    assert np.array_equal(dev, device_layout3(oracle.pack3(Wt), N, K))
    back, bad = unpack3(packed, N, K)
    assert bad == 0 and np.array_equal(back, Wt)


def test_base3_bad_inputs():
    N, K = 70, 160
    Wt = S.random_ternary(5, N, K)
    Wt[3, 7] = 2
    Wt[69, 159] = -5
    packed, bad = pack3_ternary(Wt)
    assert bad == 2
    fixed = Wt.copy()
    fixed[3, 7] = 0
    fixed[69, 159] = 0
    back, bad = unpack3(packed, N, K)
    assert bad == 0 and np.array_equal(back, fixed)
    # an out-of-range byte inside the matrix decodes as zero weights and is counted
    raw = packed.cpu().numpy()
    raw[16 * 5 + 2] = 250          # row 5, block 0, byte 2: k = 10..14
    back, bad = unpack3(to_dev(raw), N, K)
    assert bad == 1
    fixed[5, 10:15] = 0
    assert np.array_equal(back, fixed)


def test_pack_weights3_latent():
    torch = torch_cuda()
    L = bl()
    for N, K in ((100, 320), (333, 1040)):
        W = S.random_latent(11 * N + K, N, K)
        Wt_ref, g_ref = oracle.quantize_weights(W)
        packed = empty(L.bitlinear_packed3_bytes(N, K))
        ws_bytes = L.bitlinear_workspace_bytes(0, N, K)
        ws = empty(ws_bytes)
        import ctypes
        g = ctypes.c_float()
        L.bitlinear_pack_weights3(to_dev(W), N, K, packed, None, g, ws, ws_bytes)
        assert np.float32(g.value) == g_ref
        back, bad = unpack3(packed, N, K)
        assert bad == 0 and np.array_equal(back, Wt_ref)


def forward_lut(xq, eta, packed, fmt, gamma, N):
    torch = torch_cuda()
    L = bl()
    M, K = xq.shape
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_int = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws_bytes = L.bitlinear_lut_workspace_bytes(M, N, K, fmt)
    ws = empty(ws_bytes)
    L.bitlinear_forward_lut(to_dev(xq), to_dev(eta), packed, fmt, float(gamma), M, N, K, y, y_int,
                            ws, ws_bytes)
    torch.cuda.synchronize()
    return y.cpu().numpy(), y_int.cpu().numpy()


def check_lut(M, N, K, seed, dist="normal"):
    L = bl()
    x = S.random_x(seed, M, K, dist)
    Wt = S.random_ternary(seed + 1, N, K)
    gamma = np.float32(0.0173)
    xq, eta = oracle.quantize_act(x)
    y_ref, yi_ref = oracle.forward_q(xq, eta, Wt, gamma, threads=8)
    p2, _ = pack_ternary(Wt)
    p3, _ = pack3_ternary(Wt)
    for fmt, packed in ((L.BITLINEAR_FORMAT_2BIT, p2), (L.BITLINEAR_FORMAT_BASE3, p3)):
        say(f"forward_lut fmt={fmt} M={M} N={N} K={K}")
        y, yi = forward_lut(xq, eta, packed, fmt, gamma, N)
        assert np.array_equal(yi, yi_ref), np.argwhere(yi != yi_ref)[:5]
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9])
def test_lut_token_counts(M):
    check_lut(M, 200, 208, seed=700 + M)


@pytest.mark.parametrize("N,K", [(1, 16), (63, 80), (64, 96), (65, 160), (257, 1040),
                                 (1000, 4160), (2049, 336), (4100, 8208)])
def test_lut_shapes(N, K):
    check_lut(1, N, K, seed=900 + N + K)


def test_lut_config_shapes():
    # decode projections of the 3B and 70B shapes, one token
    for K, N in ((3200, 8640), (8640, 3200), (8192, 28672), (28672, 8192)):
        check_lut(1, N, K, seed=K + N, dist="t3")


def test_lut_extreme_activations():
    # int8 extremes including -128 (the tables stay within int16)
    L = bl()
    M, N, K = 2, 130, 400
    rng = np.random.default_rng(3)
    xq = rng.choice(np.array([-128, -127, 127, 0], np.int8), size=(M, K))
    eta = np.array([1.0, 2.5], np.float32)
    Wt = S.random_ternary(4, N, K)
    y_ref, yi_ref = oracle.forward_q(xq, eta, Wt, np.float32(0.5))
    for fmt, packed in ((L.BITLINEAR_FORMAT_2BIT, pack_ternary(Wt)[0]),
                        (L.BITLINEAR_FORMAT_BASE3, pack3_ternary(Wt)[0])):
        y, yi = forward_lut(xq, eta, packed, fmt, np.float32(0.5), N)
        assert np.array_equal(yi, yi_ref) and np.array_equal(y, y_ref)
