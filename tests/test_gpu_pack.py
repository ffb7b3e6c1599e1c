"""GPU parity: absmean gamma (bit-exact), ternarization (via unpack, bit-exact),
packing round trips and the handling of invalid codes."""
import numpy as np
import pytest

import oracle
from gpu_helpers import pack_ternary, pack_weights, say, to_dev, unpack
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def check_pack(W):
    N, K = W.shape
    say(f"pack N={N} K={K}")
    packed, g = pack_weights(W)
    Wt_ref, g_ref = oracle.quantize_weights(W)
    assert g.view(np.uint32) == g_ref.view(np.uint32), (g, g_ref)
    Wt, bad = unpack(packed, N, K)
    assert bad == 0
    assert np.array_equal(Wt, Wt_ref), np.argwhere(Wt != Wt_ref)[:5]
    return packed, g


@pytest.mark.parametrize("N,K", [(1, 16), (3, 48), (64, 64), (65, 80), (100, 208), (127, 1040),
                                 (300, 4096)])
def test_random_shapes(N, K):
    check_pack(S.random_latent(N * 7919 + K, N, K))


def test_config_weights():
    W, _ = S.c1_inputs()
    check_pack(W)
    check_pack(S.c2_weight(S.C2_PROJS[4]))   # gate 3200 -> 8640
    W, _ = S.c3_inputs(1)                    # 8640 -> 3200
    check_pack(W)


def test_gamma_special_cases():
    u = 2.0 ** -23
    for W in (np.array([[0.5, -0.5, 1.5, -1.5] * 4], np.float32),       # mean exactly 1
              np.array([[1.0, 1.0 + u] * 8], np.float32),               # tie -> even
              np.array([[1.0 + u, 1.0 + 2 * u] * 8], np.float32),       # tie -> even (up)
              np.array([[2.0, u + 2.0 ** -40] * 8], np.float32),        # sticky tail decides
              np.zeros((2, 16), np.float32),                            # clamp to 1e-5
              np.full((1, 16), 2.0 ** -149, np.float32),                # subnormals
              np.array([[3e38, 1.0, 1e-30, 2.5e-45] * 4], np.float32),  # wide range
              (np.float32(2.0) ** np.random.default_rng(3).integers(-140, 120, (9, 32)).astype(np.float32))):
        check_pack(W)


def test_ternary_thresholds():
    # W/gamma landing exactly on +-0.5 rounds to 0; just above rounds to +-1
    rng = np.random.default_rng(4)
    W = rng.standard_normal((64, 256), dtype=np.float32) * np.float32(0.02)
    g = oracle.absmean_gamma(W)
    W[0, :4] = [g * np.float32(0.5), -g * np.float32(0.5), np.nextafter(g * np.float32(0.5), np.float32(1)), 0]
    check_pack(W)


def test_pack_ternary_roundtrip_and_bad_codes():
    Wt, _ = S.c5_ternary(S.C5_PROJS[1])
    packed, bad = pack_ternary(Wt)
    assert bad == 0
    back, bad = unpack(packed, *Wt.shape)
    assert bad == 0 and np.array_equal(back, Wt)
    # canonical bytes agree with the oracle's packing, word by word
    canon = oracle.pack(Wt[:64, :64])
    got = np.asarray(packed.cpu().numpy()[:1024]).reshape(64, 16)  # block (0, 0)
    for r in range(64):
        for d in range(4):
            word = int.from_bytes(bytes(got[r, 4 * d:4 * d + 4]), "little")
            for q in range(16):
                k = 16 * d + q
                code = (word >> (8 * (q % 4) + 2 * (q // 4))) & 3
                assert code == (int(canon[r, k // 4]) >> (2 * (k % 4))) & 3
    bad_in = np.zeros((2, 32), np.int8)
    bad_in[0, 3] = 2
    bad_in[1, 7] = -5
    packed, bad = pack_ternary(bad_in)
    assert bad == 2
    back, _ = unpack(packed, 2, 32)
    assert back[0, 3] == 0 and back[1, 7] == 0


def test_unpack_reports_code_11():
    from gpu_helpers import torch_cuda
    torch = torch_cuda()
    N, K = 64, 64
    packed = torch.full((1024,), 0x55, dtype=torch.uint8, device="cuda")
    packed[0] = 0xFF     # four 11 codes in row 0
    Wt, bad = unpack(packed, N, K)
    assert bad == 4 and not Wt.any()
