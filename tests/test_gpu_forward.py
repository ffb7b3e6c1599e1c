"""GPU parity of the contraction and dequant epilogue: int32 sums bit-exact,
float32 outputs within 1e-6 relative (and, with the same operation order,
identical), across every kernel variant, ragged tiles and edge cases."""
import numpy as np
import pytest

import oracle
from gpu_helpers import (assert_y_close, bl, forward, forward_f32, forward_xsum, pack_ternary, pack_weights,
                         say, to_dev, torch_cuda)
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def run_case(M, N, K, seed, dist="normal", latent=True):
    say(f"forward M={M} N={N} K={K} seed={seed}")
    x = S.random_x(seed, M, K, dist)
    if latent:
        W = S.random_latent(seed + 1, N, K)
        packed, g = pack_weights(W)
        Wt, g_ref = oracle.quantize_weights(W)
        assert g == g_ref
    else:
        Wt = S.random_ternary(seed + 1, N, K)
        g = np.float32(0.0173)
        packed, bad = pack_ternary(Wt)
        assert bad == 0
    xq, eta = oracle.quantize_act(x)
    y, y_int = forward(xq, eta, packed, g, N)
    y_ref, y_int_ref = oracle.forward_q(xq, eta, Wt, g, threads=8)
    assert np.array_equal(y_int, y_int_ref), np.argwhere(y_int != y_int_ref)[:5]
    assert_y_close(y, y_ref)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))
    # row sums supplied (the definition, sum over k of xq): the same bits
    xsum = xq.astype(np.int64).sum(axis=1)
    y3, y_int3 = forward_xsum(xq, eta, xsum, packed, g, N)
    assert np.array_equal(y_int3, y_int_ref), np.argwhere(y_int3 != y_int_ref)[:5]
    assert np.array_equal(y3.view(np.uint32), y_ref.view(np.uint32))
    # fused path from float32 activations
    yf = forward_f32(x, packed, g, N)
    assert_y_close(yf, y_ref)


# Every token count class: dot4 path (1..4), MFMA with 1, 2 and 4 M-tiles per
# wave (<=16, <=32, <=64) and the 128-row prefill tiles (> 64), each with
# ragged N (not a multiple of 64 or of the column tile) and K (tail blocks).
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16, 17, 32, 33, 64, 65, 128, 130, 257])
def test_token_counts(M):
    run_case(M, 200, 208, seed=1000 + M)


@pytest.mark.parametrize("N,K", [(1, 16), (63, 32), (64, 48), (65, 64), (129, 80), (256, 1024),
                                 (333, 1040), (1000, 4160)])
@pytest.mark.parametrize("M", [1, 4, 16, 96])
def test_ragged_shapes(M, N, K):
    run_case(M, N, K, seed=M * 131 + N * 7 + K)


# Up to four tokens: the fused kernel (one workgroup per 64-row group, K split
# among its wavefronts) where each wavefront's run is short, the split GEMV
# and its epilogue where it is long; ragged N, K with a tail block, both
# paths from int8 and from float32.
@pytest.mark.parametrize("M,N,K", [(1, 2065, 4160), (2, 2065, 4160), (1, 2100, 4144), (2, 100, 1040),
                                   (2, 300, 8208), (1, 4096, 16400), (3, 2065, 4160), (4, 2100, 4144),
                                   (4, 28672, 8192), (4, 300, 8208), (3, 1000, 1040)])
def test_fused_and_split_decode(M, N, K):
    run_case(M, N, K, seed=7 * M + N + K)


def test_heavy_tails_and_direct_ternary():
    run_case(64, 512, 1024, seed=5, dist="t3")
    run_case(3, 777, 528, seed=6, latent=False)
    run_case(128, 384, 2048, seed=7, latent=False)


def test_extreme_sums():
    # every xq = +-127 and every weight +-1: |y_int| = 127 * K, the largest magnitude
    M, N, K = 4, 128, 28672
    x = np.ones((M, K), np.float32)
    x[1] *= -1
    x[2, ::2] = -1
    Wt = np.ones((N, K), np.int8)
    Wt[1::2] = -1
    packed, _ = pack_ternary(Wt)
    xq, eta = oracle.quantize_act(x)
    for m in (4, 16, 64):
        xqm = np.resize(xq, (m, K)).astype(np.int8)
        etam = np.resize(eta, m).astype(np.float32)
        y, y_int = forward(xqm, etam, packed, np.float32(1.0), N)
        ref = oracle.ternary_contract(xqm, Wt, threads=8)
        assert np.array_equal(y_int, ref)
        assert np.abs(ref).max() == 127 * K


def test_zero_inputs():
    M, N, K = 8, 64, 64
    packed, g = pack_weights(np.zeros((N, K), np.float32))
    assert g == np.float32(1e-5)
    xq, eta = oracle.quantize_act(np.zeros((M, K), np.float32))
    y, y_int = forward(xq, eta, packed, g, N)
    assert not y_int.any() and not y.any()


def test_determinism():
    M, N, K = 2, 8192, 8192   # split-K path
    x = S.random_x(11, M, K)
    Wt = S.random_ternary(12, N, K)
    packed, _ = pack_ternary(Wt)
    xq, eta = oracle.quantize_act(x)
    a = forward(xq, eta, packed, 0.02, N)
    b = forward(xq, eta, packed, 0.02, N)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


# Prefill grids many rounds deep (thousands of tiles), with ragged M, N and K;
# on a 256-CU chip (1000, 32700) takes 128 x 256 tiles, the others 64 x 256.
@pytest.mark.parametrize("M,N,K", [(130, 33000, 80), (257, 32832, 208), (200, 65600, 48),
                                   (1000, 200000, 32), (1537, 131136, 16), (1000, 32700, 208)])
def test_prefill_tall_tiles(M, N, K):
    run_case(M, N, K, seed=M + N + K, latent=False)


# Shapes for which the prefill launch picks 96 x 384 tiles (3 x 3 MFMA tiles
# per wavefront) on a 256-CU chip: M not a multiple of 96, N not a multiple of
# 384 or of 32, K with partial and odd last blocks.
@pytest.mark.parametrize("M,N,K", [(772, 10000, 1040), (1927, 4100, 208), (2949, 2600, 80)])
def test_prefill_wide_tiles(M, N, K):
    run_case(M, N, K, seed=M * 3 + N + K, latent=False)



# Prefill shapes of the batched-decode and 3B workloads and a few ragged ones,
# each run twice (identical bits), checked row by row against the oracle (or
# on sampled rows plus exact int64 checksums of every row when large).
def test_prefill_workload_shapes():
    torch = torch_cuda()
    L = bl()
    shapes = [(128, 11008, 4096), (128, 4096, 11008), (832, 8192, 2560), (96, 1000, 4160),
              (130, 200, 208), (2048, 8640, 3200)]
    for i, (M, N, K) in enumerate(shapes):
        say(f"prefill shape M={M} N={N} K={K}")
        x = S.random_x(700 + i, M, K, "t3")
        Wt = S.random_ternary(800 + i, N, K)
        packed, bad = pack_ternary(Wt)
        assert bad == 0
        xq, eta = oracle.quantize_act(x)
        xq_d, eta_d = to_dev(xq), to_dev(eta)
        ws_bytes = L.bitlinear_workspace_bytes(M, N, K)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        outs = []
        for rep in range(2):
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            y_int = torch.empty((M, N), dtype=torch.int32, device="cuda")
            L.bitlinear_forward(xq_d, eta_d, packed, 0.0173, M, N, K, y, y_int, ws, ws_bytes)
            torch.cuda.synchronize()
            outs.append((y.cpu().numpy(), y_int.cpu().numpy()))
        (y, y_int), (y2, y_int2) = outs
        assert np.array_equal(y_int, y_int2) and np.array_equal(y.view(np.uint32), y2.view(np.uint32))
        y3, y_int3 = forward_xsum(xq, eta, xq.astype(np.int64).sum(axis=1), packed, 0.0173, N)
        assert np.array_equal(y_int, y_int3) and np.array_equal(y.view(np.uint32), y3.view(np.uint32))
        rows = np.arange(M) if M * N * K <= 6e9 else \
            np.sort(np.random.default_rng(i).choice(M, 48, replace=False))
        y_ref, y_int_ref = oracle.forward_q(xq[rows], eta[rows], Wt, np.float32(0.0173), threads=8)
        assert np.array_equal(y_int[rows], y_int_ref), np.argwhere(y_int[rows] != y_int_ref)[:5]
        assert_y_close(y[rows], y_ref)
        assert np.array_equal(y[rows].view(np.uint32), y_ref.view(np.uint32))
        # every row: exact int64 checksums
        r = np.random.default_rng(i).integers(-3, 4, N).astype(np.int64)
        x64 = xq.astype(np.int64)
        assert np.array_equal(y_int.astype(np.int64).sum(axis=1), x64 @ Wt.astype(np.int64).sum(axis=0))
        assert np.array_equal(y_int.astype(np.int64) @ r, x64 @ (Wt.astype(np.int64).T @ r))


# The prefill kernel reads the given row sums (and sums nothing itself): an
# offset d[m] in xsum[m] moves row m of y_int by exactly -d[m] (int32
# wrap-around arithmetic).  Decode sizes (M <= 64) ignore the argument.
@pytest.mark.parametrize("M,N,K", [(65, 300, 208), (200, 1000, 1040), (2048, 640, 80)])
def test_forward_xsum_is_read(M, N, K):
    say(f"forward_xsum offsets M={M} N={N} K={K}")
    x = S.random_x(M + N, M, K)
    Wt = S.random_ternary(M + K, N, K)
    packed, bad = pack_ternary(Wt)
    assert bad == 0
    xq, eta = oracle.quantize_act(x)
    y_ref, y_int_ref = oracle.forward_q(xq, eta, Wt, np.float32(0.02), threads=8)
    d = np.random.default_rng(M).integers(-1000, 1001, M).astype(np.int64)
    xsum = xq.astype(np.int64).sum(axis=1)
    _, y_int = forward_xsum(xq, eta, xsum + d, packed, 0.02, N)
    assert np.array_equal(y_int.astype(np.int64), y_int_ref.astype(np.int64) - d[:, None])
    # decode sizes: the argument is not read
    yq, y_intq = forward_xsum(xq[:16], eta[:16], xsum[:16] + d[:16], packed, 0.02, N)
    assert np.array_equal(y_intq, y_int_ref[:16])
    assert np.array_equal(yq.view(np.uint32), y_ref[:16].view(np.uint32))


# Every call only queues work on the stream it is given: the fused forward on
# two non-default streams at once (decode split-K, streaming MFMA and prefill
# sizes, each with its own workspace), while a third stream is kept busy,
# gives the same bits as the default stream.
def test_non_default_streams():
    torch = torch_cuda()
    L = bl()
    N, K = 4096, 4160
    Wt = S.random_ternary(31, N, K)
    packed, bad = pack_ternary(Wt)
    assert bad == 0
    cases = [(2, S.random_x(32, 2, K)), (48, S.random_x(33, 48, K)), (300, S.random_x(34, 300, K))]
    ref = []
    for M, x in cases:
        ref.append(forward_f32(x, packed, 0.02, N))
    busy = torch.cuda.Stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    big = torch.randn(4096, 4096, device="cuda")
    outs = []
    torch.cuda.synchronize()
    with torch.cuda.stream(busy):
        for _ in range(4):
            big = big @ big.T * 1e-3
    for i, (M, x) in enumerate(cases):
        st = streams[i % 2]
        with torch.cuda.stream(st):
            xd = to_dev(x)
            ws_bytes = L.bitlinear_workspace_bytes(M, N, K)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            L.bitlinear_forward_f32(xd, packed, 0.02, M, N, K, y, ws, ws_bytes, stream=st)
            outs.append((y, xd, ws))
    torch.cuda.synchronize()
    for (M, _), r, (y, _, _) in zip(cases, ref, outs):
        say(f"stream case M={M}")
        assert np.array_equal(y.cpu().numpy().view(np.uint32), r.view(np.uint32))


# 17 .. 64 tokens take the tiled kernel with 32 x 128 tiles, whole or split
# over K: own row sums, given row sums and the fused float32 forward, with
# ragged N and K, from grids of many tiles to a handful of split ones.
@pytest.mark.parametrize("M,N,K", [(17, 12800, 80), (40, 20000, 208), (64, 11008, 1040), (17, 640, 4160),
                                   (33, 1000, 2064)])
def test_medium_token_counts_tiled(M, N, K):
    run_case(M, N, K, seed=M * 7 + N + K, latent=False)


# Tiled kernel with the K loop split over several workgroups per tile (few
# 32 x 128 tiles, long K): the slices' int32 partials are added in slice
# order, so y_int is exact; own row sums (per slice), given row sums (taken
# off by the first slice) and the fused float32 forward.  Ragged M and N, K
# with a half-empty last step (odd number of 64-k blocks) and with a last
# block only a quarter inside K.
@pytest.mark.parametrize("M,N,K", [(65, 300, 4160), (96, 1000, 4112), (200, 640, 2064), (96, 2048, 11008)])
def test_tiled_split_k(M, N, K):
    L = bl()
    # the workspace holds xq and the partial sums of at least two slices
    assert L.bitlinear_workspace_bytes(M, N, K) >= M * K + 2 * M * N * 4
    run_case(M, N, K, seed=M * 5 + N * 3 + K, latent=False)
