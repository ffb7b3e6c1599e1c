"""The allocation-free fused forward (bitlinear_forward_f32_noalloc) against
bitlinear_forward_f32 on the same inputs, through the C ABI.

Both run the same kernels; the allocation-free call keeps its workspace in
the library's fixed device array instead of a caller buffer, so y must be
bit-identical.  Two calls in a row, the second smaller than the first (the
array keeps the first call's contents), then a third in another kernel class;
each is also checked against the CPU oracle's float32 output gate."""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_y_close, bl, forward_f32, pack_weights, say, to_dev, torch_cuda
from ternary_weight_linear_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu

# (M, N, K): 32 x 128 prefill tiles with K split (partials in the array), then
# the dot4 decode GEMV with K split, then the streaming matrix-core kernel.
CASES = [(200, 1000, 4096), (3, 2048, 1024), (12, 320, 1040)]


def _noalloc(x: np.ndarray, packed, gamma, N: int):
    torch = torch_cuda()
    M, K = x.shape
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    bl().bitlinear_forward_f32_noalloc(to_dev(x), packed, float(gamma), M, N, K, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_noalloc_matches_forward_f32_on_consecutive_calls():
    L = bl()
    for i, (M, N, K) in enumerate(CASES):
        say(f"noalloc case {i}: M={M} N={N} K={K}")
        assert L.bitlinear_workspace_bytes(M, N, K) <= L.BITLINEAR_NOALLOC_SCRATCH_BYTES
        W = S.random_latent(700 + i, N, K)
        x = S.random_x(800 + i, M, K)
        packed, g = pack_weights(W)
        y_ref_gpu = forward_f32(x, packed, g, N)
        y = _noalloc(x, packed, g, N)
        assert np.array_equal(y.view(np.uint32), y_ref_gpu.view(np.uint32)), f"case {i}"
        Wt, g_ref = oracle.quantize_weights(W)
        assert np.float32(g) == g_ref
        y_oracle, _, _, _ = oracle.forward(x, Wt, g_ref, threads=8)
        assert_y_close(y, y_oracle)

