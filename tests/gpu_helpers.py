"""Helpers for the GPU parity tests: run one step of the HIP path through the
C ABI (via the ctypes binding) on device buffers, and return host copies."""
from __future__ import annotations

import ctypes
import sys

import numpy as np


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def bl():
    from ternary_weight_linear_fwd_amd import bitlinear
    return bitlinear


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def empty(n_bytes: int):
    torch = torch_cuda()
    return torch.empty(max(int(n_bytes), 256), dtype=torch.uint8, device="cuda")


def quantize(x: np.ndarray):
    torch = torch_cuda()
    M, K = x.shape
    xd = to_dev(x.astype(np.float32))
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    eta = torch.empty(M, dtype=torch.float32, device="cuda")
    xsum = torch.empty(M, dtype=torch.int32, device="cuda")
    bl().bitlinear_quantize_act(xd, M, K, xq, eta, xsum)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), eta.cpu().numpy(), xsum.cpu().numpy()


def pack_weights_dev(Wd, N: int, K: int):
    """Pack a device latent matrix; returns (packed tensor, gamma float32, gamma device tensor)."""
    torch = torch_cuda()
    L = bl()
    packed = empty(L.bitlinear_packed_bytes(N, K))
    ws_bytes = L.bitlinear_workspace_bytes(0, N, K)
    ws = empty(ws_bytes)
    g_dev = torch.empty(1, dtype=torch.float32, device="cuda")
    g_host = ctypes.c_float(0.0)
    L.bitlinear_pack_weights(Wd, N, K, packed, g_dev, g_host, ws, ws_bytes)
    return packed, np.float32(g_host.value), g_dev


def pack_weights(W: np.ndarray):
    N, K = W.shape
    packed, g, g_dev = pack_weights_dev(to_dev(W.astype(np.float32)), N, K)
    assert float(g_dev.cpu()[0]) == float(g)
    return packed, g


def pack_ternary(Wt: np.ndarray):
    torch = torch_cuda()
    L = bl()
    N, K = Wt.shape
    packed = empty(L.bitlinear_packed_bytes(N, K))
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.bitlinear_pack_ternary(to_dev(Wt.astype(np.int8)), N, K, packed, bad)
    torch.cuda.synchronize()
    return packed, int(bad.cpu()[0])


def unpack(packed, N: int, K: int):
    torch = torch_cuda()
    Wt = torch.empty((N, K), dtype=torch.int8, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    bl().bitlinear_unpack_weights(packed, N, K, Wt, bad)
    torch.cuda.synchronize()
    return Wt.cpu().numpy(), int(bad.cpu()[0])


def forward(xq: np.ndarray, eta: np.ndarray, packed, gamma, N: int, with_int=True):
    torch = torch_cuda()
    L = bl()
    M, K = xq.shape
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_int = torch.empty((M, N), dtype=torch.int32, device="cuda") if with_int else None
    ws_bytes = L.bitlinear_workspace_bytes(M, N, K)
    ws = empty(ws_bytes)
    L.bitlinear_forward(to_dev(xq.astype(np.int8)), to_dev(eta.astype(np.float32)), packed,
                        float(gamma), M, N, K, y, y_int, ws, ws_bytes)
    torch.cuda.synchronize()
    return y.cpu().numpy(), (y_int.cpu().numpy() if with_int else None)


def forward_xsum(xq: np.ndarray, eta: np.ndarray, xsum: np.ndarray, packed, gamma, N: int):
    """bitlinear_forward_xsum with the given row sums (an input, like xq)."""
    torch = torch_cuda()
    L = bl()
    M, K = xq.shape
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_int = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws_bytes = L.bitlinear_workspace_bytes(M, N, K)
    ws = empty(ws_bytes)
    L.bitlinear_forward_xsum(to_dev(xq.astype(np.int8)), to_dev(eta.astype(np.float32)),
                             to_dev(xsum.astype(np.int32)), packed, float(gamma), M, N, K, y, y_int,
                             ws, ws_bytes)
    torch.cuda.synchronize()
    return y.cpu().numpy(), y_int.cpu().numpy()


def forward_f32(x: np.ndarray, packed, gamma, N: int):
    torch = torch_cuda()
    L = bl()
    M, K = x.shape
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws_bytes = L.bitlinear_workspace_bytes(M, N, K)
    ws = empty(ws_bytes)
    L.bitlinear_forward_f32(to_dev(x.astype(np.float32)), packed, float(gamma), M, N, K, y, ws,
                            ws_bytes)
    torch.cuda.synchronize()
    return y.cpu().numpy()


REL_TOL = 1e-6  # fp32 output gate: |y_gpu - y_ref| <= 1e-6 * |y_ref|


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray):
    """The float32 output gate; y_ref == 0 requires y_gpu == 0."""
    assert y_gpu.shape == y_ref.shape
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    lim = REL_TOL * np.abs(y_ref.astype(np.float64))
    bad = err > lim
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5].tolist())


def near_tie_rows():
    """Rows whose quotients x * 127 / eta straddle half-integers k + 1/2 at
    offsets on both sides of the quantizers' 2^-12 fast-path margin, and hit
    them exactly; eta (the row's first element) varies from row to row."""
    offs = np.array([0.0, 1e-7, -1e-7, 3e-6, -3e-6, 1e-5, -1e-5, 6e-5, -6e-5,
                     2.3e-4, -2.3e-4, 2.6e-4, -2.6e-4, 1e-3, -1e-3])
    q = ((np.arange(-126, 126) + 0.5)[:, None] + offs[None, :]).ravel()
    K = ((q.size + 1 + 15) // 16) * 16
    rows = []
    for eta in (3.0, 0.7, 1e-3, 1.0e4, 2.0 ** -10, 127.0):
        r = np.zeros(K, np.float32)
        r[0] = eta
        r[1:q.size + 1] = (q * eta / 127.0).astype(np.float32)
        rows.append(r)
    return np.stack(rows)
