"""CPU oracle for the BitNet b1.58 BitLinear forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``ternary_weight_linear_fwd_amd``) never imports it and shares no code with
it.

The arithmetic lives in ``bitlinear_oracle.c`` (plain C99, scalar loops, built
with gcc and ``-ffp-contract=off``); this module only builds that file and
marshals numpy arrays into it.  Each function names the page passages it
follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """Handle on one build of the oracle library (the default build, or a
    variant compiled elsewhere, e.g. by the pin-strength tests)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_absmean_gamma.argtypes = [P, I64, I64, P]
        L.oracle_ternarize.argtypes = [P, I64, I64, ctypes.c_float, P]
        L.oracle_absmedian_gamma.argtypes = [P, I64, I64, P]
        L.oracle_pack.argtypes = [P, I64, I64, P]
        L.oracle_unpack.argtypes = [P, I64, I64, P]
        L.oracle_quantize_act.argtypes = [P, I64, I64, P, P]
        L.oracle_ternary_contract.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int]
        L.oracle_dequant.argtypes = [P, P, ctypes.c_float, I64, I64, P]
        L.oracle_forward.argtypes = [P, P, ctypes.c_float, I64, I64, I64, P, P, P, P,
                                     ctypes.c_int]
        L.oracle_rmsnorm.argtypes = [P, I64, I64, P, P, P]
        L.oracle_rmsnorm_quantize_act.argtypes = [P, I64, I64, P, P, P, P]
        L.oracle_pack3.argtypes = [P, I64, I64, P]
        L.oracle_unpack3.argtypes = [P, I64, I64, P]
        L.oracle_packed3_row_bytes.argtypes = [I64]
        L.oracle_packed3_row_bytes.restype = I64
        L.oracle_packed_row_bytes.argtypes = [I64]
        L.oracle_packed_row_bytes.restype = I64
        self.lib = L
        self.path = path

    def absmean_gamma(self, W: np.ndarray) -> np.float32:
        """Exact mean of |W| rounded once to float32, clamped below at 1e-5."""
        W = _c(W, np.float32)
        N, K = W.shape
        out = np.zeros(1, np.float32)
        _check(self.lib.oracle_absmean_gamma(_p(W), N, K, _p(out)), "absmean_gamma")
        return out[0]

    def absmedian_gamma(self, W: np.ndarray) -> np.float32:
        """Median of |W| (mean of the two middle values for an even count,
        rounded once to float32), clamped below at 1e-5."""
        W = _c(W, np.float32)
        N, K = W.shape
        out = np.zeros(1, np.float32)
        _check(self.lib.oracle_absmedian_gamma(_p(W), N, K, _p(out)), "absmedian_gamma")
        return out[0]

    def quantize_weights_absmedian(self, W: np.ndarray):
        """(W~, gamma) with the absmedian scale."""
        g = self.absmedian_gamma(W)
        return self.ternarize(W, g), g

    def ternarize(self, W: np.ndarray, gamma) -> np.ndarray:
        W = _c(W, np.float32)
        N, K = W.shape
        Wt = np.empty((N, K), np.int8)
        _check(self.lib.oracle_ternarize(_p(W), N, K, float(np.float32(gamma)), _p(Wt)),
               "ternarize")
        return Wt

    def quantize_weights(self, W: np.ndarray):
        """(W~, gamma) as the page listings return them."""
        g = self.absmean_gamma(W)
        return self.ternarize(W, g), g

    def pack(self, Wt: np.ndarray) -> np.ndarray:
        """Canonical 2-bit format: [N][ceil(K/4)] bytes."""
        Wt = _c(Wt, np.int8)
        N, K = Wt.shape
        out = np.empty((N, (K + 3) // 4), np.uint8)
        _check(self.lib.oracle_pack(_p(Wt), N, K, _p(out)), "pack")
        return out

    def unpack(self, packed: np.ndarray, K: int) -> np.ndarray:
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        assert packed.shape[1] == (K + 3) // 4
        out = np.empty((N, K), np.int8)
        _check(self.lib.oracle_unpack(_p(packed), N, K, _p(out)), "unpack")
        return out

    def pack3(self, Wt: np.ndarray) -> np.ndarray:
        """Compact base-3 format: [N][ceil(K/5)] bytes, five weights per byte."""
        Wt = _c(Wt, np.int8)
        N, K = Wt.shape
        out = np.empty((N, (K + 4) // 5), np.uint8)
        _check(self.lib.oracle_pack3(_p(Wt), N, K, _p(out)), "pack3")
        return out

    def unpack3(self, packed: np.ndarray, K: int) -> np.ndarray:
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        assert packed.shape[1] == (K + 4) // 5
        out = np.empty((N, K), np.int8)
        _check(self.lib.oracle_unpack3(_p(packed), N, K, _p(out)), "unpack3")
        return out

    def quantize_act(self, x: np.ndarray):
        """(xq int8 [M][K], eta float32 [M])."""
        x = _c(x, np.float32)
        M, K = x.shape
        xq = np.empty((M, K), np.int8)
        eta = np.empty(M, np.float32)
        _check(self.lib.oracle_quantize_act(_p(x), M, K, _p(xq), _p(eta)), "quantize_act")
        return xq, eta

    def rmsnorm(self, x: np.ndarray):
        """RMSNorm without affine parameters: (x_norm [M][K], ms [M], norm [M]),
        ms being the mean of the squares and norm = 1 / sqrt(ms + 1e-6)."""
        x = _c(x, np.float32)
        M, K = x.shape
        xn = np.empty((M, K), np.float32)
        ms = np.empty(M, np.float32)
        norm = np.empty(M, np.float32)
        _check(self.lib.oracle_rmsnorm(_p(x), M, K, _p(xn), _p(ms), _p(norm)), "rmsnorm")
        return xn, ms, norm

    def rmsnorm_quantize_act(self, x: np.ndarray):
        """RMSNorm, then the absmax quantizer: (xq, eta, ms, norm)."""
        x = _c(x, np.float32)
        M, K = x.shape
        xq = np.empty((M, K), np.int8)
        eta = np.empty(M, np.float32)
        ms = np.empty(M, np.float32)
        norm = np.empty(M, np.float32)
        _check(self.lib.oracle_rmsnorm_quantize_act(_p(x), M, K, _p(xq), _p(eta), _p(ms),
                                                    _p(norm)), "rmsnorm_quantize_act")
        return xq, eta, ms, norm

    def ternary_contract(self, xq: np.ndarray, Wt: np.ndarray, threads: int = 1) -> np.ndarray:
        xq = _c(xq, np.int8)
        Wt = _c(Wt, np.int8)
        M, K = xq.shape
        N, K2 = Wt.shape
        assert K == K2
        y = np.empty((M, N), np.int32)
        _check(self.lib.oracle_ternary_contract(_p(xq), _p(Wt), M, N, K, _p(y), int(threads)),
               "ternary_contract")
        return y

    def dequant(self, y_int: np.ndarray, eta: np.ndarray, gamma) -> np.ndarray:
        y_int = _c(y_int, np.int32)
        eta = _c(eta, np.float32)
        M, N = y_int.shape
        y = np.empty((M, N), np.float32)
        _check(self.lib.oracle_dequant(_p(y_int), _p(eta), float(np.float32(gamma)), M, N,
                                       _p(y)), "dequant")
        return y

    def forward(self, x: np.ndarray, Wt: np.ndarray, gamma, threads: int = 1):
        """Full forward from float32 x; returns (y, xq, eta, y_int)."""
        x = _c(x, np.float32)
        Wt = _c(Wt, np.int8)
        M, K = x.shape
        N = Wt.shape[0]
        y = np.empty((M, N), np.float32)
        xq = np.empty((M, K), np.int8)
        eta = np.empty(M, np.float32)
        y_int = np.empty((M, N), np.int32)
        _check(self.lib.oracle_forward(_p(x), _p(Wt), float(np.float32(gamma)), M, N, K,
                                       _p(y), _p(xq), _p(eta), _p(y_int), int(threads)),
               "forward")
        return y, xq, eta, y_int

    def forward_q(self, xq: np.ndarray, eta: np.ndarray, Wt: np.ndarray, gamma,
                  threads: int = 1):
        """Forward from already-quantized activations; returns (y, y_int)."""
        y_int = self.ternary_contract(xq, Wt, threads)
        return self.dequant(y_int, eta, gamma), y_int


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


_default = None


def default() -> Oracle:
    """The oracle built from ``bitlinear_oracle.c`` (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def compile_variant(source_text: str, out_path: str) -> Oracle:
    """Compile a modified copy of the oracle source (used only by the tests that
    check the pins catch planted mistakes) and load it."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", out_path, "-lm"])
    return Oracle(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def absmean_gamma(W):
    return default().absmean_gamma(W)


def ternarize(W, gamma):
    return default().ternarize(W, gamma)


def quantize_weights(W):
    return default().quantize_weights(W)


def pack(Wt):
    return default().pack(Wt)


def unpack(packed, K):
    return default().unpack(packed, K)


def quantize_act(x):
    return default().quantize_act(x)


def ternary_contract(xq, Wt, threads=1):
    return default().ternary_contract(xq, Wt, threads)


def dequant(y_int, eta, gamma):
    return default().dequant(y_int, eta, gamma)


def forward(x, Wt, gamma, threads=1):
    return default().forward(x, Wt, gamma, threads)


def forward_q(xq, eta, Wt, gamma, threads=1):
    return default().forward_q(xq, eta, Wt, gamma, threads)


def rmsnorm(x):
    return default().rmsnorm(x)


def rmsnorm_quantize_act(x):
    return default().rmsnorm_quantize_act(x)


def pack3(Wt):
    return default().pack3(Wt)


def unpack3(packed, K):
    return default().unpack3(packed, K)


def absmedian_gamma(W):
    return default().absmedian_gamma(W)


def quantize_weights_absmedian(W):
    return default().quantize_weights_absmedian(W)
