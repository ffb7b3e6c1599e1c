"""Thin ctypes binding of ``libbitlinear.so`` (the C ABI in include/bitlinear.h).

Argument marshalling only: every function takes torch device tensors (or raw
integers for pointers), passes ``data_ptr()`` values and the current HIP stream
to the call of the same name, and raises :class:`BitLinearError` on a non-zero
status.  All computation happens in the library's HIP kernels.

Importing this module fails loudly when the built library is missing: there
is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

# torch ships its own HIP runtime (same SONAME, libamdhip64.so.7).  Load it
# first so that the library binds to that one copy: two HIP runtimes in one
# process do not share devices, streams or memory.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m ternary_weight_linear_fwd_amd.build` "
        "(hipcc, gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

BITLINEAR_OK = 0
BITLINEAR_EINVAL = -1
BITLINEAR_EUNSUPPORTED = -2
BITLINEAR_EWORKSPACE = -3
BITLINEAR_EBADCODE = -4
BITLINEAR_EHIP = -5
BITLINEAR_MAX_K = 1 << 21

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_F = ctypes.c_float


class BitLinearProblem(ctypes.Structure):
    """Mirror of ``bitlinear_problem``."""
    _fields_ = [("x", _P), ("xq", _P), ("eta", _P), ("packed", _P), ("y", _P), ("y_int", _P),
                ("gamma", _F), ("N", _I32), ("K", _I32), ("format", _I32)]


class BitLinearGroupedPlan(ctypes.Structure):
    """Mirror of ``bitlinear_grouped_plan``."""
    _fields_ = [("table", _P), ("table_bytes", _SZ), ("units", _I64), ("quant_rows", _I64),
                ("count", _I32), ("M", _I32), ("kernel", _I32), ("max_K", _I32)]


_SIGS = {
    "bitlinear_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "bitlinear_abi_version": ([], ctypes.c_int),
    "bitlinear_last_error": ([], ctypes.c_char_p),
    "bitlinear_packed_bytes": ([_I64, _I64], _SZ),
    "bitlinear_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "bitlinear_quantize_act": ([_P, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "bitlinear_rmsnorm_quantize_act": ([_P, _I64, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "bitlinear_pack_weights": ([_P, _I64, _I64, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "bitlinear_pack_weights_absmedian": ([_P, _I64, _I64, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "bitlinear_pack_ternary": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "bitlinear_unpack_weights": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "bitlinear_forward": ([_P, _P, _P, _F, _I64, _I64, _I64, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "bitlinear_forward_xsum": ([_P, _P, _P, _P, _F, _I64, _I64, _I64, _P, _P, _P, _SZ, _P],
                               ctypes.c_int),
    "bitlinear_forward_f32": ([_P, _P, _F, _I64, _I64, _I64, _P, _P, _SZ, _P], ctypes.c_int),
    "bitlinear_forward_rmsnorm_f32": ([_P, _P, _F, _I64, _I64, _I64, _P, _P, _SZ, _P],
                                      ctypes.c_int),
    "bitlinear_forward_f32_noalloc": ([_P, _P, _F, _I64, _I64, _I64, _P, _P], ctypes.c_int),
    "bitlinear_packed3_bytes": ([_I64, _I64], _SZ),
    "bitlinear_pack_weights3": ([_P, _I64, _I64, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "bitlinear_pack_ternary3": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "bitlinear_unpack_weights3": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "bitlinear_lut_workspace_bytes": ([_I64, _I64, _I64, ctypes.c_int], _SZ),
    "bitlinear_forward_lut": ([_P, _P, _P, ctypes.c_int, _F, _I64, _I64, _I64, _P, _P, _P, _SZ,
                               _P], ctypes.c_int),
    "bitlinear_forward3_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "bitlinear_forward3": ([_P, _P, _P, _F, _I64, _I64, _I64, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "bitlinear_grouped_table_bytes": ([ctypes.POINTER(BitLinearProblem), _I32, _I64], _SZ),
    "bitlinear_grouped_plan_init": ([ctypes.POINTER(BitLinearProblem), _I32, _I64, _P, _SZ,
                                     ctypes.POINTER(BitLinearGroupedPlan), _P], ctypes.c_int),
    "bitlinear_forward_grouped": ([ctypes.POINTER(BitLinearGroupedPlan), _P], ctypes.c_int),
    # measurement probes (include/bitlinear_measure.h)
    "bitlinear_measure_sink_bytes": ([], _SZ),
    "bitlinear_measure_stream_read": ([_P, _SZ, _P, _P], ctypes.c_int),
    "bitlinear_measure_mfma_i8": ([_P, _P, _I32, _P, _P], ctypes.c_int),
    "bitlinear_measure_mfma_ops": ([_I32], ctypes.c_double),
}

for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


class BitLinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = f" [{bitlinear_last_error()}]" if status == BITLINEAR_EHIP else ""
        super().__init__(f"{what}: {bitlinear_status_string(status)} ({status}){detail}")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != BITLINEAR_OK:
        raise BitLinearError(status, what)


def _ptr(t) -> Optional[int]:
    """Device address of a tensor, an int passed through, None for NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------- pure host
def bitlinear_status_string(status: int) -> str:
    return _lib.bitlinear_status_string(status).decode()


def bitlinear_abi_version() -> int:
    return _lib.bitlinear_abi_version()


def bitlinear_last_error() -> str:
    return _lib.bitlinear_last_error().decode()


def bitlinear_packed_bytes(N: int, K: int) -> int:
    return _lib.bitlinear_packed_bytes(N, K)


def bitlinear_workspace_bytes(M: int, N: int, K: int) -> int:
    return _lib.bitlinear_workspace_bytes(M, N, K)


# ----------------------------------------------------------------- device calls
def bitlinear_quantize_act(x, M: int, K: int, xq, eta, xsum=None, stream=None) -> None:
    _check(_lib.bitlinear_quantize_act(_ptr(x), M, K, _ptr(xq), _ptr(eta), _ptr(xsum),
                                       _stream(stream)), "bitlinear_quantize_act")


def bitlinear_pack_weights(W, N: int, K: int, packed, gamma=None, gamma_host=None, ws=None,
                           ws_bytes: int = 0, stream=None) -> None:
    """gamma_host: a ctypes.c_float to receive gamma (the call then synchronizes), or None."""
    if isinstance(gamma_host, ctypes.c_float):
        gamma_host = ctypes.addressof(gamma_host)
    _check(_lib.bitlinear_pack_weights(_ptr(W), N, K, _ptr(packed), _ptr(gamma), gamma_host,
                                       _ptr(ws), ws_bytes, _stream(stream)),
           "bitlinear_pack_weights")


def bitlinear_pack_ternary(Wt, N: int, K: int, packed, bad=None, stream=None) -> None:
    _check(_lib.bitlinear_pack_ternary(_ptr(Wt), N, K, _ptr(packed), _ptr(bad), _stream(stream)),
           "bitlinear_pack_ternary")


def bitlinear_unpack_weights(packed, N: int, K: int, Wt, bad=None, stream=None) -> None:
    _check(_lib.bitlinear_unpack_weights(_ptr(packed), N, K, _ptr(Wt), _ptr(bad),
                                         _stream(stream)), "bitlinear_unpack_weights")


def bitlinear_forward(xq, eta, packed, gamma: float, M: int, N: int, K: int, y, y_int=None,
                      ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(_lib.bitlinear_forward(_ptr(xq), _ptr(eta), _ptr(packed), float(gamma), M, N, K,
                                  _ptr(y), _ptr(y_int), _ptr(ws), ws_bytes, _stream(stream)),
           "bitlinear_forward")


def bitlinear_forward_xsum(xq, eta, xsum, packed, gamma: float, M: int, N: int, K: int, y,
                           y_int=None, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(_lib.bitlinear_forward_xsum(_ptr(xq), _ptr(eta), _ptr(xsum), _ptr(packed),
                                       float(gamma), M, N, K, _ptr(y), _ptr(y_int), _ptr(ws),
                                       ws_bytes, _stream(stream)),
           "bitlinear_forward_xsum")


def bitlinear_forward_f32(x, packed, gamma: float, M: int, N: int, K: int, y, ws,
                          ws_bytes: int, stream=None) -> None:
    _check(_lib.bitlinear_forward_f32(_ptr(x), _ptr(packed), float(gamma), M, N, K, _ptr(y),
                                      _ptr(ws), ws_bytes, _stream(stream)),
           "bitlinear_forward_f32")


BITLINEAR_NOALLOC_SCRATCH_BYTES = 64 << 20


def bitlinear_forward_f32_noalloc(x, packed, gamma: float, M: int, N: int, K: int, y,
                                  stream=None) -> None:
    _check(_lib.bitlinear_forward_f32_noalloc(_ptr(x), _ptr(packed), float(gamma), M, N, K,
                                              _ptr(y), _stream(stream)),
           "bitlinear_forward_f32_noalloc")


def bitlinear_rmsnorm_quantize_act(x, M: int, K: int, xq, eta, xsum=None, ms=None,
                                   stream=None) -> None:
    _check(_lib.bitlinear_rmsnorm_quantize_act(_ptr(x), M, K, _ptr(xq), _ptr(eta), _ptr(xsum),
                                               _ptr(ms), _stream(stream)),
           "bitlinear_rmsnorm_quantize_act")


def bitlinear_forward_rmsnorm_f32(x, packed, gamma: float, M: int, N: int, K: int, y, ws,
                                  ws_bytes: int, stream=None) -> None:
    _check(_lib.bitlinear_forward_rmsnorm_f32(_ptr(x), _ptr(packed), float(gamma), M, N, K,
                                              _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "bitlinear_forward_rmsnorm_f32")


BITLINEAR_FORMAT_2BIT = 0
BITLINEAR_FORMAT_BASE3 = 1


def bitlinear_packed3_bytes(N: int, K: int) -> int:
    return _lib.bitlinear_packed3_bytes(N, K)


def bitlinear_pack_weights_absmedian(W, N: int, K: int, packed, gamma=None, gamma_host=None,
                                     ws=None, ws_bytes: int = 0, stream=None) -> None:
    """gamma_host: a ctypes.c_float to receive gamma (the call then synchronizes), or None."""
    if isinstance(gamma_host, ctypes.c_float):
        gamma_host = ctypes.addressof(gamma_host)
    _check(_lib.bitlinear_pack_weights_absmedian(_ptr(W), N, K, _ptr(packed), _ptr(gamma),
                                                 gamma_host, _ptr(ws), ws_bytes, _stream(stream)),
           "bitlinear_pack_weights_absmedian")


def bitlinear_pack_weights3(W, N: int, K: int, packed3, gamma=None, gamma_host=None, ws=None,
                            ws_bytes: int = 0, stream=None) -> None:
    """gamma_host: a ctypes.c_float to receive gamma (the call then synchronizes), or None."""
    if isinstance(gamma_host, ctypes.c_float):
        gamma_host = ctypes.addressof(gamma_host)
    _check(_lib.bitlinear_pack_weights3(_ptr(W), N, K, _ptr(packed3), _ptr(gamma), gamma_host,
                                        _ptr(ws), ws_bytes, _stream(stream)),
           "bitlinear_pack_weights3")


def bitlinear_pack_ternary3(Wt, N: int, K: int, packed3, bad=None, stream=None) -> None:
    _check(_lib.bitlinear_pack_ternary3(_ptr(Wt), N, K, _ptr(packed3), _ptr(bad),
                                        _stream(stream)), "bitlinear_pack_ternary3")


def bitlinear_unpack_weights3(packed3, N: int, K: int, Wt, bad=None, stream=None) -> None:
    _check(_lib.bitlinear_unpack_weights3(_ptr(packed3), N, K, _ptr(Wt), _ptr(bad),
                                          _stream(stream)), "bitlinear_unpack_weights3")


def bitlinear_lut_workspace_bytes(M: int, N: int, K: int, fmt: int) -> int:
    return _lib.bitlinear_lut_workspace_bytes(M, N, K, fmt)


def bitlinear_forward_lut(xq, eta, packed, fmt: int, gamma: float, M: int, N: int, K: int, y,
                          y_int=None, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(_lib.bitlinear_forward_lut(_ptr(xq), _ptr(eta), _ptr(packed), int(fmt), float(gamma),
                                      M, N, K, _ptr(y), _ptr(y_int), _ptr(ws), ws_bytes,
                                      _stream(stream)), "bitlinear_forward_lut")


def bitlinear_forward3_workspace_bytes(M: int, N: int, K: int) -> int:
    return _lib.bitlinear_forward3_workspace_bytes(M, N, K)


def bitlinear_forward3(xq, eta, packed3, gamma: float, M: int, N: int, K: int, y, y_int=None,
                       ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(_lib.bitlinear_forward3(_ptr(xq), _ptr(eta), _ptr(packed3), float(gamma), M, N, K, _ptr(y),
                                   _ptr(y_int), _ptr(ws), ws_bytes, _stream(stream)), "bitlinear_forward3")


def make_problems(specs: Sequence[dict]):
    """ctypes array of bitlinear_problem from dicts of tensors/ints."""
    arr = (BitLinearProblem * len(specs))()
    for i, s in enumerate(specs):
        arr[i].x = _ptr(s.get("x"))
        arr[i].xq = _ptr(s["xq"])
        arr[i].eta = _ptr(s["eta"])
        arr[i].packed = _ptr(s["packed"])
        arr[i].y = _ptr(s["y"])
        arr[i].y_int = _ptr(s.get("y_int"))
        arr[i].gamma = float(s["gamma"])
        arr[i].N = int(s["N"])
        arr[i].K = int(s["K"])
        arr[i].format = int(s.get("format", BITLINEAR_FORMAT_2BIT))
    return arr


def bitlinear_grouped_table_bytes(problems, count: int, M: int) -> int:
    return _lib.bitlinear_grouped_table_bytes(problems, count, M)


def bitlinear_grouped_plan_init(problems, count: int, M: int, table, table_bytes: int,
                                stream=None) -> BitLinearGroupedPlan:
    plan = BitLinearGroupedPlan()
    _check(_lib.bitlinear_grouped_plan_init(problems, count, M, _ptr(table), table_bytes,
                                            ctypes.byref(plan), _stream(stream)),
           "bitlinear_grouped_plan_init")
    return plan


def bitlinear_forward_grouped(plan: BitLinearGroupedPlan, stream=None) -> None:
    _check(_lib.bitlinear_forward_grouped(ctypes.byref(plan), _stream(stream)),
           "bitlinear_forward_grouped")


# ------------------------------------------------- measurement probes (ceilings)
def bitlinear_measure_sink_bytes() -> int:
    return _lib.bitlinear_measure_sink_bytes()


def bitlinear_measure_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    _check(_lib.bitlinear_measure_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)),
           "bitlinear_measure_stream_read")


def bitlinear_measure_mfma_i8(xq, packed, iters: int, sink, stream=None) -> None:
    _check(_lib.bitlinear_measure_mfma_i8(_ptr(xq), _ptr(packed), iters, _ptr(sink), _stream(stream)),
           "bitlinear_measure_mfma_i8")


def bitlinear_measure_mfma_ops(iters: int) -> float:
    return _lib.bitlinear_measure_mfma_ops(iters)
