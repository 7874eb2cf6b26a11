"""Python binding of libfb_ceiling.so (include/fb_ceiling.h): the streaming-read and bf16
MFMA-loop kernels whose measured rates the bench sets beside the published peaks, and the
MFMA/vector co-issue measurement.

Argument marshalling only; raises when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

from . import _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfb_ceiling.so")
EXPORTS = ("fbc_stream_read", "fbc_mfma_loop", "fbc_mfma_valu")
FLOPS_PER_WAVE_ITER = 4 * 32768   # 4 accumulators x one 32x32x16 multiply-add (2 flops each)

_lib = None


class CeilingError(RuntimeError):
    pass


def load(path: str | None = None):
    """Load the shared library (raises FileNotFoundError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing; build it with `python -m cached_kv_prefix_amd.build`")
    lib = C.CDLL(p)
    lib.fbc_stream_read.restype = C.c_int
    lib.fbc_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    lib.fbc_mfma_loop.restype = C.c_int
    lib.fbc_mfma_loop.argtypes = [C.c_int32, C.c_int64, C.c_float, C.c_float, C.c_void_p, C.c_void_p]
    lib.fbc_mfma_valu.restype = C.c_int
    lib.fbc_mfma_valu.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_void_p]
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise CeilingError(f"{where}: status {status}")


def stream_read(buf, nbytes: int, workgroups: int, sink, stream=None, nontemporal: bool = False) -> None:
    """Read nbytes of buf once (with the non-temporal hint when asked); sink (>= 16 *
    workgroups bytes) gets each workgroup's XOR."""
    _check(load().fbc_stream_read(_ptr(buf), nbytes, workgroups, int(bool(nontemporal)), _ptr(sink),
                                  _stream(stream)), "fbc_stream_read")


def mfma_loop(workgroups: int, iters: int, a: float, b: float, sink, stream=None) -> None:
    """workgroups x 4 waves x iters rounds of 4 bf16 32x32x16 MFMAs; sink (>= 4 * workgroups
    floats) gets 64 * iters * bf16(a) * bf16(b) per wave when that is exact in fp32."""
    _check(load().fbc_mfma_loop(workgroups, iters, a, b, _ptr(sink), _stream(stream)), "fbc_mfma_loop")


def mfma_flops(workgroups: int, iters: int) -> float:
    return float(workgroups) * 4 * iters * FLOPS_PER_WAVE_ITER


MFMA_VALU_MODES = {"mfma": 0, "valu": 1, "pair": 2, "interleaved": 3}


def mfma_valu(mode: str, valu_per_mfma: int, workgroups: int, rounds: int, sink, stream=None) -> None:
    """One launch of the co-issue measurement (see fbc_mfma_valu); sink >= 8 * workgroups floats."""
    _check(load().fbc_mfma_valu(MFMA_VALU_MODES[mode], valu_per_mfma, workgroups, rounds, 1.0, _ptr(sink),
                                _stream(stream)), "fbc_mfma_valu")


def mfma_valu_expected(mode: str, rounds: int):
    """The sink entries [8 per workgroup] a launch writes: (value per wave, or None if unwritten)."""
    m = MFMA_VALU_MODES[mode]
    full = float(128 * rounds)
    if m == 0 or m == 3:
        return [full] * 4 + [None] * 4
    if m == 1:
        return [0.0] * 4 + [None] * 4
    return [full] * 4 + [0.0] * 4
