"""ctypes front end of ``synth.c``: counter-based seeded draws.

Every element is a pure function of (seed, tensor id, element index), so any
slice can be drawn on its own and in parallel. The definition is in the header
comment of ``synth.c``.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` next to it (gcc, -O2)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            f = getattr(L, name)
            f.argtypes = [u64, u64, u64, u64, dbl, vp, ctypes.c_int]
            f.restype = ctypes.c_int
        L.synth_normal_f64.argtypes = [u64, u64, u64, u64, dbl, vp]
        L.synth_normal_f64.restype = ctypes.c_int
        L.synth_uniform_int.argtypes = [u64, u64, u64, u64, vp, i32, vp]
        L.synth_uniform_int.restype = ctypes.c_int
        L.synth_raw_u64.argtypes = [u64, u64, u64, u64, vp]
        L.synth_raw_u64.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed, tensor, count, std=1.0, offset=0, dtype="f32", threads=None, out=None):
    """``count`` N(0, std) draws of stream (seed, tensor) from ``offset``.

    dtype "f32" -> float32 array, "bf16" -> uint16 array of bf16 bit patterns,
    "f64" -> float64 array (single-threaded).
    """
    threads = default_threads() if threads is None else threads
    L = lib()
    if dtype == "f32":
        a = np.empty(count, np.float32) if out is None else out
        L.synth_normal_f32(seed, tensor, offset, count, std, a.ctypes.data, threads)
    elif dtype == "bf16":
        a = np.empty(count, np.uint16) if out is None else out
        L.synth_normal_bf16(seed, tensor, offset, count, std, a.ctypes.data, threads)
    elif dtype == "f64":
        a = np.empty(count, np.float64) if out is None else out
        L.synth_normal_f64(seed, tensor, offset, count, std, a.ctypes.data)
    else:
        raise ValueError(dtype)
    return a


def uniform_int(seed, tensor, count, bounds, offset=0):
    """``count`` integers; element i lies in [0, bounds[i % len(bounds)])."""
    b = np.ascontiguousarray(np.asarray(bounds, np.int32))
    out = np.empty(count, np.int32)
    lib().synth_uniform_int(seed, tensor, offset, count, b.ctypes.data, len(b), out.ctypes.data)
    return out


def raw_u64(seed, tensor, count, offset=0):
    out = np.empty(count, np.uint64)
    lib().synth_raw_u64(seed, tensor, offset, count, out.ctypes.data)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r
