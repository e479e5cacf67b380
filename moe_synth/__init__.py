"""Seeded synthetic inputs for the sparse-MoE layer.

This package generates inputs only.  It holds none of the layer's arithmetic:
no routing, no capacity formula, no expert math.  The CPU oracle (``oracle/``)
and the HIP library are both fed from the arrays built here, so that both see
identical bits.  The generator itself is defined in ``synth.c``.

bf16 tensors are returned as ``numpy.uint16`` arrays of raw bf16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import WORKLOADS, Workload, workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_synth.so")
_lib = None

# tensor ids of the counter-based streams
TID_X, TID_WG, TID_W1, TID_W3, TID_W2, TID_WS1, TID_WS3, TID_WS2, TID_SEL_BIAS = range(9)
# per-row scales of FP8 expert weights
TID_S1, TID_S3, TID_S2, TID_SS1, TID_SS3, TID_SS2 = range(9, 15)


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP) into ``libmoe_synth.so``."""
    src = os.path.join(_HERE, "synth.c")
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, u64, dbl, vp]
            fn.restype = None
        lib.synth_uniform_f32.argtypes = [u64, u64, u64, u64, dbl, dbl, vp]
        lib.synth_uniform_f32.restype = None
        lib.synth_bits.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_fp8_codes.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_fp8_codes.restype = None
        lib.synth_bits.restype = None
        lib.synth_splitmix64.argtypes = [u64, u64, vp]
        lib.synth_splitmix64.restype = None
        lib.synth_f32_to_bf16.argtypes = [vp, vp, u64]
        lib.synth_f32_to_bf16.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, tid: int, shape, std: float, dtype: str, offset: int = 0) -> np.ndarray:
    """N(0, std^2) draws of elements ``offset ..`` of stream (seed, tid).

    ``dtype`` is "f32" (float32 array) or "bf16" (uint16 array of bf16 bits).
    """
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(seed, tid, offset, n, float(std), _ptr(out))
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(seed, tid, offset, n, float(std), _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def uniform(seed: int, tid: int, shape, lo: float, hi: float, offset: int = 0) -> np.ndarray:
    """U(lo, hi] draws (float32) of elements ``offset ..`` of stream (seed, tid)."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.float32)
    lib.synth_uniform_f32(seed, tid, offset, n, float(lo), float(hi), _ptr(out))
    return out


def bits(seed: int, tid: int, count: int, offset: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty((count,), dtype=np.uint64)
    lib.synth_bits(seed, tid, offset, count, _ptr(out))
    return out


def fp8_codes(seed: int, tid: int, shape, offset: int = 0) -> np.ndarray:
    """Random FP8 E4M3 codes (uint8) of elements ``offset ..`` of stream
    (seed, tid): random sign and mantissa, exponent field 3 + Binomial(8, 1/2)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.uint8)
    _load().synth_fp8_codes(seed, tid, offset, n, _ptr(out))
    return out


def splitmix64(state: int, count: int) -> np.ndarray:
    """The plain sequential SplitMix64 stream from ``state``."""
    out = np.empty((count,), dtype=np.uint64)
    _load().synth_splitmix64(state, count, _ptr(out))
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits (uint16) to float32 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bits (nearest even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out
