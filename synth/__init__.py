"""Seeded synthetic inputs for the routed MoE layer.

The generator draws numbers and stores them (fp32, bf16 bit patterns, or OCP E4M3FN
codes with per-row fp32 scales); it computes nothing of the layer itself.  Both the
CPU oracle and the HIP library receive exactly the bytes written here.  The draws are
counter-based (SplitMix64 + Box-Muller, see ``synth.c``), so a tensor's bytes depend
only on (seed, tag, index) and never on thread count or machine.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_I64 = ctypes.c_int64


def _threads():
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise ImportError(f"generator library {_build.LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_build.LIB)
        lib.synth_normal_f32.argtypes = [_U64, _U64, _U64, _I64, ctypes.c_double, _P, ctypes.c_int]
        lib.synth_normal_bf16.argtypes = [_U64, _U64, _U64, _I64, ctypes.c_double, _P, ctypes.c_int]
        lib.synth_normal_fp8_rows.argtypes = [_U64, _U64, _U64, _I64, _I64, ctypes.c_double, _P, _P, ctypes.c_int]
        lib.synth_normal_mxfp4_rows.argtypes = [_U64, _U64, _U64, _I64, _I64, ctypes.c_double, _P, _P, ctypes.c_int]
        lib.synth_uniform_f64.argtypes = [_U64, _U64, _U64, _I64, _P]
        lib.synth_permutation.argtypes = [_U64, _U64, ctypes.c_int32, _P]
        lib.synth_u64.argtypes = [_U64, _U64, _U64, _I64, _P]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_normal_fp8_rows, lib.synth_normal_mxfp4_rows,
                  lib.synth_uniform_f64,
                  lib.synth_permutation, lib.synth_u64):
            f.restype = None
        _lib = lib
    return _lib


def normal_f32(seed, tag, shape, std, first=0):
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, tag, first, out.size, float(std), out.ctypes.data, _threads())
    return out


def normal_bf16(seed, tag, shape, std, first=0):
    """bf16 bit patterns (uint16) of N(0, std^2) draws."""
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tag, first, out.size, float(std), out.ctypes.data, _threads())
    return out


def normal_fp8_rows(seed, tag, shape, std, first=0):
    """E4M3FN codes (uint8) of N(0, std^2) draws quantised per last-axis row, and the fp32 row scales."""
    codes = np.empty(shape, dtype=np.uint8)
    rows = int(np.prod(shape[:-1]))
    scales = np.empty(shape[:-1], dtype=np.float32)
    _load().synth_normal_fp8_rows(seed, tag, first, rows, shape[-1], float(std), codes.ctypes.data,
                                  scales.ctypes.data, _threads())
    return codes, scales


def normal_mxfp4_rows(seed, tag, shape, std, first=0):
    """MXFP4 of N(0, std^2) draws along the last axis: code bytes [..., L/2] (even value in the low
    nibble) and E8M0 scale bytes [..., L/32], one per block of 32 values."""
    L = shape[-1]
    assert L % 32 == 0
    rows = int(np.prod(shape[:-1]))
    codes = np.empty(tuple(shape[:-1]) + (L // 2,), dtype=np.uint8)
    scales = np.empty(tuple(shape[:-1]) + (L // 32,), dtype=np.uint8)
    _load().synth_normal_mxfp4_rows(seed, tag, first, rows, L, float(std), codes.ctypes.data, scales.ctypes.data,
                                    _threads())
    return codes, scales


def uniform_f64(seed, tag, n, first=0):
    out = np.empty((n,), dtype=np.float64)
    _load().synth_uniform_f64(seed, tag, first, n, out.ctypes.data)
    return out


def permutation(seed, tag, n):
    out = np.empty((n,), dtype=np.int32)
    _load().synth_permutation(seed, tag, n, out.ctypes.data)
    return out


def raw_u64(seed, tag, n, first=0):
    out = np.empty((n,), dtype=np.uint64)
    _load().synth_u64(seed, tag, first, n, out.ctypes.data)
    return out
