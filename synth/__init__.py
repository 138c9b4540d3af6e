"""Seeded synthetic inputs for the DSA / CSA hot path.

This package draws random numbers and stores them in the dtypes the path consumes (fp32 as
float32, bf16 as uint16 bit patterns, MXFP4 as packed codes + E8M0 scale bytes). It holds none of
the method's arithmetic: it is the one module that both the CPU oracle (``oracle/``) and the GPU
path read from, so that both see the same stored bytes.

The generator is counter based (see ``synth.c``): element ``i`` of tensor ``tensor_id`` under
``seed`` is a pure function of those three numbers, so a single query row of a multi-GB tensor
can be regenerated on its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

# Tensor ids of the counter-based streams.
TID_QI, TID_KI, TID_W, TID_Q, TID_KV, TID_WIN, TID_SINK = 1, 2, 3, 4, 5, 6, 7


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_normal_f32.argtypes = [u64, u64, i64, i64, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, i64, i64, dbl, vp]
        L.synth_uniform_f32.argtypes = [u64, u64, i64, i64, dbl, dbl, vp]
        L.synth_normal_mxfp4.argtypes = [u64, u64, i64, i64, ctypes.c_int, dbl, vp, vp]
        L.synth_mxfp4_block.argtypes = [vp, vp, vp]
        L.synth_normal_mxfp8.argtypes = [u64, u64, i64, i64, ctypes.c_int, dbl, vp, vp]
        L.synth_mxfp8_block.argtypes = [vp, vp, vp]
        L.synth_bf16_from_double.argtypes = [dbl]
        L.synth_bf16_from_double.restype = ctypes.c_uint16
        L.synth_splitmix64.argtypes = [u64]
        L.synth_splitmix64.restype = u64
        L.synth_uniform_at.argtypes = [u64, u64, i64, ctypes.c_int]
        L.synth_uniform_at.restype = dbl
        L.synth_normal_at.argtypes = [u64, u64, i64]
        L.synth_normal_at.restype = dbl
        for f in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32",
                  "synth_normal_mxfp4", "synth_mxfp4_block", "synth_normal_mxfp8",
                  "synth_mxfp8_block"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, tid: int, shape, scale: float, dtype: str, start: int = 0) -> np.ndarray:
    """N(0,1)*scale, elements start.. start+prod(shape); dtype 'f32' (float32) or 'bf16' (uint16)."""
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(shape, np.float32)
        lib().synth_normal_f32(seed, tid, start, n, scale, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(shape, np.uint16)
        lib().synth_normal_bf16(seed, tid, start, n, scale, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def uniform(seed: int, tid: int, shape, lo: float, hi: float, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(shape, np.float32)
    lib().synth_uniform_f32(seed, tid, start, n, lo, hi, _ptr(out))
    return out


def normal_mxfp4(seed: int, tid: int, rows: int, D: int, scale: float = 1.0, start_row: int = 0):
    """MXFP4 rows of N(0,1)*scale: (codes [rows, D/2] uint8, scales [rows, D/32] uint8)."""
    assert D % 32 == 0
    codes = np.empty((rows, D // 2), np.uint8)
    scales = np.empty((rows, D // 32), np.uint8)
    lib().synth_normal_mxfp4(seed, tid, start_row, rows, D, scale, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp4_block(x: np.ndarray):
    """Quantise 32 fp64 values to (16 code bytes, 1 scale byte)."""
    x = np.ascontiguousarray(x, np.float64)
    assert x.shape == (32,)
    codes = np.empty(16, np.uint8)
    sc = np.empty(1, np.uint8)
    lib().synth_mxfp4_block(_ptr(x), _ptr(codes), _ptr(sc))
    return codes, int(sc[0])


def normal_mxfp8(seed: int, tid: int, rows: int, D: int, scale: float = 1.0, start_row: int = 0):
    """MXFP8 rows of N(0,1)*scale: (e4m3 codes [rows, D] uint8, scales [rows, D/32] uint8)."""
    assert D % 32 == 0
    codes = np.empty((rows, D), np.uint8)
    scales = np.empty((rows, D // 32), np.uint8)
    lib().synth_normal_mxfp8(seed, tid, start_row, rows, D, scale, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp8_block(x: np.ndarray):
    """Quantise 32 fp64 values to (32 e4m3 code bytes, 1 scale byte)."""
    x = np.ascontiguousarray(x, np.float64)
    assert x.shape == (32,)
    codes = np.empty(32, np.uint8)
    sc = np.empty(1, np.uint8)
    lib().synth_mxfp8_block(_ptr(x), _ptr(codes), _ptr(sc))
    return codes, int(sc[0])


def bf16_bits(x: float) -> int:
    return int(lib().synth_bf16_from_double(float(x)))


from .configs import CONFIGS, Workload, make_workload  # noqa: E402,F401
