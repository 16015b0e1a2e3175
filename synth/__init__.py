"""Seeded synthetic inputs for the CacheTune hot path (shared by the oracle
side and the GPU side of every test and of the bench).

The value model lives in ``synth.c`` (see its header).  This module holds no
arithmetic of the method itself: it only produces stored tensors, chunk
lengths and chunk orders.  bf16 tensors are numpy ``uint16`` bit patterns,
fp32 tensors are ``float32``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")
SRC_PATH = os.path.join(HERE, "synth.c")

K, V, Q = 0, 1, 2
SUFFIX_CHUNK = 1 << 20  # chunk id used for the uncached suffix rows

_lib = None


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared",
           SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        u64, i32, f64, vp = C.c_uint64, C.c_int, C.c_double, C.c_void_p
        L.synth_spikes.argtypes = [u64, i32, i32, vp]
        L.synth_rows.argtypes = [u64, i32, i32, i32, i32, i32, i32, vp, i32, f64, i32, vp]
        L.synth_chunk.argtypes = [u64, i32, i32, i32, i32, i32, i32, i32, i32, vp]
        L.synth_uniform_ints.argtypes = [u64, i32, i32, i32, i32, vp]
        L.synth_permutation.argtypes = [u64, i32, i32, vp]
        L.synth_normal.argtypes = [u64, i32, C.c_longlong, f64, f64, i32, vp]
        _lib = L
    return _lib


def _code(dtype: str) -> int:
    if dtype == "f32":
        return 0
    if dtype == "bf16":
        return 1
    raise ValueError(dtype)


def _np(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def chunk(seed: int, tensor: int, chunk_id: int, L: int, N: int, H: int, D: int,
          dtype: str, l0: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Stored pre-RoPE tensor of one chunk, [L][N][H][D] (layers l0..l0+L-1)."""
    if out is None:
        out = np.empty((L, N, H, D), dtype=_np(dtype))
    assert out.shape == (L, N, H, D) and out.flags.c_contiguous and out.dtype == _np(dtype)
    lib().synth_chunk(seed, tensor, chunk_id, l0, L, N, H, D, _code(dtype),
                      out.ctypes.data_as(C.c_void_p))
    return out


def rows(seed: int, tensor: int, chunk_id: int, layer: int, N: int, H: int, D: int,
         idx, dtype: str, extra_sigma: float = 0.0) -> np.ndarray:
    """Value model at the listed token rows of one (tensor, chunk, layer):
    [len(idx)][H][D].  extra_sigma > 0 adds independent N(0, sigma^2) noise to
    the stored value (rows recomputed in the new context)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.empty((idx.shape[0], H, D), dtype=_np(dtype))
    if idx.shape[0]:
        lib().synth_rows(seed, tensor, chunk_id, layer, N, H, D,
                         idx.ctypes.data_as(C.c_void_p), idx.shape[0], float(extra_sigma),
                         _code(dtype), out.ctypes.data_as(C.c_void_p))
    return out


def spikes(seed: int, chunk_id: int, N: int) -> np.ndarray:
    out = np.zeros(4, np.int32)
    lib().synth_spikes(seed, chunk_id, N, out.ctypes.data_as(C.c_void_p))
    return out[:min(4, N)]


def uniform_ints(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.zeros(n, np.int32)
    lib().synth_uniform_ints(seed, stream, n, lo, hi, out.ctypes.data_as(C.c_void_p))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.int32)
    lib().synth_permutation(seed, stream, n, out.ctypes.data_as(C.c_void_p))
    return out


def normal(seed: int, stream: int, shape, dtype: str, mean: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(mean, sigma^2) values of one stream, stored in dtype (weights,
    gains and hidden rows of the recompute layer)."""
    out = np.empty(shape, dtype=_np(dtype))
    lib().synth_normal(seed, stream, out.size, float(mean), float(sigma), _code(dtype),
                       out.ctypes.data_as(C.c_void_p))
    return out
