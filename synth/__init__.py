"""Seeded synthetic inputs for the LSA decode path (shared by the GPU path's
tests/bench and by the oracle's tests; holds none of the method's arithmetic).

The element generator is SplitMix64 used counter-style (see ``synth.c``); this
module binds it with ctypes and assembles the workload tensors from it in
:mod:`synth.workloads`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Tensor tags: the high 32 bits of a stream id.  The low 32 bits carry a
# sub-index (interval, step, request) where a tensor has several instances.
TAG_QIDX = 1        # indexer query, per interval
TAG_KIDX = 2        # indexer keys (background)
TAG_GOLD_POS = 3    # golden-chunk positions, per (request, interval)
TAG_GOLD_NOISE = 4  # noise added to golden keys
TAG_KV = 5          # K/V store
TAG_Q = 6           # attention query, per step
TAG_MISC = 7        # test-only streams
TAG_RING = 8        # ring positions of the chunks (churn-controlled indexer), per request
TAG_RING_PHASE = 9  # starting angle of the ring query, per request


def stream(tag: int, sub: int = 0) -> int:
    return (int(tag) << 32) | (int(sub) & 0xFFFFFFFF)


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.synth_key.argtypes = [u64, u64]
        L.synth_key.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_draw.restype = u64
        L.synth_fill_i8.argtypes = [vp, i64, u64, i64, i32, i32]
        L.synth_fill_i32.argtypes = [vp, i64, u64, i64, i32, i32]
        L.synth_fill_u64.argtypes = [vp, i64, u64, i64]
        L.synth_fill_normal_bf16.argtypes = [vp, i64, u64, i64, ctypes.c_double]
        L.synth_fill_normal_bf16_runs.argtypes = [vp, vp, i64, i64, u64, ctypes.c_double]
        L.synth_choose.argtypes = [vp, i64, i64, vp, u64, vp]
        L.synth_choose.restype = i64
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(seed: int, strm: int) -> int:
    return int(lib().synth_key(seed & (2**64 - 1), strm & (2**64 - 1)))


def draw(k: int, i: int) -> int:
    return int(lib().synth_draw(k, i))


def uniform_i8(shape, seed: int, strm: int, lo: int, hi: int, first: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.int8)
    lib().synth_fill_i8(_ptr(out), out.size, key(seed, strm), first, lo, hi)
    return out


def uniform_i32(shape, seed: int, strm: int, lo: int, hi: int, first: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.int32)
    lib().synth_fill_i32(_ptr(out), out.size, key(seed, strm), first, lo, hi)
    return out


def raw_u64(n: int, seed: int, strm: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_fill_u64(_ptr(out), n, key(seed, strm), first)
    return out


def normal_bf16_into(out: np.ndarray, seed: int, strm: int, first: int = 0, scale: float = 1.0) -> np.ndarray:
    """Fill ``out`` (uint16 bf16 bits, any shape, C-contiguous) with N(0,1)*scale."""
    assert out.dtype == np.uint16
    lib().synth_fill_normal_bf16(_ptr(out), out.size, key(seed, strm), first, float(scale))
    return out


def normal_bf16(shape, seed: int, strm: int, first: int = 0, scale: float = 1.0) -> np.ndarray:
    return normal_bf16_into(np.empty(shape, dtype=np.uint16), seed, strm, first, scale)


def normal_bf16_runs(src_first: np.ndarray, run_len: int, seed: int, strm: int, scale: float = 1.0) -> np.ndarray:
    """Regenerate runs of a large bf16 normal tensor: run r is elements
    src_first[r] .. src_first[r]+run_len-1.  Returns uint16 [runs, run_len]."""
    src_first = np.ascontiguousarray(src_first, dtype=np.int64)
    out = np.empty((src_first.size, run_len), dtype=np.uint16)
    lib().synth_fill_normal_bf16_runs(_ptr(out), _ptr(src_first), src_first.size, run_len,
                                      key(seed, strm), float(scale))
    return out


def choose(count: int, n: int, seed: int, strm: int, excluded: np.ndarray | None = None) -> np.ndarray:
    """``count`` distinct positions of [0, n), uniform without replacement,
    avoiding positions where ``excluded`` is nonzero."""
    out = np.empty(count, dtype=np.int32)
    work = np.empty(max(n, 1), dtype=np.int32)
    ex = 0
    if excluded is not None:
        excluded = np.ascontiguousarray(excluded, dtype=np.uint8)
        assert excluded.size == n
        ex = _ptr(excluded)
    got = lib().synth_choose(_ptr(out), count, n, ex, key(seed, strm), _ptr(work))
    return out[:got]


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (bit shift, no rounding)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
