"""Seeded synthetic inputs for the histogram workloads.

This module draws bin indices and nothing else: it holds none of the
histogram's arithmetic. The HIP path and the CPU oracle are both fed from the
arrays it returns, so a disagreement between them is never the generator's.

The random source is SplitMix64 in counter form and the distributions are
described in ``gen.c``. The five workloads below are the sizes and value
distributions the benchmark quotes; ``generate(cfg, n)`` applies the same
recipe at any length so that parity tests can use smaller instances that keep
the shape (skew, hot bins, the Gaussian mass on a range boundary).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gen.c")
LIBRARY = os.path.join(_HERE, "libpca_gen.so")

TAG_UNIFORM = 0x554E49464F524D31
TAG_SHUFFLE = 0x53485546464C4531


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    n: int
    num_bins: int
    seed: int
    recipe: str


WORKLOADS = {
    1: Workload(1, "uniform-8k", 1_048_576, 8_192, 0,
                "int32 uniform in [0, 8192), seed 0"),
    2: Workload(2, "uniform-64k", 67_108_864, 65_536, 1,
                "int32 uniform in [0, 65536), seed 1"),
    3: Workload(3, "zipf1.1-256k", 268_435_456, 262_144, 2,
                "int32 Zipf s=1.1 over 262144 ranks, ranks permuted to bins, seed 2"),
    4: Workload(4, "hot10-1m", 268_435_456, 1_048_576, 3,
                "int32: floor(n/10) copies of 524287 + uniform [0, 2^20), shuffled, seed 3"),
    5: Workload(5, "gauss-half-512k", 536_870_912, 524_288, 4,
                "int32: n/2 uniform [0, 2^19) + n/2 round(N(262144, 1000^2)) clamped, "
                "shuffled, seed 4"),
}

_lib = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    tmp = output + ".tmp"
    subprocess.run(
        ["gcc", "-O3", "-std=gnu11", "-fopenmp", "-Wall", "-Wextra", "-Werror", "-fPIC",
         "-shared", source, "-o", tmp, "-lm"],
        check=True,
    )
    os.replace(tmp, output)
    return output


def _library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        lib = ctypes.CDLL(LIBRARY)
        u64, i32, u32, vp = ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
        lib.gen_key.restype = u64
        lib.gen_key.argtypes = [u64, u64]
        lib.gen_stream.restype = None
        lib.gen_stream.argtypes = [u64, u64, u64, vp]
        lib.gen_uniform.restype = None
        lib.gen_uniform.argtypes = [u64, u64, vp, u64, i32, u32]
        lib.gen_shuffle.restype = None
        lib.gen_shuffle.argtypes = [u64, vp, u64]
        lib.gen_zipf.restype = ctypes.c_int
        lib.gen_zipf.argtypes = [u64, vp, u64, u32, ctypes.c_double]
        lib.gen_config.restype = ctypes.c_int
        lib.gen_config.argtypes = [ctypes.c_int, vp, u64, vp]
        _lib = lib
    return _lib


def key(seed: int, tag: int) -> int:
    return int(_library().gen_key(seed, tag))


def stream(key_: int, first: int, count: int) -> np.ndarray:
    """Raw SplitMix64 draws ``first .. first + count - 1`` of a stream."""
    out = np.empty(count, dtype=np.uint64)
    if count:
        _library().gen_stream(key_, first, count, out.ctypes.data)
    return out


def uniform(seed: int, n: int, num_bins: int, lo: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """int32 values ``lo + U[0, num_bins)`` from the seed's uniform stream."""
    if out is None:
        out = np.empty(n, dtype=np.int32)
    if n:
        _library().gen_uniform(key(seed, TAG_UNIFORM), 0, out.ctypes.data, n, lo, num_bins)
    return out


def zipf(seed: int, n: int, num_bins: int, s: float) -> np.ndarray:
    """int32 finite Zipf values: rank k in 1..num_bins with P(k) ~ k^-s, the
    ranks permuted to bins (the recipe of the 262,144-bin Zipf workload, any size and exponent)."""
    out = np.empty(n, dtype=np.int32)
    rc = _library().gen_zipf(seed, out.ctypes.data if n else None, n, num_bins, float(s))
    if rc != 0:
        raise RuntimeError(f"gen_zipf failed with {rc}")
    return out


def shuffle(seed: int, values: np.ndarray) -> np.ndarray:
    """Fisher-Yates shuffle in place (int32 array); returns the array."""
    assert values.dtype == np.int32 and values.flags.c_contiguous
    _library().gen_shuffle(key(seed, TAG_SHUFFLE), values.ctypes.data, values.size)
    return values


def generate(cfg: int, n: int | None = None, out: np.ndarray | None = None,
             return_aux: bool = False):
    """The workload ``cfg`` (1..5) at its published length, or at length ``n``."""
    w = WORKLOADS[cfg]
    n = w.n if n is None else int(n)
    if out is None:
        out = np.empty(n, dtype=np.int32)
    assert out.dtype == np.int32 and out.size == n and out.flags.c_contiguous
    aux = np.zeros(1, dtype=np.uint64)
    rc = _library().gen_config(cfg, out.ctypes.data if n else None, n, aux.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"gen_config({cfg}) failed with {rc}")
    return (out, int(aux[0])) if return_aux else out
