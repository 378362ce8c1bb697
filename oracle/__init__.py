"""CPU oracle for the partitioned on-chip histogram.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports, loads or calls it, and
the two share no code.

The arithmetic lives in ``oracle_hist.c`` (a plain sequential counting loop,
built with gcc); this module only builds and calls it. The definition it
follows is the page "Distributed Shared Memory", section "The cluster
histogram": each input element adds one to the bin it names, and the final
value of a bin is the sum of every block's private count for it, i.e. the
number of input elements equal to that bin.

Parity status: pinned. The tests check it against closed forms (empty input,
all elements in one bin), an independent sort-and-run-length count, a
brute-force per-bin comparison, the invariants sum(counts) + dropped == n,
permutation invariance and split additivity, and they show that planted
mistakes in copies of the C source fail those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_hist.c")
LIBRARY = os.path.join(_HERE, "liboracle_hist.so")

_lib = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (-O2, no vectorisation flags needed)."""
    tmp = output + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
         source, "-o", tmp],
        check=True,
    )
    os.replace(tmp, output)
    return output


def load(path: str = LIBRARY):
    lib = ctypes.CDLL(path)
    fn = lib.oracle_hist
    fn.restype = ctypes.c_uint64
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p]
    return lib


def _library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _lib = load()
    return _lib


def hist(values: np.ndarray, num_bins: int, lib=None) -> tuple[np.ndarray, int]:
    """Return ``(counts, dropped)`` for an int32 array.

    ``counts`` is a uint32 array of ``num_bins`` entries, ``counts[b]`` the
    number of elements equal to ``b``; ``dropped`` counts elements outside
    ``[0, num_bins)``.
    """
    lib = lib or _library()
    x = np.ascontiguousarray(values, dtype=np.int32)
    if num_bins <= 0:
        raise ValueError("num_bins must be positive")
    counts = np.empty(int(num_bins), dtype=np.uint32)
    dropped = lib.oracle_hist(
        x.ctypes.data if x.size else None, x.size, int(num_bins), counts.ctypes.data
    )
    if dropped == 2**64 - 1:
        raise ValueError("oracle_hist rejected its arguments")
    return counts, int(dropped)
