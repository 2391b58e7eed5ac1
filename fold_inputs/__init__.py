"""Seeded synthetic inputs for the fixed-order fold (no fold arithmetic here).

The same module feeds the CPU oracle's tests and the GPU path's tests and
bench, so both sides fold identical bits.  The value families and their
seeding follow the generators printed on the pages:

* ``vecf``   -- memra-engine ``tests/tp_ar_gpu.rs``, helper ``vecf``: uniform
  multiples of 2^-23 in [-1, 1).
* ``varied`` -- memra-engine ``tests/gdn_packed_gpu.rs``, helper ``varied``:
  full-mantissa values in [-spread, spread).
* ``mixed``  -- sign random, binary exponent uniform in [-20, 20], mantissa
  uniform (the gradient-arena input family with mixed magnitudes).

Multi-slot fills draw slot ``r`` with seed ``seed0 + r``.  The generators are
C (``gen.c``) because the large arenas hold up to 4e8 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libfoldgen.so")

FAMILIES = {"vecf": 0, "varied": 1, "mixed": 2}

_lib = None


def build_lib() -> str:
    """Compile ``gen.c`` into ``libfoldgen.so`` next to it (gcc, no fast-math)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(
        ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC],
        check=True,
    )
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build_lib()
    lib = ctypes.CDLL(_LIB)
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.gen_vecf.argtypes = [f32p, ctypes.c_int64, ctypes.c_uint64]
    lib.gen_vecf.restype = None
    lib.gen_varied.argtypes = [f32p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float]
    lib.gen_varied.restype = None
    lib.gen_mixed.argtypes = [f32p, ctypes.c_int64, ctypes.c_uint64]
    lib.gen_mixed.restype = None
    lib.gen_slots.argtypes = [ctypes.c_int, f32p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                              ctypes.c_int32]
    lib.gen_slots.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def vecf(n: int, seed: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().gen_vecf(_ptr(out), n, seed & (2**64 - 1))
    return out


def varied(n: int, seed: int, spread: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().gen_varied(_ptr(out), n, seed & (2**64 - 1), spread)
    return out


def mixed(n: int, seed: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().gen_mixed(_ptr(out), n, seed & (2**64 - 1))
    return out


def slots(family: str, W: int, length: int, seed0: int, spread: float = 1.0,
          out: np.ndarray | None = None) -> np.ndarray:
    """Return (or fill) a C-contiguous ``[W, length]`` float32 array; slot r
    is drawn with seed ``seed0 + r``."""
    if out is None:
        out = np.empty((W, length), dtype=np.float32)
    if out.dtype != np.float32 or out.shape != (W, length) or not out.flags.c_contiguous:
        raise ValueError("out must be a C-contiguous float32 [W, length] array")
    rc = _load().gen_slots(FAMILIES[family], _ptr(out), W, length, length,
                           seed0 & (2**64 - 1), spread, _threads())
    if rc != 0:
        raise ValueError("gen_slots rejected its arguments")
    return out
