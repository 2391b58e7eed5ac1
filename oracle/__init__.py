"""CPU oracle for the fixed-order fold -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never imports it.

The arithmetic lives in ``oracle.c`` (plain serial loops, gcc
``-O2 -ffp-contract=off``, no fast-math); this module only marshals numpy
arrays.  What it computes (mamba-rs ``src/dist/reducer.rs``: the
FixedOrder-contract module note, the ``det_sum_ranks`` kernel source and
``reduce_sum_reference``; memra-engine ``tests/tp_ar_gpu.rs``:
``memra_tp_ar_fold``):

* ``fold(slots)``                       -- ``acc = s_0; acc = acc + s_r`` for r
  ascending, each ``+`` one binary32 round-to-nearest-even addition,
  subnormals kept.
* ``fold_stacked(stacked)``             -- ``fold`` over the rows of a ``[W, len]``
  array (row r = slot r).
* ``fold_stacked_scaled(stacked, inv_w)`` -- the same sum, then one binary32
  multiply by ``inv_w`` (the caller's inverse world size).
* ``fold_into(dst, stage)``             -- ``dst + stage`` elementwise.

Pins (tests/test_oracle_pins.py): exact-rational brute force with an explicit
round-to-nearest-even, the binary64 double-path, hand-derived IEEE 754 cases in
``tests/golden/``, closed forms (doubling, power-of-two scale, exact sums of
the uniform generator) and planted-mistake mutants that the pins must reject.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build_lib() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc, contraction off)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(
        ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-msse2", "-mfpmath=sse",
         "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC],
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
    lib.oracle_fold_slots.argtypes = [f32p, ctypes.POINTER(f32p), ctypes.c_int32, ctypes.c_int64]
    lib.oracle_fold_stacked.argtypes = [f32p, f32p, ctypes.c_int32, ctypes.c_int64]
    lib.oracle_fold_stacked_scaled.argtypes = [f32p, f32p, ctypes.c_int32, ctypes.c_int64,
                                               ctypes.c_float]
    lib.oracle_fold_into.argtypes = [f32p, f32p, ctypes.c_int64]
    for fn in (lib.oracle_fold_slots, lib.oracle_fold_stacked,
               lib.oracle_fold_stacked_scaled, lib.oracle_fold_into):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _fp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _as_f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle inputs must be float32, got %s" % a.dtype)
    return np.ascontiguousarray(a)


def _as_stacked(stacked) -> np.ndarray:
    s = _as_f32(stacked)
    if s.ndim != 2 or s.shape[0] < 1:
        raise ValueError("stacked must be [W, len] with W >= 1")
    return s


def fold(slots: Sequence[np.ndarray]) -> np.ndarray:
    """Fixed-order fold of W equal-length float32 slots (W >= 1)."""
    arrs = [_as_f32(s).reshape(-1) for s in slots]
    if not arrs:
        raise ValueError("need at least one addend")
    n = arrs[0].size
    if any(a.size != n for a in arrs):
        raise ValueError("addend length mismatch")
    out = np.empty(n, dtype=np.float32)
    ptrs = (ctypes.POINTER(ctypes.c_float) * len(arrs))(*[_fp(a) for a in arrs])
    rc = _load().oracle_fold_slots(_fp(out), ptrs, len(arrs), n)
    if rc != 0:
        raise ValueError("oracle_fold_slots rc=%d" % rc)
    return out


def fold_stacked(stacked) -> np.ndarray:
    """Fixed-order fold of the rows of a ``[W, len]`` float32 array."""
    s = _as_stacked(stacked)
    out = np.empty(s.shape[1], dtype=np.float32)
    rc = _load().oracle_fold_stacked(_fp(out), _fp(s), s.shape[0], s.shape[1])
    if rc != 0:
        raise ValueError("oracle_fold_stacked rc=%d" % rc)
    return out


def fold_stacked_scaled(stacked, inv_w) -> np.ndarray:
    """Fold of the rows, then one binary32 multiply by ``inv_w``."""
    s = _as_stacked(stacked)
    w = np.float32(inv_w)
    out = np.empty(s.shape[1], dtype=np.float32)
    rc = _load().oracle_fold_stacked_scaled(_fp(out), _fp(s), s.shape[0], s.shape[1],
                                            float(w))
    if rc != 0:
        raise ValueError("oracle_fold_stacked_scaled rc=%d" % rc)
    return out


def fold_into(dst, stage) -> np.ndarray:
    """Return ``dst + stage`` (binary32, elementwise) as a new array."""
    d = _as_f32(dst).reshape(-1).copy()
    s = _as_f32(stage).reshape(-1)
    if d.size != s.size:
        raise ValueError("length mismatch")
    rc = _load().oracle_fold_into(_fp(d), _fp(s), d.size)
    if rc != 0:
        raise ValueError("oracle_fold_into rc=%d" % rc)
    return d
