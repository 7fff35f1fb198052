"""Python front end of the CPU oracle (``csa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The GPU library and
its binding never import this module.

The oracle computes the Compressed Sparse Attention lightning-indexer top-k the
plain way (page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
Streaming Top-k", Abstract: score compressed keys with the indexer, keep the
top-k per query; the materialise path is the ground truth).  It runs one query
row at a time, in fp32 with a fixed summation order, and sorts the whole row.
See ``csa_oracle.c`` for the exact definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "libcsa_oracle.so")

# -ffp-contract=off: no fused multiply-add; no -ffast-math: no reassociation.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-pthread"]

_lib = None


def compile_source(src: str, out: str) -> str:
    """Compile one oracle source file into a shared library with gcc."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``libcsa_oracle.so`` next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def open_library(path: str):
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.csa_oracle_topk.argtypes = [f32p, f32p, f32p, i64p, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int64, i32p, f32p,
                                    ctypes.c_int32]
    lib.csa_oracle_topk.restype = ctypes.c_int
    lib.csa_oracle_row_scores.argtypes = [f32p, f32p, f32p, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_int32, f32p]
    lib.csa_oracle_row_scores.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = open_library(_LIB)
    return _lib


def _f32(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def n_valid(pos, T: int, m: int):
    """Keys usable by the query at absolute position ``pos``: key j counts
    iff (j+1)*m <= pos+1, capped by the T keys that exist."""
    p = np.asarray(pos, dtype=np.int64)
    return np.minimum(np.int64(T), np.maximum((p + 1) // m, 0))


def topk(q, w, kc, m: int, k: int, pos=None, q_pos0: int = 0, nthreads: int | None = None,
         lib=None):
    """Oracle top-k.

    q  [R, H, D], w [R, H], kc [T, D]: float arrays (bf16 data must already be
    upcast exactly to fp32).  ``pos`` gives the absolute position of each of
    the R rows; by default rows are consecutive from ``q_pos0``.
    Returns (idx [R, k] int32, score [R, k] float32).
    """
    q = _f32(q)
    w = _f32(w)
    kc = _f32(kc)
    if q.ndim != 3 or w.ndim != 2 or kc.ndim != 2:
        raise ValueError("q must be [R,H,D], w [R,H], kc [T,D]")
    R, H, D = q.shape
    T = kc.shape[0]
    if w.shape != (R, H) or (T > 0 and kc.shape[1] != D):
        raise ValueError("shape mismatch")
    if pos is None:
        pos = np.arange(R, dtype=np.int64) + q_pos0
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    if pos.shape != (R,):
        raise ValueError("pos must have one entry per row")
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    idx = np.empty((R, k), dtype=np.int32)
    score = np.empty((R, k), dtype=np.float32)
    if R == 0:
        return idx, score
    kc_arg = kc if T > 0 else np.zeros((1, D), dtype=np.float32)
    rc = (lib or _load()).csa_oracle_topk(_ptr(q, ctypes.c_float), _ptr(w, ctypes.c_float),
                                 _ptr(kc_arg, ctypes.c_float), _ptr(pos, ctypes.c_int64),
                                 R, T, H, D, m, k, _ptr(idx, ctypes.c_int32),
                                 _ptr(score, ctypes.c_float), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    return idx, score


def row_scores(q_row, w_row, kc, n: int, lib=None) -> np.ndarray:
    """fp32 scores of one query row (q_row [H, D], w_row [H]) for keys 0..n-1."""
    q_row = _f32(q_row)
    w_row = _f32(w_row)
    kc = _f32(kc)
    H, D = q_row.shape
    out = np.empty((n,), dtype=np.float32)
    kc_arg = kc if kc.size else np.zeros((1, D), dtype=np.float32)
    rc = (lib or _load()).csa_oracle_row_scores(_ptr(q_row, ctypes.c_float), _ptr(w_row, ctypes.c_float),
                                       _ptr(kc_arg, ctypes.c_float), n, H, D,
                                       _ptr(out, ctypes.c_float))
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    return out
