"""Plain float64 CPU oracle for head-major, non-causal attention.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``non_causal_flash_amd``) never imports, links or calls it.

The arithmetic lives in ``vattn_oracle.c`` (plain C, float64, OpenMP over
independent rows) and follows the docs.rs page "rullama 0.1.0",
src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl: per head,
``out = softmax(Q K^T) V`` row-wise over every patch, no scale inside, tensors
laid out ``[n_heads][n_patches][head_dim]``.  ``rope_neox_f64`` is the NeoX
rotary transform of the docs.rs page "rullama 0.2.0",
src/kernels/wgsl/rope_neox_backward.wgsl (forward rotation of its header
comment, angle of its main function), one position per patch.  This module
only compiles that file with gcc and marshals numpy arrays into it; inputs
of any float type are promoted to float64 exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``vattn_oracle.c`` into ``oracle/liboracle.so`` with gcc."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        cl = ctypes.c_long
        lib.vattn_oracle_f64.argtypes = [dp, dp, dp, dp, cl, cl, cl, ctypes.c_int]
        lib.vattn_oracle_f64.restype = ctypes.c_int
        lib.vattn_oracle_rows_f64.argtypes = [dp, dp, dp, cl, cl, cl, lp, cl, dp,
                                              ctypes.c_int]
        lib.vattn_oracle_rows_f64.restype = ctypes.c_int
        lib.vattn_oracle_rope_f64.argtypes = [dp, dp, cl, cl, cl, cl, ctypes.c_double,
                                              dp, cl]
        lib.vattn_oracle_rope_f64.restype = ctypes.c_int
        _lib = lib
    return _lib


def _as_f64(x):
    """Exact float64 copy (float16 / float32 / float64 inputs)."""
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError("expected a float16, float32 or float64 array")
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.ndim != 3:
        raise ValueError("expected a [n_heads][n_patches][head_dim] array")
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def attention_f64(q, k, v, n_threads: int = 0) -> np.ndarray:
    """Full ``[H][N][d]`` float64 result of softmax(Q K^T) V per head."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must share one [H][N][d] shape")
    h, n, d = q.shape
    out = np.empty((h, n, d), dtype=np.float64)
    rc = _load().vattn_oracle_f64(_ptr(q, ctypes.c_double),
                                  _ptr(k, ctypes.c_double),
                                  _ptr(v, ctypes.c_double),
                                  _ptr(out, ctypes.c_double), h, n, d,
                                  int(n_threads))
    if rc != 0:
        raise RuntimeError("vattn_oracle_f64 failed with status %d" % rc)
    return out


def attention_rows_f64(q, k, v, rows, n_threads: int = 0) -> np.ndarray:
    """Rows ``rows[r] = h * N + i`` of the result, as float64 ``[R][d]``."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must share one [H][N][d] shape")
    h, n, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), dtype=np.float64)
    rc = _load().vattn_oracle_rows_f64(_ptr(q, ctypes.c_double),
                                       _ptr(k, ctypes.c_double),
                                       _ptr(v, ctypes.c_double), h, n, d,
                                       _ptr(rows, ctypes.c_long), rows.size,
                                       _ptr(out, ctypes.c_double),
                                       int(n_threads))
    if rc != 0:
        raise RuntimeError("vattn_oracle_rows_f64 failed with status %d" % rc)
    return out


def rope_neox_f64(x, rope_dims: int, base: float = 10000.0, factors=None,
                  pos_offset: int = 0) -> np.ndarray:
    """NeoX rotary transform of a ``[H][N][d]`` array in float64: patch n of
    every head sits at position ``pos_offset + n``; pairs (i, i + rope_dims/2)
    are rotated by pos * base^(-2i/rope_dims) (divided by ``factors[i]`` when
    given); dimensions from ``rope_dims`` on are copied unchanged."""
    x = _as_f64(x)
    h, n, d = x.shape
    y = np.empty_like(x)
    fac = None
    if factors is not None:
        fac = np.ascontiguousarray(factors, dtype=np.float64)
        if fac.shape != (int(rope_dims) // 2,):
            raise ValueError("factors must hold rope_dims/2 values")
    rc = _load().vattn_oracle_rope_f64(_ptr(x, ctypes.c_double), _ptr(y, ctypes.c_double),
                                       h, n, d, int(rope_dims), float(base),
                                       None if fac is None else _ptr(fac, ctypes.c_double),
                                       int(pos_offset))
    if rc != 0:
        raise ValueError("vattn_oracle_rope_f64 rejected its arguments (status %d)" % rc)
    return y
