"""The oracle: a plain, slow, obviously correct CPU GEMM (see ``oracle.c``),
and the row sums of the hazard demonstrator (``row_sums``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library under ``software_pipelined_tiled_loop_amd/`` and imports
nothing from it; both sides receive the same seeded inputs from
``software_pipelined_tiled_loop_amd.inputs``, which holds no GEMM arithmetic.

Definition followed (page "Double Buffering: Software Pipelining the K-Loop",
section "The Kernel"; general leading dimensions added):

    C = alpha * A @ B + beta * C0     (row-major, per-element sum in increasing k)

Float inputs are decoded exactly to double and summed in double; int8 is summed
in exact integers and stored modulo 2^32.  beta == 0 never reads C0.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, exact rational brute force and independent library decoders.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_KIND = {"f32": 0, "f16": 1, "bf16": 2}


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_gemm_float.argtypes = [ctypes.c_int, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64,
                                      vp, i64, vp]
    lib.oracle_gemm_float.restype = ctypes.c_int
    lib.oracle_gemm_i8.argtypes = [i64, i64, i64, i64, vp, i64, vp, i64, i64, vp, i64, vp, i64,
                                   ctypes.POINTER(i64)]
    lib.oracle_gemm_i8.restype = i64
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f16.restype = dbl
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = dbl
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(LIB_PATH)
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def decode_f16(bits: int) -> float:
    return float(_load().oracle_decode_f16(int(bits) & 0xFFFF))


def decode_bf16(bits: int) -> float:
    return float(_load().oracle_decode_bf16(int(bits) & 0xFFFF))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _runs(rows):
    """Split a row list into runs of consecutive rows: (output offset, first row, length)."""
    out, start = [], 0
    rows = [int(r) for r in rows]
    while start < len(rows):
        end = start + 1
        while end < len(rows) and rows[end] == rows[end - 1] + 1:
            end += 1
        out.append((start, rows[start], end - start))
        start = end
    return out


def _check_2d(name, a, rows, min_ld, dtype):
    if a.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, a.dtype))
    if a.ndim != 2 or not a.flags.c_contiguous:
        raise ValueError("%s must be a C-contiguous 2-D array (rows x leading dimension)" % name)
    if a.shape[0] < rows or a.shape[1] < min_ld:
        raise ValueError("%s is %s, needs at least %d x %d" % (name, a.shape, rows, min_ld))


def gemm(dtype: str, M: int, N: int, K: int, alpha, A: np.ndarray, B: np.ndarray,
         beta=0.0, C0: np.ndarray | None = None, rows=None, lib=None):
    """Reference C = alpha*A@B + beta*C0.

    dtype: "f32" (A, B float32), "f16"/"bf16" (A, B uint16 raw bits), "i8" (A, B int8).
    A is (>=M) x lda, B is (>=K) x ldb, C0 is (>=M) x ldc (float32, or int32 for i8);
    the leading dimension of each is its second extent.  ``rows`` optionally
    restricts the computation to a list/range of output rows (used to sample
    large problems); the result then has len(rows) rows.  ``lib`` substitutes
    another build of oracle.c (the mutation tests use it).
    Returns float64 (M x N) for float dtypes and int32 (M x N) for i8.
    """
    lib = _load() if lib is None else lib
    row_sel = None if rows is None else np.asarray(list(rows), dtype=np.int64)
    if dtype == "i8":
        _check_2d("A", A, M, K, np.int8)
        _check_2d("B", B, K, N, np.int8)
        if int(alpha) != alpha or int(beta) != beta:
            raise ValueError("int8 GEMM takes integer alpha and beta")
        alpha_i, beta_i = int(alpha), int(beta)
        if beta_i != 0:
            _check_2d("C0", C0, M, N, np.int32)
        c0 = C0 if beta_i != 0 else np.zeros((1, 1), np.int32)
        ldc = c0.shape[1]
        if row_sel is None:
            out = np.empty((M, N), np.int32)
            ovf = ctypes.c_int64(0)
            r = lib.oracle_gemm_i8(M, N, K, alpha_i, _ptr(A), A.shape[1], _ptr(B), B.shape[1], beta_i,
                                   _ptr(c0), ldc, _ptr(out), N, ctypes.byref(ovf))
            if r < 0:
                raise ValueError("oracle rejected arguments")
            gemm.last_overflow = (int(r), int(ovf.value))
            return out
        out = np.empty((len(row_sel), N), np.int32)
        tot = [0, 0]
        for start, i0, n in _runs(row_sel):
            ovf = ctypes.c_int64(0)
            r = lib.oracle_gemm_i8(n, N, K, alpha_i, _ptr(A) + i0 * A.shape[1], A.shape[1], _ptr(B),
                                   B.shape[1], beta_i, _ptr(c0) + (i0 * ldc * 4 if beta_i else 0), ldc,
                                   _ptr(out) + start * N * 4, N, ctypes.byref(ovf))
            if r < 0:
                raise ValueError("oracle rejected arguments")
            tot[0] += int(r)
            tot[1] += int(ovf.value)
        gemm.last_overflow = tuple(tot)
        return out

    if dtype not in _KIND:
        raise ValueError("unknown dtype %r" % dtype)
    kind = _KIND[dtype]
    in_dt = np.float32 if dtype == "f32" else np.uint16
    _check_2d("A", A, M, K, in_dt)
    _check_2d("B", B, K, N, in_dt)
    beta = float(beta)
    if beta != 0.0:
        _check_2d("C0", C0, M, N, np.float32)
    c0 = C0 if beta != 0.0 else np.zeros((1, 1), np.float32)
    ldc = c0.shape[1]
    esz = A.itemsize
    if row_sel is None:
        out = np.empty((M, N), np.float64)
        r = lib.oracle_gemm_float(kind, M, N, K, float(alpha), _ptr(A), A.shape[1], _ptr(B), B.shape[1],
                                  beta, _ptr(c0), ldc, _ptr(out), N, None)
        if r < 0:
            raise ValueError("oracle rejected arguments")
        return out
    out = np.empty((len(row_sel), N), np.float64)
    for start, i0, n in _runs(row_sel):
        r = lib.oracle_gemm_float(kind, n, N, K, float(alpha), _ptr(A) + i0 * A.shape[1] * esz,
                                  A.shape[1], _ptr(B), B.shape[1], beta,
                                  _ptr(c0) + (i0 * ldc * 4 if beta != 0.0 else 0), ldc,
                                  _ptr(out) + start * N * 8, N, None)
        if r < 0:
            raise ValueError("oracle rejected arguments")
    return out


gemm.last_overflow = (0, 0)


def row_sums(X: np.ndarray, rows: int, cols: int, ldx: int | None = None) -> np.ndarray:
    """Row sums of a row-major int32 array with leading dimension ldx, wrapped
    to int32 (two's complement).

    This is the deterministic reduction that consumes each stage of the
    copy-and-reduce of page "Software pipelines and asynchronous copies",
    section "Practice": every element X[r, c] with c < cols enters the sum of
    row r exactly once; padding columns (cols <= c < ldx) never do.  Each row
    is summed exactly in int64 (|sum| < 2^63 for any int32 row shorter than
    2^32) and then reduced modulo 2^32.
    """
    ldx = cols if ldx is None else ldx
    flat = np.ascontiguousarray(X, dtype=np.int32).reshape(-1)
    if rows and flat.size < (rows - 1) * ldx + cols:
        raise ValueError("X holds %d elements, rows/cols/ldx need %d" % (flat.size, (rows - 1) * ldx + cols))
    out = np.empty(rows, np.int32)
    for r in range(rows):
        s = int(flat[r * ldx:r * ldx + cols].astype(np.int64).sum())
        out[r] = (s + 2 ** 31) % 2 ** 32 - 2 ** 31
    return out
