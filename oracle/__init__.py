"""CPU oracle for the strided, batched fp32 matrix product.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product library neither imports nor links it, and this package imports
nothing from the product: the two share no code.

The arithmetic lives in ``ref_sgemm.c`` (plain C, fp64 accumulation, one
output element at a time).  This module only compiles it with gcc, checks that
every operand view stays inside its host buffer, and passes pointers through
ctypes.

Definition (StaleyNET "GPU Implementation", section "The matrix product"):
for b < batch, i < m, j < n

    C[b,i,j] <- alpha * sum_{p<k} A[b,i,p] * B[b,p,j]  (+ C[b,i,j] if accumulate)

with X[b,r,c] = X_storage[b*sX_batch + r*sX_row + c*sX_col], strides counted in
elements.  Sums are formed in fp64 in ascending p and rounded to fp32 once.

The general epilogue (``ref_sgemm_ex``) adds beta * C_old (not read when
beta == 0), a per-row term r[b,i] and a per-column term c[b,j]; ``ref_sqnorms``
and ``ref_sqdist`` are squared Euclidean norms and distances from their plain
definitions; ``ref_sgemm_batched2`` takes two batch levels with grouped inputs,
and ``ref_attention`` is scaled dot-product attention (scores, softmax, times
V) over the same two levels.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref_sgemm.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_sgemm.so")

_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_int = ctypes.c_int
_fptr = ctypes.POINTER(ctypes.c_float)
_i64ptr = ctypes.POINTER(ctypes.c_int64)

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           *extra_flags, src, "-lm", "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    lib.oracle_sgemm.restype = _int
    lib.oracle_sgemm.argtypes = [
        _i64, _i64, _i64, _i64, _f32,
        _fptr, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64,
        _int,
        _fptr, _i64, _i64, _i64,
        _int,
    ]
    lib.oracle_sgemm_entries.restype = _int
    lib.oracle_sgemm_entries.argtypes = [
        _i64, _i64, _i64, _i64, _f32,
        _fptr, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64,
        _int,
        _fptr, _i64, _i64, _i64,
        _i64, _i64ptr, _fptr,
    ]
    ex_args = [
        _i64, _i64, _i64, _i64, _f32,
        _fptr, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64,
        _f32,
        _fptr, _i64, _i64, _i64,
        _fptr, _i64, _i64,
        _fptr, _i64, _i64,
    ]
    lib.oracle_sgemm_ex.restype = _int
    lib.oracle_sgemm_ex.argtypes = ex_args + [_int]
    lib.oracle_sgemm_ex_entries.restype = _int
    lib.oracle_sgemm_ex_entries.argtypes = ex_args + [_i64, _i64ptr, _fptr]
    lib.oracle_sqnorms.restype = _int
    lib.oracle_sqnorms.argtypes = [_i64, _i64, _i64, _fptr, _i64, _i64, _i64, _fptr, _i64, _i64]
    lib.oracle_sqdist.restype = _int
    lib.oracle_sqdist.argtypes = [_i64, _i64, _i64, _i64,
                                  _fptr, _i64, _i64, _i64,
                                  _fptr, _i64, _i64, _i64,
                                  _fptr, _i64, _i64, _i64,
                                  _i64, _i64ptr, _fptr]
    lib.oracle_sgemm_batched2.restype = _int
    lib.oracle_sgemm_batched2.argtypes = [
        _i64, _i64, _i64, _i64, _i64, _f32,
        _fptr, _i64, _i64, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64, _i64, _i64,
        _int,
        _fptr, _i64, _i64, _i64, _i64,
    ]
    lib.oracle_attention.restype = _int
    lib.oracle_attention.argtypes = [
        _i64, _i64, _i64, _i64, _i64, _f32, _int,
        _fptr, _i64, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64, _i64,
        _fptr, _i64, _i64, _i64, _i64,
    ]
    lib.oracle_num_threads.restype = _int
    lib.oracle_num_threads.argtypes = []
    return lib


def load_library(path: str):
    """Load an oracle build from `path` (used for the default build and for
    deliberately broken copies in the oracle's own mutation tests)."""
    return _bind(ctypes.CDLL(path))


def _get_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def _as_storage(x, name, writable=False):
    if not isinstance(x, np.ndarray) or x.dtype != np.float32 or x.ndim != 1:
        raise TypeError(f"{name} must be a 1-D float32 numpy array (the flat storage)")
    if not x.flags.c_contiguous:
        raise TypeError(f"{name} storage must be contiguous")
    if writable and not x.flags.writeable:
        raise TypeError(f"{name} must be writable")
    return x


def _check_view(storage, name, extents, strides):
    """Every element the view can address must lie inside `storage`."""
    if any(s < 0 for s in strides):
        raise ValueError(f"{name}: negative stride")
    if any(e == 0 for e in extents):
        return
    last = sum((e - 1) * s for e, s in zip(extents, strides))
    if last >= storage.size:
        raise ValueError(f"{name}: view reaches element {last}, storage has {storage.size}")


def _ptr(x):
    return x.ctypes.data_as(_fptr)


def ref_sgemm(batch, m, n, k, alpha,
              A, sA_batch, sA_row, sA_col,
              B, sB_batch, sB_row, sB_col,
              accumulate,
              C, sC_batch, sC_row, sC_col,
              reverse=False, lib=None):
    """C <- alpha*A*B (+C) over host storages; writes C in place."""
    lib = lib or _get_lib()
    A = _as_storage(A, "A")
    B = _as_storage(B, "B")
    C = _as_storage(C, "C", writable=True)
    if min(batch, m, n, k) < 0:
        raise ValueError("negative size")
    if batch and m and k:
        _check_view(A, "A", (batch, m, k), (sA_batch, sA_row, sA_col))
    if batch and n and k:
        _check_view(B, "B", (batch, k, n), (sB_batch, sB_row, sB_col))
    _check_view(C, "C", (batch, m, n), (sC_batch, sC_row, sC_col))
    rc = lib.oracle_sgemm(batch, m, n, k, float(alpha),
                          _ptr(A), sA_batch, sA_row, sA_col,
                          _ptr(B), sB_batch, sB_row, sB_col,
                          int(bool(accumulate)),
                          _ptr(C), sC_batch, sC_row, sC_col,
                          int(bool(reverse)))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm returned {rc}")
    return C


def ref_entries(batch, m, n, k, alpha,
                A, sA_batch, sA_row, sA_col,
                B, sB_batch, sB_row, sB_col,
                accumulate,
                C, sC_batch, sC_row, sC_col,
                idx, lib=None):
    """Return the float32 values the full product would store at the (b,i,j)
    rows of `idx` (shape [count, 3]); C is only read (as C_old)."""
    lib = lib or _get_lib()
    A = _as_storage(A, "A")
    B = _as_storage(B, "B")
    C = _as_storage(C, "C")
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
    if batch and m and k:
        _check_view(A, "A", (batch, m, k), (sA_batch, sA_row, sA_col))
    if batch and n and k:
        _check_view(B, "B", (batch, k, n), (sB_batch, sB_row, sB_col))
    if accumulate:
        _check_view(C, "C", (batch, m, n), (sC_batch, sC_row, sC_col))
    out = np.empty(idx.shape[0], dtype=np.float32)
    rc = lib.oracle_sgemm_entries(batch, m, n, k, float(alpha),
                                  _ptr(A), sA_batch, sA_row, sA_col,
                                  _ptr(B), sB_batch, sB_row, sB_col,
                                  int(bool(accumulate)),
                                  _ptr(C), sC_batch, sC_row, sC_col,
                                  idx.shape[0], idx.ctypes.data_as(_i64ptr), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_sgemm_entries: index outside the product")
    return out


def _opt_vector(v, name, batch, count, s_batch, s_item):
    """A NULL pointer for None, else the checked storage of a batch of
    vectors v[b*s_batch + i*s_item]."""
    if v is None:
        return None
    v = _as_storage(v, name)
    if batch and count:
        _check_view(v, name, (batch, count), (s_batch, s_item))
    return v


def _ex_args(batch, m, n, k, alpha, A, sA, B, sB, beta, C, sC, row_add, sR, col_add, sL):
    A = _as_storage(A, "A")
    B = _as_storage(B, "B")
    if min(batch, m, n, k) < 0:
        raise ValueError("negative size")
    if batch and m and k:
        _check_view(A, "A", (batch, m, k), sA)
    if batch and n and k:
        _check_view(B, "B", (batch, k, n), sB)
    _check_view(C, "C", (batch, m, n), sC)
    row_add = _opt_vector(row_add, "row_add", batch, m, *sR)
    col_add = _opt_vector(col_add, "col_add", batch, n, *sL)
    nul = ctypes.cast(None, _fptr)
    return [batch, m, n, k, float(alpha), _ptr(A), *sA, _ptr(B), *sB, float(beta), _ptr(C), *sC,
            _ptr(row_add) if row_add is not None else nul, *sR,
            _ptr(col_add) if col_add is not None else nul, *sL]


def ref_sgemm_ex(batch, m, n, k, alpha, A, sA, B, sB, beta, C, sC,
                 row_add=None, sR=(0, 0), col_add=None, sL=(0, 0), reverse=False, lib=None):
    """C <- alpha*A*B + beta*C + row_add[b,i] + col_add[b,j] over host
    storages (each s* a stride tuple: (batch, row, col) for the matrices,
    (batch, index) for the vectors); writes C in place.  beta == 0 never
    reads C; a vector given as None drops its term."""
    lib = lib or _get_lib()
    C = _as_storage(C, "C", writable=True)
    args = _ex_args(batch, m, n, k, alpha, A, sA, B, sB, beta, C, sC, row_add, sR, col_add, sL)
    rc = lib.oracle_sgemm_ex(*args, int(bool(reverse)))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_ex returned {rc}")
    return C


def ref_sgemm_ex_entries(batch, m, n, k, alpha, A, sA, B, sB, beta, C, sC, idx,
                         row_add=None, sR=(0, 0), col_add=None, sL=(0, 0), lib=None):
    """Values ref_sgemm_ex would store at the (b,i,j) rows of `idx`; C is
    only read (as C_old, when beta != 0)."""
    lib = lib or _get_lib()
    C = _as_storage(C, "C")
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
    args = _ex_args(batch, m, n, k, alpha, A, sA, B, sB, beta, C, sC, row_add, sR, col_add, sL)
    out = np.empty(idx.shape[0], dtype=np.float32)
    rc = lib.oracle_sgemm_ex_entries(*args, idx.shape[0], idx.ctypes.data_as(_i64ptr), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_sgemm_ex_entries: index outside the product")
    return out


def ref_sqnorms(batch, count, length, X, sX, out, sO, lib=None):
    """out[b*sO[0] + i*sO[1]] = sum_p X[b,i,p]^2 for X strides sX =
    (batch, item, element); writes out in place."""
    lib = lib or _get_lib()
    X = _as_storage(X, "X")
    out = _as_storage(out, "out", writable=True)
    if min(batch, count, length) < 0:
        raise ValueError("negative size")
    if batch and count and length:
        _check_view(X, "X", (batch, count, length), sX)
    if batch and count:
        _check_view(out, "out", (batch, count), sO)
    rc = lib.oracle_sqnorms(batch, count, length, _ptr(X), *sX, _ptr(out), *sO)
    if rc != 0:
        raise RuntimeError(f"oracle_sqnorms returned {rc}")
    return out


def _sqdist_views(batch, m, n, k, X, sX, Y, sY):
    X = _as_storage(X, "X")
    Y = _as_storage(Y, "Y")
    if min(batch, m, n, k) < 0:
        raise ValueError("negative size")
    if batch and m and k:
        _check_view(X, "X", (batch, m, k), sX)
    if batch and n and k:
        _check_view(Y, "Y", (batch, n, k), sY)
    return X, Y


def ref_sqdist(batch, m, n, k, X, sX, Y, sY, D, sD, lib=None):
    """D[b,i,j] = sum_p (X[b,i,p] - Y[b,j,p])^2 (rows of X against rows of
    Y, both [batch][rows][k] views); writes D in place."""
    lib = lib or _get_lib()
    X, Y = _sqdist_views(batch, m, n, k, X, sX, Y, sY)
    D = _as_storage(D, "D", writable=True)
    _check_view(D, "D", (batch, m, n), sD)
    rc = lib.oracle_sqdist(batch, m, n, k, _ptr(X), *sX, _ptr(Y), *sY, _ptr(D), *sD,
                           0, ctypes.cast(None, _i64ptr), ctypes.cast(None, _fptr))
    if rc != 0:
        raise RuntimeError(f"oracle_sqdist returned {rc}")
    return D


def ref_sqdist_entries(batch, m, n, k, X, sX, Y, sY, idx, lib=None):
    """Distances at the (b,i,j) rows of `idx` only."""
    lib = lib or _get_lib()
    X, Y = _sqdist_views(batch, m, n, k, X, sX, Y, sY)
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
    out = np.empty(idx.shape[0], dtype=np.float32)
    nul = ctypes.cast(None, _fptr)
    rc = lib.oracle_sqdist(batch, m, n, k, _ptr(X), *sX, _ptr(Y), *sY, nul, 0, 0, 0,
                           idx.shape[0], idx.ctypes.data_as(_i64ptr), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_sqdist: index outside the table")
    return out


def ref_sgemm_batched2(nb_outer, nb_inner, m, n, k, alpha,
                       A, sA_outer, sA_inner, gA, sA_row, sA_col,
                       B, sB_outer, sB_inner, gB, sB_row, sB_col,
                       accumulate,
                       C, sC_outer, sC_inner, sC_row, sC_col, lib=None):
    """Two batch levels with group divisors on the inner level of A and B:
    C[o,i] <- alpha * A[o, i/gA] @ B[o, i/gB] (+ C); writes C in place."""
    lib = lib or _get_lib()
    A = _as_storage(A, "A")
    B = _as_storage(B, "B")
    C = _as_storage(C, "C", writable=True)
    if min(nb_outer, nb_inner, m, n, k) < 0 or gA < 1 or gB < 1:
        raise ValueError("negative size or group below 1")
    inner_a = -(-nb_inner // gA) if nb_inner else 0
    inner_b = -(-nb_inner // gB) if nb_inner else 0
    if nb_outer and inner_a and m and k:
        _check_view(A, "A", (nb_outer, inner_a, m, k), (sA_outer, sA_inner, sA_row, sA_col))
    if nb_outer and inner_b and n and k:
        _check_view(B, "B", (nb_outer, inner_b, k, n), (sB_outer, sB_inner, sB_row, sB_col))
    _check_view(C, "C", (nb_outer, nb_inner, m, n), (sC_outer, sC_inner, sC_row, sC_col))
    rc = lib.oracle_sgemm_batched2(nb_outer, nb_inner, m, n, k, float(alpha),
                                   _ptr(A), sA_outer, sA_inner, gA, sA_row, sA_col,
                                   _ptr(B), sB_outer, sB_inner, gB, sB_row, sB_col,
                                   int(bool(accumulate)),
                                   _ptr(C), sC_outer, sC_inner, sC_row, sC_col)
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_batched2 returned {rc}")
    return C


def ref_attention(nb_outer, nb_inner, tq, tk, d, alpha, causal,
                  Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                  K, sK_outer, sK_inner, g, sK_row, sK_col,
                  V, sV_outer, sV_inner, sV_row, sV_col,
                  O, sO_outer, sO_inner, sO_row, sO_col, lib=None):
    """O[o,i] <- softmax(alpha * Q[o,i] K[o,i//g]^T (causal: query q sees keys
    j <= q + tk - tq)) V[o,i//g], row by row in fp64; writes O in place."""
    lib = lib or _get_lib()
    Q, K, V = _as_storage(Q, "Q"), _as_storage(K, "K"), _as_storage(V, "V")
    O = _as_storage(O, "O", writable=True)
    if min(nb_outer, nb_inner, tq, tk, d) < 0 or g < 1:
        raise ValueError("negative size or group below 1")
    kv = -(-nb_inner // g) if nb_inner else 0
    _check_view(Q, "Q", (nb_outer, nb_inner, tq, d), (sQ_outer, sQ_inner, sQ_row, sQ_col))
    _check_view(K, "K", (nb_outer, kv, tk, d), (sK_outer, sK_inner, sK_row, sK_col))
    _check_view(V, "V", (nb_outer, kv, tk, d), (sV_outer, sV_inner, sV_row, sV_col))
    _check_view(O, "O", (nb_outer, nb_inner, tq, d), (sO_outer, sO_inner, sO_row, sO_col))
    rc = lib.oracle_attention(nb_outer, nb_inner, tq, tk, d, float(alpha), int(bool(causal)),
                              _ptr(Q), sQ_outer, sQ_inner, sQ_row, sQ_col,
                              _ptr(K), sK_outer, sK_inner, g, sK_row, sK_col,
                              _ptr(V), sV_outer, sV_inner, sV_row, sV_col,
                              _ptr(O), sO_outer, sO_inner, sO_row, sO_col)
    if rc != 0:
        raise RuntimeError(f"oracle_attention returned {rc}")
    return O


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return (lib or _get_lib()).oracle_num_threads()
