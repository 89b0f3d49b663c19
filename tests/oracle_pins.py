"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Each `pin_*` takes an oracle library handle (the default build, or a
deliberately broken copy in the mutation tests) and raises AssertionError on a
mismatch.  None of them re-types the oracle's sum: they use closed forms
(all-ones gives k*alpha), identities, the pages' printed worked examples
(tests/golden/), exact integer brute force checked by numpy's int64 matmul,
numpy's float64 matmul on strided views, and invariants the definition
implies (stride exchange, C^T = B^T A^T, batch slicing, broadcast,
accumulation, order independence).
"""
from __future__ import annotations

import numpy as np

import oracle
from helpers import view, load_golden, ints, column_major_strides
from strided_fp32_gemm_amd.workloads import random_problem, layout_strides

LAYOUTS = [(a, b) for a in ("row", "col") for b in ("row", "col")]


def _run(p, lib, C=None, reverse=False):
    C = p.C.storage.copy() if C is None else C
    oracle.ref_sgemm(*p.call_args(p.A.storage, p.B.storage, C), reverse=reverse, lib=lib)
    return C


def _out(p, C):
    return np.array(view(C, p.batch, p.m, p.n, p.C.strides))


def _mat_problem(A2, B2, a_major="row", b_major="row", alpha=1.0):
    """Problem over explicit 2-D logical matrices stored in the given orders."""
    from strided_fp32_gemm_amd.workloads import Operand, Problem
    m, k = A2.shape
    _, n = B2.shape

    def store(M, major):
        r, c = M.shape
        if major == "row":
            return Operand(np.ascontiguousarray(M, np.float32).ravel(), (r * c, c, 1))
        return Operand(np.ascontiguousarray(M.T, np.float32).ravel(), (r * c, 1, r))
    return Problem("mat", 1, m, n, k, alpha, False, store(A2, a_major), store(B2, b_major),
                   Operand(np.zeros(max(m * n, 1), np.float32), (m * n, n, 1)))


# ---------------------------------------------------------------- closed forms

def pin_all_ones(lib):
    """A = 1, B = 1 => C = k*alpha exactly (+ C_old); every transpose case."""
    for a_major, b_major in LAYOUTS:
        for k in (1, 7, 64, 960, 4096):
            for alpha in (1.0, 0.5):
                for acc in (False, True):
                    p = random_problem(k, 2, 3, 5, k, a_major=a_major, b_major=b_major,
                                       alpha=alpha, accumulate=acc, dist="ones")
                    C = _run(p, lib)
                    c_old = view(p.C.storage, 2, 3, 5, p.C.strides).astype(np.float64)
                    want = (c_old if acc else 0.0) + k * alpha
                    got = _out(p, C)
                    assert np.array_equal(got, np.float32(want) + np.zeros_like(got)), \
                        (a_major, b_major, k, alpha, acc)


def pin_identity(lib):
    """A I = A and I B = B, bitwise, with each operand in both orientations."""
    rng = np.random.default_rng(7)
    A = rng.standard_normal((6, 9)).astype(np.float32)
    for a_major in ("row", "col"):
        for i_major in ("row", "col"):
            p = _mat_problem(A, np.eye(9, dtype=np.float32), a_major, i_major)
            assert np.array_equal(_out(p, _run(p, lib))[0], A), ("A I", a_major, i_major)
            p = _mat_problem(np.eye(6, dtype=np.float32), A, i_major, a_major)
            assert np.array_equal(_out(p, _run(p, lib))[0], A), ("I B", i_major, a_major)


def pin_k_zero(lib):
    """k = 0 is the empty sum: C <- 0, or C unchanged when accumulating."""
    for acc in (False, True):
        p = random_problem(3, 2, 4, 5, 0, accumulate=acc)
        C = _run(p, lib)
        want = view(p.C.storage, 2, 4, 5, p.C.strides) if acc else 0.0
        assert np.array_equal(_out(p, C), np.zeros((2, 4, 5), np.float32) + want), acc


# ---------------------------------------------------- the pages' worked values

def pin_golden_transpose_trace(lib):
    """kael ch. 09, "Moving tensors between devices": x.T of 0..5 read with
    strides (1, 3) and copied contiguously is 0 3 1 4 2 5."""
    g = load_golden("kael_transpose_trace.txt")
    storage = np.array(ints(g["storage"]), np.float32)
    rows, cols = ints(g["transposed_shape"])
    s_row, s_col = ints(g["transposed_strides"])
    from strided_fp32_gemm_amd.workloads import Operand, Problem
    p = Problem("trace", 1, rows, cols, cols, 1.0, False,
                Operand(storage, (0, s_row, s_col)),
                Operand(np.eye(cols, dtype=np.float32).ravel(), (0, cols, 1)),
                Operand(np.zeros(rows * cols, np.float32), (0, cols, 1)))
    C = _run(p, lib)
    assert C.tolist() == [float(v) for v in ints(g["transposed_contiguous"])]


def pin_golden_column_major(lib):
    """kael ch. 09, "cuBLAS": the bytes 1..6 read row-major as 2 x 3 give
    [[1,2,3],[4,5,6]]; read column-major as 3 x 2 they give its transpose."""
    g = load_golden("kael_column_major.txt")
    storage = np.array(ints(g["storage"]), np.float32)
    from strided_fp32_gemm_amd.workloads import Operand, Problem
    for shape_key, vals_key, strides in (
            ("row_major_shape", "row_major", None),
            ("column_major_shape", "column_major", "cm")):
        rows, cols = ints(g[shape_key])
        st = (cols, 1) if strides is None else column_major_strides(rows)
        p = Problem("cm", 1, rows, cols, cols, 1.0, False,
                    Operand(storage, (0, *st)),
                    Operand(np.eye(cols, dtype=np.float32).ravel(), (0, cols, 1)),
                    Operand(np.zeros(rows * cols, np.float32), (0, cols, 1)))
        assert _run(p, lib).tolist() == [float(v) for v in ints(g[vals_key])], shape_key


def _blas_operand(trans: str, ld: int, rows: int, cols: int):
    """(row, col) strides of op(X) for a column-major X with leading
    dimension ld, where op(X) is rows x cols."""
    r, c = column_major_strides(ld)
    return (c, r) if trans == "T" else (r, c)


def pin_blas_linear_mapping(lib):
    """rvllm, "Matmuls go to cuBLAS": the column-major call (transa T, transb
    N, m = out, n = rows, k = in, lda = ldb = in, ldc = out) on the row-major
    buffers computes the same bytes as y = x W^T with W read transposed."""
    g = load_golden("rvllm_linear_blas.txt")
    rows, in_f, out_f = 7, 13, 5
    sym = {"out_features": out_f, "rows": rows, "in_features": in_f}
    rng = np.random.default_rng(11)
    x = rng.standard_normal((rows, in_f)).astype(np.float32).ravel()
    W = rng.standard_normal((out_f, in_f)).astype(np.float32).ravel()
    bufs = {"weight": W, "x": x}
    m, n, k = sym[g["m"]], sym[g["n"]], sym[g["k"]]
    sa = _blas_operand(g["transa"], sym[g["lda"]], m, k)
    sb = _blas_operand(g["transb"], sym[g["ldb"]], k, n)
    sc = column_major_strides(sym[g["ldc"]])
    y_blas = np.zeros(rows * out_f, np.float32)
    oracle.ref_sgemm(1, m, n, k, float(g["alpha"]), bufs[g["first_operand"]], 0, *sa,
                     bufs[g["second_operand"]], 0, *sb, 0, y_blas, 0, *sc, lib=lib)
    y_rm = np.zeros(rows * out_f, np.float32)
    oracle.ref_sgemm(1, rows, out_f, in_f, 1.0, x, 0, in_f, 1, W, 0, 1, in_f,
                     0, y_rm, 0, out_f, 1, lib=lib)
    assert np.array_equal(y_blas, y_rm)
    ref = x.reshape(rows, in_f).astype(np.float64) @ W.reshape(out_f, in_f).astype(np.float64).T
    assert np.allclose(y_rm.reshape(rows, out_f), ref, rtol=1e-6, atol=1e-6)


def pin_blas_rowmajor_trick(lib):
    """kael ch. 09, "cuBLAS": (N, N, columns, rows, inner) with b first
    (ld columns) and a second (ld inner), output ld columns, is row-major
    a @ b; also C^T = B^T A^T through an output with exchanged strides."""
    g = load_golden("kael_cublas_rowmajor.txt")
    rows, inner, cols = 6, 11, 9
    sym = {"rows": rows, "inner": inner, "columns": cols}
    rng = np.random.default_rng(12)
    a = rng.standard_normal((rows, inner)).astype(np.float32).ravel()
    b = rng.standard_normal((inner, cols)).astype(np.float32).ravel()
    bufs = {"a": a, "b": b}
    m, n, k = sym[g["m"]], sym[g["n"]], sym[g["k"]]
    sa = _blas_operand(g["transa"], sym[g["lda"]], m, k)
    sb = _blas_operand(g["transb"], sym[g["ldb"]], k, n)
    sc = column_major_strides(sym[g["ldc"]])
    out_blas = np.zeros(rows * cols, np.float32)
    oracle.ref_sgemm(1, m, n, k, 1.0, bufs[g["first_operand"]], 0, *sa,
                     bufs[g["second_operand"]], 0, *sb, 0, out_blas, 0, *sc, lib=lib)
    out_rm = np.zeros(rows * cols, np.float32)
    oracle.ref_sgemm(1, rows, cols, inner, 1.0, a, 0, inner, 1, b, 0, cols, 1,
                     0, out_rm, 0, cols, 1, lib=lib)
    assert np.array_equal(out_blas, out_rm)


# ------------------------------------------------------ exact brute force

def pin_exact_bruteforce(lib, sizes=range(1, 9)):
    """Every m, n, k in 1..8, all four transpose cases, batch 1 and 3,
    accumulate on/off, alpha 1 and 0.5, integer data in [-3, 3]: each partial
    sum is exact, so the result is unique; numpy's int64 matmul gives it."""
    rng = np.random.default_rng(2024)
    for m in sizes:
        for n in sizes:
            for k in sizes:
                for a_major, b_major in LAYOUTS:
                    for batch in (1, 3):
                        acc = (m + n + k + batch) % 2 == 0
                        alpha = 0.5 if (m * n * k) % 2 else 1.0
                        for acc_, alpha_ in ((acc, alpha), (not acc, 1.5 - alpha)):
                            _exact_case(lib, rng, batch, m, n, k, a_major, b_major, alpha_, acc_)


def _exact_case(lib, rng, batch, m, n, k, a_major, b_major, alpha, acc):
    per_a, sa = layout_strides(m, k, a_major)
    per_b, sb = layout_strides(k, n, b_major)
    per_c, sc = layout_strides(m, n, "row")
    A = rng.integers(-3, 4, per_a * batch).astype(np.float32)
    B = rng.integers(-3, 4, per_b * batch).astype(np.float32)
    C = rng.integers(-3, 4, per_c * batch).astype(np.float32)
    Ai = view(A, batch, m, k, sa).astype(np.int64)
    Bi = view(B, batch, k, n, sb).astype(np.int64)
    exact = np.matmul(Ai, Bi).astype(np.float64) * alpha
    if acc:
        exact = exact + view(C, batch, m, n, sc)
    out = C.copy()
    oracle.ref_sgemm(batch, m, n, k, alpha, A, *sa, B, *sb, int(acc), out, *sc, lib=lib)
    got = view(out, batch, m, n, sc)
    assert np.array_equal(got, exact.astype(np.float32)), (batch, m, n, k, a_major, b_major, alpha, acc)


def pin_denormals(lib):
    """Denormal operands and results are exact powers of two times the
    integer case: A scaled by 2^-130 (denormal inputs), A and B each by
    2^-70 (normal inputs, denormal products), and a denormal C_old added to
    a zero product; int64 matmul times the scale gives each result, which
    fp32 represents exactly (nothing is flushed to zero)."""
    rng = np.random.default_rng(77)
    m, n, k, batch = 6, 5, 7, 2
    per_a, sa = layout_strides(m, k, "row")
    per_b, sb = layout_strides(k, n, "col")
    per_c, sc = layout_strides(m, n, "row")
    Ai = rng.integers(-3, 4, per_a * batch).astype(np.float32)
    Bi = rng.integers(-3, 4, per_b * batch).astype(np.float32)
    exact_i = np.matmul(view(Ai, batch, m, k, sa).astype(np.int64),
                        view(Bi, batch, k, n, sb).astype(np.int64)).astype(np.float64)
    for sa_scale, sb_scale in ((2.0 ** -130, 1.0), (2.0 ** -70, 2.0 ** -70)):
        A = (Ai.astype(np.float64) * sa_scale).astype(np.float32)
        B = (Bi.astype(np.float64) * sb_scale).astype(np.float32)
        out = np.zeros(per_c * batch, np.float32)
        oracle.ref_sgemm(batch, m, n, k, 1.0, A, *sa, B, *sb, 0, out, *sc, lib=lib)
        want = (exact_i * sa_scale * sb_scale).astype(np.float32)
        assert np.count_nonzero(want) > 0 and np.abs(want[want != 0]).min() < 2.0 ** -126   # some denormal
        assert np.array_equal(view(out, batch, m, n, sc), want), (sa_scale, sb_scale)
    C0 = ((np.arange(per_c * batch) % 7 + 1) * 2.0 ** -135).astype(np.float32)
    out = C0.copy()
    oracle.ref_sgemm(batch, m, n, k, 1.0, np.zeros(per_a * batch, np.float32), *sa,
                     Bi, *sb, 1, out, *sc, lib=lib)
    assert np.array_equal(out, C0)


# ------------------------------------------------ library cross-check (fp64)

AWKWARD = [(17, 33, 9), (5, 129, 31), (1, 1, 1), (4, 4, 4), (5, 3, 9), (8, 16, 7),
           (33, 20, 65), (64, 1, 64), (1, 64, 1), (127, 129, 128), (3, 514, 70)]


def pin_numpy_float64(lib, shapes=AWKWARD):
    """Against numpy float64 matmul on the strided views: the oracle must be
    the fp32 rounding of the fp64 result (half an ulp, plus fp64 noise).
    Shapes (rows, inner, columns) are the pages' awkward test sizes:
    StaleyNET "Testing the kernels" and kael ch. 09 "How it is tested"."""
    for idx, (m, k, n) in enumerate(shapes):
        for a_major, b_major in LAYOUTS:
            p = random_problem(100 + idx, 2, m, n, k, a_major=a_major, b_major=b_major,
                               alpha=0.75, accumulate=True, pad=3)
            C = _run(p, lib)
            Av = view(p.A.storage, 2, m, k, p.A.strides).astype(np.float64)
            Bv = view(p.B.storage, 2, k, n, p.B.strides).astype(np.float64)
            Cold = view(p.C.storage, 2, m, n, p.C.strides).astype(np.float64)
            ref = 0.75 * np.matmul(Av, Bv) + Cold
            got = _out(p, C).astype(np.float64)
            scale = k * np.abs(Av).max() * np.abs(Bv).max() + np.abs(Cold).max()
            tol = 0.5 * np.spacing(np.abs(got).astype(np.float32)).astype(np.float64) + 1e-12 * scale
            assert np.all(np.abs(got - ref) <= tol), (m, n, k, a_major, b_major)


# ------------------------------------------------------------- invariants

def pin_stride_swap(lib):
    """Reading a stored X^T with exchanged strides equals using an explicit
    row-major copy of X, bitwise (StaleyNET "The matrix product": a
    transposed matrix is the same memory with the two distances exchanged)."""
    for a_major, b_major in LAYOUTS:
        p = random_problem(21, 2, 13, 11, 10, a_major=a_major, b_major=b_major, dist="normal")
        Acopy = np.ascontiguousarray(view(p.A.storage, 2, 13, 10, p.A.strides)).ravel()
        Bcopy = np.ascontiguousarray(view(p.B.storage, 2, 10, 11, p.B.strides)).ravel()
        C1 = _run(p, lib)
        C2 = p.C.storage.copy()
        oracle.ref_sgemm(2, 13, 11, 10, p.alpha, Acopy, 130, 10, 1, Bcopy, 110, 11, 1,
                         0, C2, *p.C.strides, lib=lib)
        assert np.array_equal(C1, C2), (a_major, b_major)


def pin_transpose_identity(lib):
    """C^T = B^T A^T: the product of the exchanged-stride views of B and A,
    written through C's exchanged strides, gives the same bytes as C."""
    for a_major, b_major in LAYOUTS:
        p = random_problem(22, 3, 9, 14, 12, a_major=a_major, b_major=b_major, dist="normal")
        C1 = _run(p, lib)
        C2 = p.C.storage.copy()
        sa, sb, sc = p.A.strides, p.B.strides, p.C.strides
        oracle.ref_sgemm(3, 14, 9, 12, p.alpha, p.B.storage, sb[0], sb[2], sb[1],
                         p.A.storage, sa[0], sa[2], sa[1], 0, C2, sc[0], sc[2], sc[1], lib=lib)
        assert np.array_equal(C1, C2), (a_major, b_major)


def pin_batch_slices(lib):
    """Each batch of a batched call equals a batch-1 call on its slice, and a
    batch stride of 0 equals explicit replication, bitwise."""
    p = random_problem(23, 3, 10, 7, 9, a_major="col", b_major="row", pad=2, dist="normal",
                       accumulate=True, alpha=-1.25)
    C = _run(p, lib)
    for b in range(3):
        Cb = p.C.storage.copy()
        sa, sb, sc = p.A.strides, p.B.strides, p.C.strides
        oracle.ref_sgemm(1, 10, 7, 9, p.alpha, p.A.storage[b * sa[0]:], 0, sa[1], sa[2],
                         p.B.storage[b * sb[0]:], 0, sb[1], sb[2], 1,
                         Cb[b * sc[0]:], 0, sc[1], sc[2], lib=lib)
        assert np.array_equal(view(Cb, 3, 10, 7, sc)[b], view(C, 3, 10, 7, sc)[b]), b
    q = random_problem(24, 4, 6, 5, 8, b_broadcast=True, dist="normal")
    Cq = _run(q, lib)
    per_b = 8 * 5
    Brep = np.tile(q.B.storage[:per_b], 4)
    Cr = q.C.storage.copy()
    oracle.ref_sgemm(4, 6, 5, 8, 1.0, q.A.storage, *q.A.strides, Brep, per_b, 5, 1,
                     0, Cr, *q.C.strides, lib=lib)
    assert np.array_equal(Cq, Cr)


def pin_accumulate(lib):
    """accumulate = 1 equals C_old plus a separate fresh alpha*A*B call:
    bitwise on integer data, within one rounding otherwise."""
    p = random_problem(25, 2, 9, 8, 7, dist="int", accumulate=True, alpha=2.0)
    acc = _out(p, _run(p, lib))
    fresh_p = random_problem(25, 2, 9, 8, 7, dist="int", accumulate=False, alpha=2.0)
    fresh = _out(fresh_p, _run(fresh_p, lib))
    cold = view(p.C.storage, 2, 9, 8, p.C.strides)
    assert np.array_equal(acc, cold + fresh)
    p = random_problem(26, 2, 9, 8, 300, dist="normal", accumulate=True, alpha=0.3)
    acc = _out(p, _run(p, lib)).astype(np.float64)
    fresh_p = random_problem(26, 2, 9, 8, 300, dist="normal", accumulate=False, alpha=0.3)
    fresh = _out(fresh_p, _run(fresh_p, lib)).astype(np.float64)
    cold = view(p.C.storage, 2, 9, 8, p.C.strides).astype(np.float64)
    both = cold + fresh
    assert np.all(np.abs(acc - both) <= np.spacing(np.abs(acc).astype(np.float32)) + 1e-7 * np.abs(fresh))


def pin_order_and_entries(lib):
    """Visiting the elements in reverse order changes no bit (kael ch. 09,
    "The host emulation" runs work items backwards for the same reason), and
    the one-by-one entry routine returns exactly the full product's values."""
    p = random_problem(27, 3, 21, 19, 33, a_major="col", b_major="col", dist="normal",
                       accumulate=True, alpha=0.5, pad=1)
    C1 = _run(p, lib)
    C2 = _run(p, lib, reverse=True)
    assert np.array_equal(C1, C2)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.integers(0, 3, 50), rng.integers(0, 21, 50), rng.integers(0, 19, 50)], 1)
    vals = oracle.ref_entries(*p.call_args(p.A.storage, p.B.storage, p.C.storage), idx=idx, lib=lib)
    full = _out(p, C1)
    assert np.array_equal(vals, full[idx[:, 0], idx[:, 1], idx[:, 2]])


def pin_nan_and_canaries(lib):
    """A NaN in A[0, 2, 1] makes row 2 of batch 0 NaN and nothing else;
    gaps between C's rows keep their sentinel; with accumulate = 0 a
    NaN-filled C is never read."""
    p = random_problem(28, 2, 5, 6, 4, pad=3, dist="normal")
    sa, sc = p.A.strides, p.C.strides
    A = p.A.storage.copy()
    A[0 * sa[0] + 2 * sa[1] + 1 * sa[2]] = np.nan
    C = np.full_like(p.C.storage, np.nan)
    oracle.ref_sgemm(2, 5, 6, 4, 1.0, A, *sa, p.B.storage, *p.B.strides, 0, C, *sc, lib=lib)
    out = view(C, 2, 5, 6, sc)
    nan_mask = np.zeros((2, 5, 6), bool)
    nan_mask[0, 2, :] = True
    assert np.array_equal(np.isnan(out), nan_mask)
    covered = np.zeros(C.size, bool)
    for b in range(2):
        for i in range(5):
            covered[b * sc[0] + i * sc[1]: b * sc[0] + i * sc[1] + 6] = True
    assert np.all(np.isnan(C[~covered]))


# ------------------------------------------------ general epilogue, distances

def _ex_case(lib, rng, batch, m, n, k, a_major, b_major, alpha, beta, use_row, use_col,
             vec_batch_stride=True, reverse=False):
    """Integer data: alpha*A@B + beta*C_old + r[i] + c[j] is exact in fp32
    for these sizes, so numpy's int64 arithmetic gives the unique result."""
    per_a, sa = layout_strides(m, k, a_major)
    per_b, sb = layout_strides(k, n, b_major)
    per_c, sc = layout_strides(m, n, "row")
    A = rng.integers(-3, 4, per_a * batch).astype(np.float32)
    B = rng.integers(-3, 4, per_b * batch).astype(np.float32)
    C = rng.integers(-3, 4, per_c * batch).astype(np.float32)
    nvb = batch if vec_batch_stride else 1
    r = rng.integers(-9, 10, m * nvb + 2).astype(np.float32)
    c = rng.integers(-9, 10, n * nvb + 2).astype(np.float32)
    sR = (m if vec_batch_stride else 0, 1)
    sL = (n if vec_batch_stride else 0, 1)
    exact = np.matmul(view(A, batch, m, k, sa).astype(np.int64),
                      view(B, batch, k, n, sb).astype(np.int64)).astype(np.float64) * alpha
    if beta != 0:
        exact = exact + beta * view(C, batch, m, n, sc)
    if use_row:
        exact = exact + np.array([[r[b * sR[0] + i] for i in range(m)] for b in range(batch)])[:, :, None]
    if use_col:
        exact = exact + np.array([[c[b * sL[0] + j] for j in range(n)] for b in range(batch)])[:, None, :]
    out = C.copy()
    oracle.ref_sgemm_ex(batch, m, n, k, alpha, A, sa, B, sb, beta, out, sc,
                        row_add=r if use_row else None, sR=sR, col_add=c if use_col else None,
                        sL=sL, reverse=reverse, lib=lib)
    got = view(out, batch, m, n, sc)
    assert np.array_equal(got, exact.astype(np.float32)), (batch, m, n, k, alpha, beta, use_row, use_col)


def pin_epilogue_bruteforce(lib):
    """C <- alpha*A*B + beta*C_old + r[b,i] + c[b,j] on integer data, every
    transpose case, beta in {0, 1, -2, 0.5}, each vector term on and off,
    per-batch and shared (batch stride 0) vectors: exact against int64."""
    rng = np.random.default_rng(7)
    for a_major, b_major in LAYOUTS:
        for beta in (0.0, 1.0, -2.0, 0.5):
            for use_row in (False, True):
                for use_col in (False, True):
                    for shared in (False, True):
                        _ex_case(lib, rng, 3, 5, 6, 4, a_major, b_major, -2.0, beta, use_row, use_col,
                                 vec_batch_stride=not shared)
    for m, n, k in ((1, 1, 1), (7, 3, 8), (2, 9, 1)):
        _ex_case(lib, rng, 2, m, n, k, "col", "row", 1.0, 1.0, True, True, reverse=True)


def pin_epilogue_closed_forms(lib):
    """All-ones A, B: C = k*alpha + beta*C_old + r[i] + c[j] exactly; beta = 1
    with no vector terms is "optionally plus C" (the accumulate flag gives
    the same bits); beta = 0 never reads C_old (a NaN-filled C stays out)."""
    batch, m, n = 2, 3, 5
    for k in (1, 64, 4096):
        p = random_problem(k + 1, batch, m, n, k, dist="ones", alpha=0.5, accumulate=True)
        r = np.arange(m * batch, dtype=np.float32) * 0.25
        c = -np.arange(n * batch, dtype=np.float32)
        for beta in (1.0, -0.5):
            out = p.C.storage.copy()
            oracle.ref_sgemm_ex(batch, m, n, k, 0.5, p.A.storage, p.A.strides, p.B.storage, p.B.strides,
                                beta, out, p.C.strides, row_add=r, sR=(m, 1), col_add=c, sL=(n, 1), lib=lib)
            cold = view(p.C.storage, batch, m, n, p.C.strides).astype(np.float64)
            want = k * 0.5 + beta * cold + r.reshape(batch, m, 1) + c.reshape(batch, 1, n)
            assert np.array_equal(view(out, batch, m, n, p.C.strides), want.astype(np.float32)), (k, beta)
        flag = _run(p, lib)
        plain = p.C.storage.copy()
        oracle.ref_sgemm_ex(batch, m, n, k, 0.5, p.A.storage, p.A.strides, p.B.storage, p.B.strides,
                            1.0, plain, p.C.strides, lib=lib)
        assert np.array_equal(flag, plain)
    q = random_problem(31, 2, 4, 6, 5, dist="normal")
    nanC = np.full_like(q.C.storage, np.nan)
    oracle.ref_sgemm_ex(2, 4, 6, 5, 1.0, q.A.storage, q.A.strides, q.B.storage, q.B.strides, 0.0, nanC,
                        q.C.strides, row_add=np.ones(8, np.float32), sR=(4, 1), lib=lib)
    assert not np.any(np.isnan(view(nanC, 2, 4, 6, q.C.strides)))
    idx = np.array([[0, 0, 0], [1, 3, 5], [1, 2, 0]])
    r = np.arange(8, dtype=np.float32)
    full = q.C.storage.copy()
    oracle.ref_sgemm_ex(2, 4, 6, 5, 1.5, q.A.storage, q.A.strides, q.B.storage, q.B.strides, -1.0, full,
                        q.C.strides, row_add=r, sR=(4, 1), lib=lib)
    one = oracle.ref_sgemm_ex_entries(2, 4, 6, 5, 1.5, q.A.storage, q.A.strides, q.B.storage,
                                      q.B.strides, -1.0, q.C.storage, q.C.strides, idx,
                                      row_add=r, sR=(4, 1), lib=lib)
    assert np.array_equal(one, view(full, 2, 4, 6, q.C.strides)[idx[:, 0], idx[:, 1], idx[:, 2]])


def pin_sqnorms(lib):
    """Squared norms of rows and of columns (the same storage read along
    either axis) equal numpy's int64 sums of squares; norms of all-ones
    vectors are their lengths."""
    rng = np.random.default_rng(8)
    X = rng.integers(-5, 6, 3 * 7 * 9).astype(np.float32)
    Xi = X.reshape(3, 7, 9).astype(np.int64)
    rows = np.zeros(3 * 7, np.float32)
    oracle.ref_sqnorms(3, 7, 9, X, (63, 9, 1), rows, (7, 1), lib=lib)
    assert np.array_equal(rows.reshape(3, 7), (Xi ** 2).sum(2).astype(np.float32))
    cols = np.zeros(3 * 9 * 2, np.float32)
    oracle.ref_sqnorms(3, 9, 7, X, (63, 1, 9), cols, (18, 2), lib=lib)
    assert np.array_equal(cols.reshape(3, 9, 2)[:, :, 0], (Xi ** 2).sum(1).astype(np.float32))
    ones = np.ones(5 * 300, np.float32)
    out = np.zeros(5, np.float32)
    oracle.ref_sqnorms(1, 5, 300, ones, (0, 300, 1), out, (0, 1), lib=lib)
    assert np.array_equal(out, np.full(5, 300.0, np.float32))


def pin_sqdist(lib):
    """Squared distances: integer brute force ((x - y)^2 summed in int64),
    zero from a point to itself, D(X, Y) = D(Y, X)^T, invariance under a
    common integer shift, and the expansion |x|^2 + |y|^2 - 2 x.y."""
    rng = np.random.default_rng(9)
    for batch, m, n, k in ((1, 1, 1, 1), (2, 5, 4, 7), (3, 8, 9, 3), (1, 16, 2, 33)):
        X = rng.integers(-4, 5, batch * m * k).astype(np.float32)
        Y = rng.integers(-4, 5, batch * n * k).astype(np.float32)
        sX, sY, sD = (m * k, k, 1), (n * k, k, 1), (m * n, n, 1)
        D = np.zeros(batch * m * n, np.float32)
        oracle.ref_sqdist(batch, m, n, k, X, sX, Y, sY, D, sD, lib=lib)
        Xi, Yi = X.reshape(batch, m, 1, k).astype(np.int64), Y.reshape(batch, 1, n, k).astype(np.int64)
        exact = ((Xi - Yi) ** 2).sum(3)
        assert np.array_equal(D.reshape(batch, m, n), exact.astype(np.float32))
        expand = (Xi ** 2).sum(3) + (Yi ** 2).sum(3) - 2 * (Xi * Yi).sum(3)
        assert np.array_equal(exact, expand)
        DT = np.zeros(batch * n * m, np.float32)
        oracle.ref_sqdist(batch, n, m, k, Y, sY, X, sX, DT, (n * m, m, 1), lib=lib)
        assert np.array_equal(DT.reshape(batch, n, m), D.reshape(batch, m, n).transpose(0, 2, 1))
        t = rng.integers(-3, 4, k).astype(np.float32)
        Ds = np.zeros_like(D)
        oracle.ref_sqdist(batch, m, n, k, (X.reshape(-1, k) + t).ravel(), sX,
                          (Y.reshape(-1, k) + t).ravel(), sY, Ds, sD, lib=lib)
        assert np.array_equal(Ds, D)
        self_d = np.zeros(batch * m * m, np.float32)
        oracle.ref_sqdist(batch, m, m, k, X, sX, X, sX, self_d, (m * m, m, 1), lib=lib)
        assert np.all(np.diagonal(self_d.reshape(batch, m, m), axis1=1, axis2=2) == 0)
        idx = np.stack([rng.integers(0, batch, 9), rng.integers(0, m, 9), rng.integers(0, n, 9)], 1)
        one = oracle.ref_sqdist_entries(batch, m, n, k, X, sX, Y, sY, idx, lib=lib)
        assert np.array_equal(one, D.reshape(batch, m, n)[idx[:, 0], idx[:, 1], idx[:, 2]])


def pin_batched2_bthd_gqa(lib):
    """Both attention products straight on [sequence][token][head][dim]
    buffers with grouped KV heads (G query heads per KV head): integer data,
    checked against numpy's int64 einsum of the definition, scores written
    head-major, outputs written back in [B][T][H][D]."""
    rng = np.random.default_rng(11)
    for B_, T, Hq, G, D in ((2, 5, 4, 2, 3), (3, 7, 6, 3, 8), (1, 9, 2, 1, 4), (2, 4, 8, 4, 5)):
        Hk = Hq // G
        Q = rng.integers(-3, 4, B_ * T * Hq * D).astype(np.float32)
        K = rng.integers(-3, 4, B_ * T * Hk * D).astype(np.float32)
        V = rng.integers(-3, 4, B_ * T * Hk * D).astype(np.float32)
        Qi, Ki, Vi = (x.reshape(B_, T, h, D).astype(np.int64) for x, h in ((Q, Hq), (K, Hk), (V, Hk)))
        head_of = np.arange(Hq) // G
        S_exact = np.einsum("bthd,bshd->bhts", Qi, Ki[:, :, head_of, :])
        S = np.full(B_ * Hq * T * T, 0.25, np.float32)
        oracle.ref_sgemm_batched2(B_, Hq, T, T, D, 2.0,
                                  Q, T * Hq * D, D, 1, Hq * D, 1,
                                  K, T * Hk * D, D, G, 1, Hk * D,
                                  True, S, Hq * T * T, T * T, T, 1, lib=lib)
        assert np.array_equal(S.reshape(B_, Hq, T, T), (2 * S_exact + 0.25).astype(np.float32))
        P = rng.integers(-2, 3, B_ * Hq * T * T).astype(np.float32)
        Pi = P.reshape(B_, Hq, T, T).astype(np.int64)
        O_exact = np.einsum("bhts,bshd->bthd", Pi, Vi[:, :, head_of, :])
        O = np.zeros(B_ * T * Hq * D, np.float32)
        oracle.ref_sgemm_batched2(B_, Hq, T, D, T, 1.0,
                                  P, Hq * T * T, T * T, 1, T, 1,
                                  V, T * Hk * D, D, G, Hk * D, 1,
                                  False, O, T * Hq * D, D, Hq * D, 1, lib=lib)
        assert np.array_equal(O.reshape(B_, T, Hq, D), O_exact.astype(np.float32))


def pin_batched2_gqa_row_folding(lib):
    """With head-major buffers the query heads of one KV head are adjacent,
    so stacking them as extra rows of one product (the rvllm post's folding,
    "Matmuls go to cuBLAS") is the same computation as one product per query
    head with the KV head index divided by the group size: same bits."""
    rng = np.random.default_rng(12)
    B_, Hq, G, T, D = 2, 8, 4, 6, 5
    Hk = Hq // G
    Q = rng.standard_normal(B_ * Hq * T * D).astype(np.float32)
    K = rng.standard_normal(B_ * Hk * T * D).astype(np.float32)
    S1 = np.zeros(B_ * Hq * T * T, np.float32)
    oracle.ref_sgemm_batched2(B_, Hq, T, T, D, 0.125, Q, Hq * T * D, T * D, 1, D, 1,
                              K, Hk * T * D, T * D, G, 1, D, False, S1, Hq * T * T, T * T, T, 1, lib=lib)
    S2 = np.zeros_like(S1)
    oracle.ref_sgemm(B_ * Hk, G * T, T, D, 0.125, Q, G * T * D, D, 1, K, T * D, 1, D, 0,
                     S2, G * T * T, T, 1, lib=lib)
    assert np.array_equal(S1, S2)


# ------------------------------------------------------------------ attention

def _attn(lib, Q, K, V, alpha, causal, g=1, order="heads"):
    """Run the oracle's attention on logical [outer][head][token][dim] arrays
    stored head-major or token-major ([outer][token][head][dim]); returns O as
    a logical [outer][head][tq][dim] float32 array."""
    def store(X):
        no, h, t, d = X.shape
        if order == "heads":
            return np.ascontiguousarray(X, np.float32).ravel(), (h * t * d, t * d, d, 1)
        return (np.ascontiguousarray(X.transpose(0, 2, 1, 3), np.float32).ravel(),
                (t * h * d, d, h * d, 1))
    no, h, tq, d = Q.shape
    tk = K.shape[2]
    q, sq = store(Q)
    k, sk = store(K)
    v, sv = store(V)
    o, so = store(np.zeros((no, h, tq, d), np.float32))
    oracle.ref_attention(no, h, tq, tk, d, alpha, causal, q, *sq, k, sk[0], sk[1], g, sk[2], sk[3],
                         v, *sv, o, *so, lib=lib)
    if order == "heads":
        return o.reshape(no, h, tq, d)
    return o.reshape(no, tq, h, d).transpose(0, 2, 1, 3)


def _visible(tq, tk, causal):
    """mask[q, j]: key j is seen by query q (the queries are the last tq of tk
    positions)."""
    if not causal:
        return np.ones((tq, tk), bool)
    return np.arange(tk)[None, :] <= np.arange(tq)[:, None] + (tk - tq)


def pin_attention_closed_forms(lib):
    """Closed forms of softmax attention: equal scores (Q = 0, or alpha = 0)
    weight every visible key alike, so each output row is the mean of the
    visible V rows; a query that sees one key returns that V row exactly; a
    key whose score leads by 40 or more takes all the weight (e^-40 is below
    fp32 resolution), so the output is that key's V row.  Causal and not, decode
    (tq < tk) and prefill, one and several KV groups, both layouts."""
    rng = np.random.default_rng(21)
    for no, h, g, tq, tk, d, causal, order in ((1, 1, 1, 7, 7, 5, False, "heads"),
                                               (2, 4, 2, 7, 7, 3, True, "tokens"),
                                               (1, 3, 3, 3, 8, 4, True, "heads"),
                                               (2, 2, 1, 1, 9, 6, True, "tokens")):
        hk = h // g
        V = rng.standard_normal((no, hk, tk, d)).astype(np.float32)
        K = rng.standard_normal((no, hk, tk, d)).astype(np.float32)
        Qr = rng.standard_normal((no, h, tq, d)).astype(np.float32)
        mask = _visible(tq, tk, causal)
        Vh = V[:, np.arange(h) // g].astype(np.float64)                  # [no][h][tk][d]
        mean = (mask[None, None, :, :, None] * Vh[:, :, None]).sum(3) / mask.sum(1)[None, None, :, None]
        for Q, alpha in ((np.zeros_like(Qr), 0.7), (Qr, 0.0)):
            O = _attn(lib, Q, K, V, alpha, causal, g, order)
            tol = 4 * np.spacing(np.float32(np.abs(V).max()))
            assert np.abs(O - mean).max() <= tol, (no, h, g, tq, tk, causal, order)
        if causal and tq == tk:
            O = _attn(lib, Qr, K, V, 0.5, True, g, order)
            assert np.array_equal(O[:, :, 0], V[:, np.arange(h) // g, 0])
    # One key of one row: every query sees exactly that V row.
    V1 = rng.standard_normal((2, 2, 1, 5)).astype(np.float32)
    K1 = rng.standard_normal((2, 2, 1, 5)).astype(np.float32)
    Q1 = rng.standard_normal((2, 2, 4, 5)).astype(np.float32)
    O = _attn(lib, Q1, K1, V1, 3.0, False)
    assert np.array_equal(O, np.broadcast_to(V1, O.shape))
    # A dominant key: K = c I, Q[q] = e_pick[q], alpha 0.5 -> score c/2 for
    # the picked key, 0 for the rest; causal picks stay visible (pick[q] <= q).
    # c = 4000 puts the lead far past exp's range, so only a softmax that
    # subtracts the true row maximum stays finite.
    d = tk = tq = 8
    pick = np.array([0, 1, 0, 2, 4, 3, 6, 1])
    Q = np.eye(d, dtype=np.float32)[pick][None, None]
    V = rng.standard_normal((1, 1, tk, d)).astype(np.float32)
    for c in (80.0, 4000.0):
        K = (c * np.eye(tk, d, dtype=np.float32))[None, None]
        for causal in (False, True):
            for order in ("heads", "tokens"):
                O = _attn(lib, Q, K, V, 0.5, causal, 1, order)
                assert np.array_equal(O[0, 0], V[0, 0, pick]), (c, causal, order)


def pin_attention_invariants(lib):
    """Invariants of the definition: adding the same amount to every score of
    a row changes nothing (an extra dimension with Q = 1 and K = 1e4 shifts
    the scores by alpha*1e4, far past exp's range); permuting the keys (K and
    V rows together) changes nothing without a mask; one decode query equals
    the last row of the causal prefill over the same context; grouped KV heads
    equal each KV head repeated for its query heads (same bits)."""
    rng = np.random.default_rng(22)
    no, h, g, t, d = 2, 4, 2, 9, 6
    hk = h // g
    Q = rng.standard_normal((no, h, t, d)).astype(np.float32)
    K = rng.standard_normal((no, hk, t, d)).astype(np.float32)
    V = rng.standard_normal((no, hk, t, d)).astype(np.float32)
    for causal in (False, True):
        base = _attn(lib, Q, K, V, 0.25, causal, g)
        Qs = np.concatenate([Q, np.ones((no, h, t, 1), np.float32)], 3)
        Ks = np.concatenate([K, np.full((no, hk, t, 1), 1e4, np.float32)], 3)
        Vs = np.concatenate([V, np.zeros((no, hk, t, 1), np.float32)], 3)
        shifted = _attn(lib, Qs, Ks, Vs, 0.25, causal, g)[..., :d]
        assert np.all(np.isfinite(shifted))
        assert np.abs(shifted - base).max() <= 1e-6 * np.abs(V).max(), causal
        rep = _attn(lib, Q, np.repeat(K, g, 1), np.repeat(V, g, 1), 0.25, causal, 1)
        assert np.array_equal(rep, base), causal
    perm = rng.permutation(t)
    Op = _attn(lib, Q, K[:, :, perm], V[:, :, perm], 0.25, False, g)
    assert np.abs(Op - _attn(lib, Q, K, V, 0.25, False, g)).max() <= 1e-6 * np.abs(V).max()
    prefill = _attn(lib, Q, K, V, 0.25, True, g, "tokens")
    for last in (t, 5):
        dec = _attn(lib, Q[:, :, last - 1:last], K[:, :, :last], V[:, :, :last], 0.25, True, g, "tokens")
        full = prefill if last == t else _attn(lib, Q[:, :, :last], K[:, :, :last], V[:, :, :last],
                                               0.25, True, g, "tokens")
        assert np.array_equal(dec[:, :, 0], full[:, :, last - 1]), last


def pin_attention_numpy_float64(lib):
    """Against numpy's float64 route (matmul, exp, sum) on random data in
    both layouts with grouped heads: the oracle rounds once, so it must sit
    within one fp32 spacing of the float64 result."""
    rng = np.random.default_rng(23)
    for no, h, g, tq, tk, d, causal, order in ((2, 6, 3, 13, 13, 16, True, "tokens"),
                                               (1, 2, 1, 5, 17, 8, True, "heads"),
                                               (3, 4, 4, 11, 7, 12, False, "tokens")):
        hk = h // g
        Q = rng.standard_normal((no, h, tq, d)).astype(np.float32)
        K = rng.standard_normal((no, hk, tk, d)).astype(np.float32)
        V = rng.standard_normal((no, hk, tk, d)).astype(np.float32)
        alpha = 1.0 / np.sqrt(d)
        O = _attn(lib, Q, K, V, alpha, causal, g, order)
        Kh = K[:, np.arange(h) // g].astype(np.float64)
        Vh = V[:, np.arange(h) // g].astype(np.float64)
        S = np.float64(np.float32(alpha)) * (Q.astype(np.float64) @ Kh.transpose(0, 1, 3, 2))
        S = np.where(_visible(tq, tk, causal), S, -np.inf)
        P = np.exp(S - S.max(-1, keepdims=True))
        ref = (P / P.sum(-1, keepdims=True)) @ Vh
        assert np.all(np.abs(O - ref) <= np.spacing(np.abs(ref).astype(np.float32))), (no, h, tq, tk)


PINS = [pin_all_ones, pin_identity, pin_k_zero, pin_golden_transpose_trace,
        pin_golden_column_major, pin_blas_linear_mapping, pin_blas_rowmajor_trick,
        pin_exact_bruteforce, pin_denormals, pin_numpy_float64, pin_stride_swap, pin_transpose_identity,
        pin_batch_slices, pin_accumulate, pin_order_and_entries, pin_nan_and_canaries,
        pin_epilogue_bruteforce, pin_epilogue_closed_forms, pin_sqnorms, pin_sqdist,
        pin_batched2_bthd_gqa, pin_batched2_gqa_row_folding, pin_attention_closed_forms,
        pin_attention_invariants, pin_attention_numpy_float64]
