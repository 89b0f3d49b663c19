"""GPU parity of the general epilogue, the squared norms and the distance
table, through the C ABI, against the CPU oracle.

Tolerances (stated with the readings of the pages in the design notes):
  * general epilogue: max |C_gpu - C_ref| over the logical outputs divided by
    max(|alpha|, 1) * k * max|A| * max|B| + |beta| * max|C_old| + max|row|
    + max|col| must stay <= 1e-6 (the product's own bound plus one rounding
    per added term);
  * squared norms: |out - ref| <= 1e-6 * len * max|X|^2;
  * distances: |D - D_ref| <= 1e-6 * (2 k max|X| max|Y| + k max|X|^2
    + k max|Y|^2), the product's bound for alpha = -2 plus the two norms.
"""
import numpy as np
import pytest
import torch

import oracle
import strided_fp32_gemm_amd as sg
from strided_fp32_gemm_amd import workloads as wl
from helpers import view

pytestmark = pytest.mark.gpu

TOL = 1e-6
LAYOUTS = [(a, b) for a in ("row", "col") for b in ("row", "col")]
FAMILIES = [sg.PATH_AUTO, sg.PATH_MFMA, sg.PATH_WAVE, sg.PATH_GENERIC]
FAM_IDS = ["auto", "mfma", "wave", "generic"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible: GPU parity cannot pass without one"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _vectors(rng, batch, count, shared, stride=1, scale=2.0):
    """A batch of vectors (or one shared one, batch stride 0) with element
    stride `stride`, as (storage, (s_batch, s_index))."""
    per = (count - 1) * stride + 1
    nb = 1 if shared else batch
    store = (rng.standard_normal(per * nb + 3) * scale).astype(np.float32)
    return store, (0 if shared else per, stride)


def _ex_problem(seed, batch, m, n, k, a_major, b_major, c_major="row", alpha=0.75, beta=0.0,
                row=False, col=False, shared=False, vstride=1):
    p = wl.random_problem(seed, batch, m, n, k, a_major=a_major, b_major=b_major, c_major=c_major,
                          alpha=alpha, accumulate=beta != 0.0, dist="normal")
    rng = np.random.default_rng(seed + 1000)
    p.beta = beta
    p.row = wl.Vector(*_vectors(rng, batch, m, shared, vstride)) if row else None
    p.col = wl.Vector(*_vectors(rng, batch, n, shared, vstride)) if col else None
    return p


def _vec_dev(v):
    return dev(v.storage) if v is not None else None


def gpu_ex(p, path=sg.PATH_AUTO, C0=None):
    dA, dB = dev(p.A.storage), dev(p.B.storage)
    dC = dev(p.C.storage if C0 is None else C0)
    dr, dl = _vec_dev(p.row), _vec_dev(p.col)
    sg.sgemm_strided_batched_ex_path(*p.ex_call_args(dA, dB, dC, dr, dl), path=path,
                                     stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def _oracle_vec_args(p):
    return dict(row_add=p.row.storage if p.row is not None else None,
                sR=p.row.strides if p.row is not None else (0, 0),
                col_add=p.col.storage if p.col is not None else None,
                sL=p.col.strides if p.col is not None else (0, 0))


def oracle_ex(p, C0=None):
    C = (p.C.storage if C0 is None else C0).copy()
    oracle.ref_sgemm_ex(p.batch, p.m, p.n, p.k, p.alpha, p.A.storage, p.A.strides, p.B.storage,
                        p.B.strides, p.beta_value, C, p.C.strides, **_oracle_vec_args(p))
    return C


def ex_err(p, got, ref):
    """Error over the logical outputs divided by the epilogue's bound."""
    amax = float(np.abs(view(p.A.storage, p.batch, p.m, p.k, p.A.strides)).max()) if p.k else 0.0
    bmax = float(np.abs(view(p.B.storage, p.batch, p.k, p.n, p.B.strides)).max()) if p.k else 0.0
    denom = max(abs(p.alpha), 1.0) * p.k * amax * bmax
    if p.beta_value != 0.0:
        denom += abs(p.beta_value) * float(np.abs(view(p.C.storage, p.batch, p.m, p.n, p.C.strides)).max())
    for v in (p.row, p.col):
        if v is not None:
            denom += float(np.abs(v.storage).max())
    diff = float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max())
    return 0.0 if diff == 0.0 else diff / denom


def out(p, C):
    return np.array(view(C, p.batch, p.m, p.n, p.C.strides))


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_general_epilogue_every_family(path):
    """beta in {0, 1, -0.75} x {no vector, row term, column term, both}, all
    four transpose cases, ragged multi-tile shapes, every kernel family."""
    case = 0
    for a_major, b_major in LAYOUTS:
        for beta in (0.0, 1.0, -0.75):
            for row, col in ((False, False), (True, False), (False, True), (True, True)):
                case += 1
                p = _ex_problem(300 + case, 2, 150, 190, 70, a_major, b_major, beta=beta, row=row,
                                col=col)
                got, ref = out(p, gpu_ex(p, path)), out(p, oracle_ex(p))
                e = ex_err(p, got, ref)
                assert e <= TOL, (path, a_major, b_major, beta, row, col, e)


@pytest.mark.parametrize("tile", ["w32x32", "w16x64", "w64x16"])
def test_general_epilogue_wave_split(tile, monkeypatch):
    """The general epilogue after the split partials are summed: a wave tile
    forced with k split over 4 wavefronts, beta in {0, -0.75} with and
    without row and column terms, 16-byte and element C stores."""
    monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
    monkeypatch.setenv("SGEMM_WAVE_SPLIT", "4")
    case = 0
    for (m, n, k), (a_major, b_major) in (((70, 96, 300), ("row", "col")), ((33, 50, 129), ("col", "row"))):
        for beta in (0.0, -0.75):
            for row, col in ((False, False), (True, True), (False, True)):
                case += 1
                p = _ex_problem(600 + case, 2, m, n, k, a_major, b_major, beta=beta, row=row, col=col)
                info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
                assert info["kernel"].startswith("wave_" + tile) and info["waves"] == 4, info
                got, ref = out(p, gpu_ex(p)), out(p, oracle_ex(p))
                e = ex_err(p, got, ref)
                assert e <= TOL, (tile, m, n, k, beta, row, col, e)


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_epilogue_layouts_and_vector_strides(path):
    """Column-major C (solved as C^T = B^T A^T, where the row and column
    terms trade places), vectors shared over the batch (batch stride 0) and
    with element stride 3, 16-byte and element loads, k = 0."""
    for c_major, shared, vstride, (m, n, k) in (("col", False, 1, (130, 70, 40)),
                                                ("row", True, 3, (64, 96, 64)),
                                                ("col", True, 2, (33, 129, 17)),
                                                ("row", False, 1, (70, 50, 0))):
        for a_major, b_major in (("row", "col"), ("col", "row")):
            p = _ex_problem(400 + m + n + k, 3, m, n, k, a_major, b_major, c_major=c_major, alpha=-2.0,
                            beta=0.5, row=True, col=True, shared=shared, vstride=vstride)
            got, ref = out(p, gpu_ex(p, path)), out(p, oracle_ex(p))
            e = ex_err(p, got, ref)
            assert e <= TOL, (path, c_major, shared, vstride, m, n, k, e)


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_epilogue_contiguous_column_terms(path):
    """Column terms read 16 bytes at a time (contiguous, aligned vector, C
    rows of a multiple of 4 floats), per batch and shared, with and
    without a row term."""
    for shared in (False, True):
        for row in (False, True):
            p = _ex_problem(450 + 2 * shared + row, 3, 130, 96, 48, "row", "col", beta=-1.0, row=row,
                            col=True, shared=shared)
            got, ref = out(p, gpu_ex(p, path)), out(p, oracle_ex(p))
            e = ex_err(p, got, ref)
            assert e <= TOL, (path, shared, row, e)


def test_beta_zero_never_reads_c_and_beta_one_is_accumulate():
    """beta = 0 with NaN in every C element gives finite outputs; beta = 1
    with no vectors gives the accumulate entry point's bits."""
    for path in FAMILIES:
        p = _ex_problem(501, 2, 97, 65, 33, "row", "col", beta=0.0, row=True, col=True)
        nanC = np.full_like(p.C.storage, np.nan)
        got = out(p, gpu_ex(p, path, C0=nanC))
        assert np.all(np.isfinite(got)), path
        q = wl.random_problem(502, 2, 97, 65, 33, dist="normal", accumulate=True, alpha=0.5)
        dA, dB, dC = dev(q.A.storage), dev(q.B.storage), dev(q.C.storage)
        sg.sgemm_strided_batched_path(*q.call_args(dA, dB, dC), path=path,
                                      stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        q.beta = 1.0
        assert np.array_equal(dC.cpu().numpy(), gpu_ex(q, path)), path


def test_epilogue_rejects_vectors_overlapping_c():
    p = _ex_problem(503, 1, 32, 32, 16, "row", "row", row=True)
    dA, dB, dC = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage)
    args = p.ex_call_args(dA, dB, dC, dC, None)
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_strided_batched_ex(*args, stream=torch.cuda.current_stream())
    assert e.value.status == -4


def test_sqnorms_rows_and_columns():
    """Norms of rows (contiguous elements: one wavefront per vector) and of
    columns (strided elements: one thread per vector), ragged lengths,
    several batches, an output stride, len = 0."""
    rng = np.random.default_rng(601)
    for batch, rows, cols in ((1, 1, 1), (3, 70, 129), (2, 513, 64), (4, 37, 1000), (2, 5, 0)):
        X = rng.standard_normal(batch * rows * cols + 1).astype(np.float32)
        dX = dev(X)
        for count, length, sX in ((rows, cols, (rows * cols, cols, 1)), (cols, rows, (rows * cols, 1, cols))):
            if count == 0:
                continue
            ref = np.zeros(batch * count * 2, np.float32)
            oracle.ref_sqnorms(batch, count, length, X, sX, ref, (count * 2, 2))
            dout = torch.full((batch * count * 2,), -7.0, device="cuda")
            sg.sgemm_sqnorms(batch, count, length, dX, *sX, dout, count * 2, 2,
                             stream=torch.cuda.current_stream())
            torch.cuda.synchronize()
            got = dout.cpu().numpy()
            assert np.all(got[1::2] == -7.0), "odd output slots must stay untouched"
            bound = TOL * max(length, 1) * max(float(np.abs(X).max()) ** 2, 1e-30)
            assert np.abs(got[0::2].astype(np.float64) - ref[0::2]).max() <= bound, (batch, count, length)


def _dist_err(X, Y, k, got, ref):
    xm, ym = float(np.abs(X).max()), float(np.abs(Y).max())
    bound = 2 * k * xm * ym + k * xm * xm + k * ym * ym
    return float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()) / bound


def test_pairwise_sqdist_small():
    """Distances of ragged shapes against the oracle's plain definition, Y
    per batch and shared, X read transposed, and zero self-distance within
    the bound."""
    rng = np.random.default_rng(701)
    for batch, m, n, k, shared, x_major in ((2, 70, 45, 33, False, "row"), (3, 129, 64, 96, True, "row"),
                                            (1, 5, 300, 7, True, "col"), (2, 64, 64, 512, False, "col")):
        X = rng.standard_normal(batch * m * k).astype(np.float32)
        Y = rng.standard_normal((1 if shared else batch) * n * k).astype(np.float32)
        sX = (m * k, k, 1) if x_major == "row" else (m * k, 1, m)
        sY = (0 if shared else n * k, k, 1)
        sD = (m * n, n, 1)
        ref = np.zeros(batch * m * n, np.float32)
        oracle.ref_sqdist(batch, m, n, k, X, sX, Y, sY, ref, sD)
        ws_n = batch * m + (1 if shared else batch) * n
        dD = torch.full((batch * m * n,), np.nan, device="cuda")
        ws = torch.empty(ws_n, device="cuda")
        sg.sgemm_pairwise_sqdist(batch, m, n, k, dev(X), *sX, dev(Y), *sY, dD, *sD, ws, ws_n,
                                 stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        e = _dist_err(X, Y, k, dD.cpu().numpy(), ref)
        assert e <= TOL, (batch, m, n, k, shared, x_major, e)
    X = rng.standard_normal(40 * 64).astype(np.float32)
    dX = dev(X)
    dD = torch.empty(40 * 40, device="cuda")
    ws = torch.empty(80, device="cuda")
    sg.sgemm_pairwise_sqdist(1, 40, 40, 64, dX, 0, 64, 1, dX, 0, 64, 1, dD, 0, 40, 1, ws, 80,
                             stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    diag = np.diagonal(dD.cpu().numpy().reshape(40, 40))
    assert np.abs(diag).max() <= TOL * 4 * 64 * float(np.abs(X).max()) ** 2


def test_pairwise_sqdist_workspace_errors():
    X = torch.zeros(8 * 4, device="cuda")
    D = torch.zeros(8 * 8, device="cuda")
    ws = torch.zeros(16, device="cuda")
    for bad_ws, floats in ((None, 16), (ws, 15)):
        with pytest.raises(sg.SgemmError) as e:
            sg.sgemm_pairwise_sqdist(1, 8, 8, 4, X, 0, 4, 1, X, 0, 4, 1, D, 0, 8, 1, bad_ws, floats)
        assert e.value.status == -8
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_pairwise_sqdist(1, 8, 8, 4, X, 0, 4, 1, X, 0, 4, 1, D, 0, 8, 1, D, 64)
    assert e.value.status == -4


def test_linear_bias_full_size():
    """The bias-fused linear layer at full size, as the benchmark runs it:
    every output against the oracle, and two calls give the same bits."""
    p = wl.workload("linear_bias")
    dA, dB, dC, dl = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage), dev(p.col.storage)
    s = torch.cuda.current_stream()
    sg.sgemm_strided_batched_ex(*p.ex_call_args(dA, dB, dC, None, dl), stream=s)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    ref = p.C.storage.copy()
    oracle.ref_sgemm_ex(p.batch, p.m, p.n, p.k, p.alpha, p.A.storage, p.A.strides, p.B.storage,
                        p.B.strides, p.beta_value, ref, p.C.strides, **_oracle_vec_args(p))
    gv = view(got, p.batch, p.m, p.n, p.C.strides)
    rv = view(ref, p.batch, p.m, p.n, p.C.strides)
    assert ex_err(p, gv, rv) <= TOL
    dC2 = dev(p.C.storage)
    sg.sgemm_strided_batched_ex(*p.ex_call_args(dA, dB, dC2, None, dl), stream=s)
    torch.cuda.synchronize()
    assert torch.equal(dC, dC2)


def test_sqdist_full_size():
    """The distance table at full size (4 x 4096 vectors against a shared
    1024-entry codebook, 512 features): every distance against the plain
    definition, and two calls give the same bits."""
    p = wl.workload("sqdist")
    dX, dY, dD = dev(p.X.storage), dev(p.Y.storage), dev(p.D.storage)
    ws = torch.empty(p.workspace_floats, device="cuda")
    s = torch.cuda.current_stream()
    sg.sgemm_pairwise_sqdist(*p.call_args(dX, dY, dD, ws), stream=s)
    torch.cuda.synchronize()
    got = dD.cpu().numpy()
    ref = p.D.storage.copy()
    oracle.ref_sqdist(p.batch, p.m, p.n, p.k, p.X.storage, p.X.strides, p.Y.storage, p.Y.strides,
                      ref, p.D.strides)
    gv = view(got, p.batch, p.m, p.n, p.D.strides)
    rv = view(ref, p.batch, p.m, p.n, p.D.strides)
    assert _dist_err(p.X.storage, p.Y.storage, p.k, gv, rv) <= TOL
    dD2 = torch.zeros_like(dD)
    sg.sgemm_pairwise_sqdist(*p.call_args(dX, dY, dD2, ws), stream=s)
    torch.cuda.synchronize()
    assert torch.equal(dD, dD2)
