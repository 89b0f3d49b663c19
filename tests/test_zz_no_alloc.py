"""The allocation-free distance entry point (sgemm_pairwise_sqdist_noalloc)
against the workspace entry point (sgemm_pairwise_sqdist), through the C ABI.

Both run the same norm and product kernels in the same order, so the
distances must agree bit for bit; they are also held to the oracle's bound.
Two calls in a row, the second smaller than the first, show that what the
first call left in the library's device scratch does not leak into the
second.  A call at the scratch's exact capacity works, one float beyond it
is refused before anything is enqueued.
"""
import numpy as np
import pytest

import oracle
import strided_fp32_gemm_amd as sg

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _case(rng, batch, m, n, k, shared):
    X = rng.standard_normal(batch * m * k).astype(np.float32)
    ny = 1 if shared else batch
    Y = rng.standard_normal(ny * n * k).astype(np.float32)
    sX = (m * k, k, 1)
    sY = (0 if shared else n * k, k, 1)
    sD = (m * n, n, 1)
    return X, Y, sX, sY, sD


def _both(batch, m, n, k, X, Y, sX, sY, sD):
    s = torch.cuda.current_stream()
    dX, dY = dev(X), dev(Y)
    d_ref = torch.full((batch * m * n,), float("nan"), device="cuda")
    d_new = torch.full((batch * m * n,), float("nan"), device="cuda")
    ny = 1 if sY[0] == 0 else batch
    ws = torch.empty(batch * m + ny * n, device="cuda")
    sg.sgemm_pairwise_sqdist(batch, m, n, k, dX, *sX, dY, *sY, d_ref, *sD, ws, ws.numel(), stream=s)
    sg.sgemm_pairwise_sqdist_noalloc(batch, m, n, k, dX, *sX, dY, *sY, d_new, *sD, stream=s)
    torch.cuda.synchronize()
    return d_ref.cpu().numpy(), d_new.cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls():
    rng = np.random.default_rng(1207)
    for batch, m, n, k, shared in ((3, 300, 200, 96, False), (1, 50, 70, 33, True)):
        X, Y, sX, sY, sD = _case(rng, batch, m, n, k, shared)
        ref_gpu, got = _both(batch, m, n, k, X, Y, sX, sY, sD)
        assert np.array_equal(got, ref_gpu), (batch, m, n, k)
        ref = np.zeros(batch * m * n, np.float32)
        oracle.ref_sqdist(batch, m, n, k, X, sX, Y, sY, ref, sD)
        xm, ym = float(np.abs(X).max()), float(np.abs(Y).max())
        bound = 2 * k * xm * ym + k * xm * xm + k * ym * ym
        assert float(np.abs(got.astype(np.float64) - ref).max()) / bound <= TOL


def test_noalloc_capacity_limit():
    cap = sg.SCRATCH_FLOATS
    rng = np.random.default_rng(1208)
    n, k = 64, 4
    m = cap - n                       # batch*m + n == capacity: accepted
    X, Y, sX, sY, sD = _case(rng, 1, m, n, k, True)
    ref_gpu, got = _both(1, m, n, k, X, Y, sX, sY, sD)
    assert np.array_equal(got, ref_gpu)
    # One norm beyond the capacity: refused, nothing written.
    dX, dY = dev(np.zeros((m + 1) * k, np.float32)), dev(Y)
    D = torch.full(((m + 1) * n,), 7.0, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_pairwise_sqdist_noalloc(1, m + 1, n, k, dX, (m + 1) * k, k, 1, dY, 0, k, 1,
                                         D, (m + 1) * n, n, 1)
    assert e.value.status == -8 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((D == 7.0).all())
