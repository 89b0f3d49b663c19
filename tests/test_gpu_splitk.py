"""GPU parity of the split-k entry point (sgemm_strided_batched_splitk)
against the CPU oracle, through the C ABI.

The partitions' partial products go to a caller workspace and one kernel
adds them in partition order, so the result must meet the product's error
bound (max |C - ref| / (k max|A| max|B|) <= 1e-6, as for every other path),
be reproducible bit for bit, and, when no split is planned (no workspace,
or SGEMM_SPLITK=1), equal sgemm_strided_batched exactly.  Forced splits
(SGEMM_SPLITK) cover partitions of equal depth and a shorter last one, the
vector and element reductions, accumulation, batches, column-major and
padded C, and a workspace filled with NaN on entry (every partial it reads
must have been written).
"""
import numpy as np
import pytest

import oracle
import strided_fp32_gemm_amd as sg
from strided_fp32_gemm_amd import workloads as wl
from helpers import view

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-6
LAYOUTS = [(a, b) for a in ("row", "col") for b in ("row", "col")]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def describe(p, ws=-1):
    """The plan with a workspace of ws floats (a stand-in address past the
    operands'), or with no cap when ws < 0."""
    return sg.sgemm_splitk_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42),
                                    workspace=(1 << 44) if ws >= 0 else None, workspace_floats=ws)


def split_call(p, ws_floats=None, poison=True):
    """Run p through the split-k entry point with a workspace of ws_floats
    (default: what the plan asks for); returns (C storage, plan)."""
    info = describe(p)
    floats = info["workspace_floats"] if ws_floats is None else ws_floats
    dA, dB, dC = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage)
    W = torch.full((max(floats, 1),), float("nan") if poison else 0.0, device="cuda")
    sg.sgemm_strided_batched_splitk(*p.call_args(dA, dB, dC), W if floats else None, floats,
                                    stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return dC.cpu().numpy(), info


def plain_call(p):
    dA, dB, dC = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage)
    sg.sgemm_strided_batched(*p.call_args(dA, dB, dC), stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def oracle_call(p):
    C = p.C.storage.copy()
    oracle.ref_sgemm(*p.call_args(p.A.storage, p.B.storage, C))
    return C


def out(p, C):
    return np.array(view(C, p.batch, p.m, p.n, p.C.strides))


def err_ratio(p, got, ref):
    amax = np.abs(view(p.A.storage, p.batch, p.m, p.k, p.A.strides)).max()
    bmax = np.abs(view(p.B.storage, p.batch, p.k, p.n, p.B.strides)).max()
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()
    return diff / (p.k * float(amax) * float(bmax))


@pytest.mark.parametrize("splits", [2, 3, 8])
def test_forced_splits_every_layout(splits, monkeypatch):
    """Forced splits on ragged shapes in all four transpose cases,
    accumulating and not: k a multiple of the partition depth and not (a
    shorter last partition, one more launch), n a multiple of 4 (16-byte
    reduction) and not, batches of 1 to 3, padded C rows (gaps untouched)."""
    monkeypatch.setenv("SGEMM_SPLITK", str(splits))
    shapes = [(2, 70, 96, 1024, 0), (1, 33, 50, 1000, 0), (3, 64, 128, 777, 2), (1, 130, 20, 520, 1)]
    for batch, m, n, k, pad in shapes:
        for a_major, b_major in LAYOUTS:
            for acc in (False, True):
                p = wl.random_problem(m + n + k + splits, batch, m, n, k, a_major=a_major, b_major=b_major,
                                      dist="normal", alpha=-0.625, accumulate=acc, pad=pad)
                got, info = split_call(p)
                # Partitions are a multiple of 64 deep: a short k gets fewer than asked.
                assert 2 <= info["splits"] <= splits, info
                assert info["launches"] == (2 if info["k_last"] == info["kc"] else 3), info
                ref = oracle_call(p)
                e = err_ratio(p, out(p, got), out(p, ref))
                assert e <= TOL, (splits, batch, m, n, k, a_major, b_major, acc, e)
                if pad:
                    # Gaps between C rows keep their initial values.
                    mask = np.ones(p.C.storage.size, bool)
                    idx = np.arange(p.C.storage.size, dtype=np.int32)   # view() takes 4-byte items
                    mask[np.array(view(idx, p.batch, p.m, p.n, p.C.strides)).ravel()] = False
                    assert np.array_equal(got[mask], p.C.storage[mask])


def test_shared_weight_and_integer_data(monkeypatch):
    """A B shared by every batch entry (batch stride 0, the partitions
    advance along its k only), and integer data in [-3, 3], where every
    partial sum and their total are exact in fp32, so the split result
    equals the oracle bit for bit."""
    monkeypatch.setenv("SGEMM_SPLITK", "4")
    for a_major, b_major in LAYOUTS:
        p = wl.random_problem(93, 3, 80, 72, 1100, a_major=a_major, b_major=b_major, dist="int",
                              b_broadcast=True, accumulate=True)
        got, info = split_call(p)
        assert info["splits"] == 4 and p.B.strides[0] == 0, info
        assert np.array_equal(out(p, got), out(p, oracle_call(p))), (a_major, b_major)


def test_column_major_c_and_determinism(monkeypatch):
    """A column-major C (element-wise reduction with a row stride of 1) and
    two calls with the same arguments giving the same bits."""
    monkeypatch.setenv("SGEMM_SPLITK", "4")
    p = wl.random_problem(77, 2, 90, 60, 900, a_major="row", b_major="col", c_major="col",
                          dist="normal", alpha=1.5, accumulate=True)
    got, info = split_call(p)
    assert info["splits"] == 4, info
    assert np.array_equal(got, split_call(p)[0])
    e = err_ratio(p, out(p, got), out(p, oracle_call(p)))
    assert e <= TOL, e


def test_unsplit_plan_equals_the_plain_entry_point(monkeypatch):
    """With no workspace, or SGEMM_SPLITK=1, the call is the plain product:
    same bits as sgemm_strided_batched."""
    p = wl.random_problem(91, 1, 128, 128, 8192, a_major="col", b_major="row", dist="normal",
                          accumulate=True)
    want = plain_call(p)
    got, _ = split_call(p, ws_floats=0)
    assert np.array_equal(got, want)
    monkeypatch.setenv("SGEMM_SPLITK", "1")
    got, info = split_call(p, ws_floats=1 << 20)
    assert info["splits"] == 1 and np.array_equal(got, want)


def test_workspace_cap_gives_a_smaller_split():
    """A workspace smaller than the best split needs gives the largest
    split that fits (here 4 partitions of 128 x 128), still within the
    bound."""
    p = wl.random_problem(92, 1, 128, 128, 65536, a_major="row", b_major="row", dist="normal")
    best = describe(p)
    assert best["splits"] >= 16, best
    cap = 4 * 128 * 128
    capped = describe(p, ws=cap)
    assert 2 <= capped["splits"] <= 4 and capped["workspace_floats"] <= cap, capped
    got, _ = split_call(p, ws_floats=cap)
    e = err_ratio(p, out(p, got), out(p, oracle_call(p)))
    assert e <= TOL, e


@pytest.mark.parametrize("shape", [(1, 256, 256, 16384, "col", "row"), (1, 128, 128, 65536, "row", "col"),
                                   (1, 64, 64, 262144, "col", "row"), (4, 256, 256, 8192, "row", "row"),
                                   (1, 384, 768, 16384, "col", "col")])
def test_deep_k_products_on_the_planner_choice(shape):
    """Small outputs over deep contractions, the case the split is for: the
    planner splits them (its own choice of partitions and kernels) and every
    output meets the bound."""
    batch, m, n, k, a_major, b_major = shape
    p = wl.random_problem(sum(shape[:4]), batch, m, n, k, a_major=a_major, b_major=b_major, dist="normal",
                          alpha=0.5, accumulate=True)
    got, info = split_call(p)
    assert info["splits"] >= 4, info
    e = err_ratio(p, out(p, got), out(p, oracle_call(p)))
    assert e <= TOL, (shape, info["splits"], info["parts"]["kernel"], e)


@pytest.mark.parametrize("name", [w for w in wl.WORKLOADS if wl.kind(w) == "splitk"])
def test_workload_full_size(name):
    """The split-k benchmark workload at full size, in the configuration
    the benchmark times (the planner's split, its workspace), compared with
    the oracle on every output; two calls give the same bits."""
    p = wl.workload(name)
    got, info = split_call(p, poison=True)
    assert info["splits"] > 1, info
    assert np.array_equal(got, split_call(p, poison=False)[0])
    e = err_ratio(p, out(p, got), out(p, oracle_call(p)))
    assert e <= TOL, (name, info["splits"], e)


def test_torch_helper_splitk():
    """sgemm(..., splitk=True) on torch views: the weight gradient dy^T x
    (dy.t() passed as a view, no copy), on a side stream, accumulating; the
    helper allocates the workspace the plan asks for with torch."""
    g = torch.Generator().manual_seed(5)
    dy = torch.randn(12288, 192, generator=g)
    x = torch.randn(12288, 160, generator=g)
    c0 = torch.randn(192, 160, generator=g)
    ref = (dy.double().t() @ x.double()) * 0.5 + c0.double()
    dyd, xd = dy.cuda(), x.cuda()
    C = c0.cuda()
    plan = sg.sgemm_splitk_describe(1, 192, 160, 12288, 0.5, dyd, 0, 1, 192, xd, 0, 160, 1, 1, C, 0, 160, 1)
    assert plan["splits"] > 1, plan
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sg.sgemm(dyd.t(), xd, C, alpha=0.5, accumulate=True, splitk=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    e = float((C.cpu().double() - ref).abs().max()) / (12288 * float(dy.abs().max()) * float(x.abs().max()))
    assert e <= TOL, e
