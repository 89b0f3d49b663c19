"""GPU parity of the two-level batch (sgemm_strided_batched2) through the C
ABI, against the CPU oracle's two-level product on the same host bytes.

Layouts are those of attention over [sequence][token][head][dim] buffers
(outer = sequence, inner = head, rows = tokens) with grouped key/value heads
(several query heads read one KV head), and head-major ones.  The bar is the
product's: max |C_gpu - C_ref| / (k * max|A| * max|B|) <= 1e-6 over the
logical outputs, bitwise where the result is unique (integer operands) or
where two calls must do the same arithmetic (one batch level, repeated KV
heads).  A missing GPU is a failure here, not a skip.
"""
import numpy as np
import pytest

import oracle
import strided_fp32_gemm_amd as sg
from strided_fp32_gemm_amd import workloads as wl
from helpers import view4

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-6
FAMILIES = [sg.PATH_AUTO, sg.PATH_MFMA, sg.PATH_WAVE, sg.PATH_GENERIC]
FAM_IDS = ["auto", "mfma", "wave", "generic"]
# (a_order, a_trans, b_order, b_trans, c_order, c_trans): the scores Q K^T
# from token-major Q and K into head-major S; the context P V from head-major P
# and token-major V into token-major O; head-major throughout; and the scores
# stored transposed (C column-major, computed as C^T = B^T A^T).
LAYOUTS = {
    "qk": ("tokens", False, "tokens", True, "heads", False),
    "pv": ("heads", False, "tokens", False, "tokens", False),
    "heads": ("heads", False, "heads", False, "heads", False),
    "qk_ct": ("tokens", False, "tokens", True, "heads", True),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible: GPU parity cannot pass without one"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def problem(seed, no, ni, m, n, k, layout, gA=1, gB=1, **kw):
    ao, at, bo, bt, co, ct = LAYOUTS[layout]
    return wl.random_problem2(seed, no, ni, m, n, k, gA=gA, gB=gB, a_order=ao, a_trans=at,
                              b_order=bo, b_trans=bt, c_order=co, c_trans=ct, **kw)


def gpu_call(p, path=sg.PATH_AUTO):
    dA, dB, dC = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage)
    sg.sgemm_strided_batched2_path(*p.call_args(dA, dB, dC), path=path,
                                   stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def oracle_call(p):
    C = p.C.storage.copy()
    oracle.ref_sgemm_batched2(*p.call_args(p.A.storage, p.B.storage, C))
    return C


def describe(p, path=sg.PATH_AUTO):
    return sg.sgemm_plan_describe2(*p.call_args(1 << 40, 1 << 41, 1 << 42), path=path)


def out(p, storage):
    return np.array(view4(storage, (p.nb_outer, p.nb_inner, p.m, p.n), p.C.strides))


def err_ratio(p, got, ref):
    na, nb = -(-p.nb_inner // p.A.group), -(-p.nb_inner // p.B.group)
    amax = np.abs(view4(p.A.storage, (p.nb_outer, na, p.m, p.k), p.A.strides)).max(initial=0.0)
    bmax = np.abs(view4(p.B.storage, (p.nb_outer, nb, p.k, p.n), p.B.strides)).max(initial=0.0)
    scale = max(p.k * float(amax) * float(bmax), 1e-30)
    return float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max(initial=0.0)) / scale


CASES = [  # (nb_outer, nb_inner, m, n, k, layout, gA, gB)
    (3, 6, 77, 45, 37, "qk", 1, 3),
    (2, 4, 130, 200, 64, "qk", 1, 2),
    (1, 15, 64, 64, 64, "qk", 1, 3),
    (2, 6, 150, 64, 96, "pv", 1, 3),
    (3, 5, 33, 20, 70, "pv", 1, 5),
    (2, 4, 96, 130, 40, "heads", 2, 1),
    (2, 7, 65, 66, 67, "heads", 3, 2),
    (4, 1, 100, 90, 50, "qk", 1, 1),
    (2, 6, 90, 140, 64, "qk_ct", 1, 3),
    (3, 4, 72, 56, 48, "qk_ct", 2, 1),
]


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_two_levels_every_family(path):
    """Every kernel family, forced, over the attention layouts with grouped
    heads on either input, ragged multi-tile shapes, accumulating and not."""
    for no, ni, m, n, k, layout, gA, gB in CASES:
        for acc in (False, True):
            p = problem(no * 1000 + ni * 100 + m + n + k, no, ni, m, n, k, layout, gA, gB,
                        alpha=0.6, accumulate=acc)
            got, ref = out(p, gpu_call(p, path)), out(p, oracle_call(p))
            e = err_ratio(p, got, ref)
            assert e <= TOL, (path, no, ni, m, n, k, layout, gA, gB, acc, e)


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_two_levels_integer_bitwise(path):
    """Integer operands make every partial sum exact: the result is unique and
    must match the oracle bit for bit."""
    for no, ni, m, n, k, layout, gA, gB in CASES:
        p = problem(7 + m * n, no, ni, m, n, k, layout, gA, gB, alpha=1.0, accumulate=True,
                    dist="int")
        got, ref = gpu_call(p, path), oracle_call(p)
        assert np.array_equal(got, ref), (path, no, ni, m, n, k, layout)


@pytest.mark.parametrize("tile", ["p64x64k64", "p128x64k64", "p64x128k64", "s64k64", "s128k64", "s128r2k64"])
def test_two_levels_persistent(tile, monkeypatch):
    """Each persistent short-k tile, forced, with the tile list crossing
    sequences and heads (grid capped so each workgroup visits many tiles),
    and each strip tile on the score layouts it serves."""
    monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
    monkeypatch.setenv("SGEMM_PERSIST_WGS", "13")
    for no, ni, m, n, k, layout, gB in [(3, 6, 200, 136, 64, "qk", 3), (2, 4, 64, 64, 32, "qk", 2),
                                        (2, 6, 132, 64, 64, "pv", 3), (5, 3, 68, 72, 16, "heads", 3),
                                        (2, 6, 136, 200, 64, "qk_ct", 3)]:
        for acc in (False, True):
            p = problem(no + ni + m + n + k, no, ni, m, n, k, layout, 1, gB, alpha=-1.25,
                        accumulate=acc)
            if tile.startswith("s") and not (layout.startswith("qk")):
                continue   # the strip kernel serves k-contiguous A and B only
            assert describe(p)["kernel"].startswith(("persist_", "strip_")) and tile in describe(p)["kernel"], \
                describe(p)
            got, ref = out(p, gpu_call(p)), out(p, oracle_call(p))
            e = err_ratio(p, got, ref)
            assert e <= TOL, (tile, no, ni, m, n, k, layout, acc, e)


def test_one_level_is_the_plain_entry_point():
    """nb_inner = 1 is sgemm_strided_batched over the outer level, and
    nb_outer = 1 with groups 1 is sgemm_strided_batched over the inner level:
    same plan, same bits."""
    p = problem(11, 5, 1, 140, 96, 64, "qk")
    got = gpu_call(p)
    dA, dB, dC = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage)
    (ao, _, ar, ac), (bo, _, br, bc), (co, _, cr, cc) = p.A.strides, p.B.strides, p.C.strides
    sg.sgemm_strided_batched(5, p.m, p.n, p.k, p.alpha, dA, ao, ar, ac, dB, bo, br, bc, 0,
                             dC, co, cr, cc, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(got, dC.cpu().numpy())

    p = problem(12, 1, 6, 140, 96, 64, "pv")
    got = gpu_call(p)
    dA, dB, dC = dev(p.A.storage), dev(p.B.storage), dev(p.C.storage)
    (_, ai, ar, ac), (_, bi, br, bc), (_, ci, cr, cc) = p.A.strides, p.B.strides, p.C.strides
    sg.sgemm_strided_batched(6, p.m, p.n, p.k, p.alpha, dA, ai, ar, ac, dB, bi, br, bc, 0,
                             dC, ci, cr, cc, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(got, dC.cpu().numpy())


def test_grouped_heads_equal_repeated_heads():
    """Reading one KV head for a group of query heads gives the very bits of
    the same call with that head copied once per query head (gB = 1)."""
    p = problem(21, 2, 6, 128, 192, 64, "qk", 1, 3)
    assert p.nb_inner // p.B.group == 2
    no, ni, d, t = p.nb_outer, p.nb_inner, p.k, p.n
    K = view4(p.B.storage, (no, 2, d, t), p.B.strides)            # [o][kv][d][t]
    rep = np.repeat(np.array(K), 3, axis=1)                       # [o][ni][d][t]
    Kt = np.ascontiguousarray(rep.transpose(0, 3, 1, 2))          # stored [o][t][ni][d]
    q = wl.Problem2(p.name, no, ni, p.m, p.n, p.k, p.alpha, False, p.A,
                    wl.Operand2(Kt.ravel(), (t * ni * d, d, 1, ni * d), 1), p.C)
    assert describe(q)["kernel"] == describe(p)["kernel"]
    assert np.array_equal(gpu_call(p), gpu_call(q))


def test_gaps_between_heads_are_untouched():
    """C with unused elements between rows, heads and sequences: only the
    logical outputs change; the gaps keep their bytes."""
    for path in FAMILIES:
        p = problem(31, 2, 3, 70, 90, 40, "qk", 1, 3, alpha=1.5)
        m, n = p.m, p.n
        sc = (3 * (m * (n + 3) + 11) + 5, m * (n + 3) + 11, n + 3, 1)
        size = 2 * sc[0]
        fill = np.full(size, -7.5, np.float32)
        q = wl.Problem2(p.name, 2, 3, m, n, p.k, p.alpha, False, p.A, p.B,
                        wl.Operand2(fill, sc))
        got = gpu_call(q, path)
        ref = oracle_call(q)
        e = err_ratio(q, out(q, got), out(q, ref))
        assert e <= TOL, (path, e)
        mask = np.ones(size, bool)
        idx = (np.arange(2)[:, None, None, None] * sc[0] + np.arange(3)[None, :, None, None] * sc[1]
               + np.arange(m)[None, None, :, None] * sc[2] + np.arange(n)[None, None, None, :])
        mask[idx.ravel()] = False
        assert np.all(got[mask] == -7.5), path


@pytest.mark.parametrize("name", ["attn_qk_gqa", "attn_pv_gqa"])
def test_full_size_workload(name):
    """The benchmark's two-level attention products at full size, in the
    configuration it times (planner's choice), against the oracle on every
    output; a second call gives the same bits."""
    p = wl.workload(name)
    got = gpu_call(p)
    ref = oracle_call(p)
    e = err_ratio(p, out(p, got), out(p, ref))
    assert e <= TOL, (name, describe(p)["kernel"], e)
    assert np.array_equal(got, gpu_call(p)), name
