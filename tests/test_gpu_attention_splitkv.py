"""GPU parity of split-KV attention (sgemm_attention_splitkv) against the CPU
oracle's attention, through the C ABI.

The chunked softmax and the merge regroup the keys' sums; the result must
meet the same derived bound as the fused kernel (tests/test_gpu_attention.py:
2 max|V| (2 Delta + (5 tk + 16) u), Delta the scores' rounding), be
reproducible bit for bit, and, when the call is not split (a prefill, g * tq
above 64, no workspace), equal sgemm_attention exactly.  Decode shapes cover
grouped KV heads with a partial last group, several queries per head (one to
four 16-row tiles per group, partial tiles, a last group whose second tile
has no row), causal and not, both layouts, ragged key counts and chunk
edges, forced chunk counts, and a workspace filled with NaN on entry.
"""
import numpy as np
import pytest

import oracle
import strided_fp32_gemm_amd as sg
from strided_fp32_gemm_amd import workloads as wl
from helpers import view4

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def describe(p, ws=-1):
    return sg.sgemm_attention_splitkv_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42, 1 << 43),
                                               workspace_floats=ws)


def split_call(p, ws=None, poison=True):
    plan = describe(p)
    floats = plan["workspace_floats"] if ws is None else ws
    dq, dk, dv, do = dev(p.Q.storage), dev(p.K.storage), dev(p.V.storage), dev(p.O.storage)
    W = torch.full((max(floats, 1),), float("nan") if poison else 0.0, device="cuda")
    sg.sgemm_attention_splitkv(*p.call_args(dq, dk, dv, do), W if floats else None, floats,
                               stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return do.cpu().numpy(), plan


def fused_call(p):
    dq, dk, dv, do = dev(p.Q.storage), dev(p.K.storage), dev(p.V.storage), dev(p.O.storage)
    sg.sgemm_attention(*p.call_args(dq, dk, dv, do), stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return do.cpu().numpy()


def oracle_call(p):
    O = p.O.storage.copy()
    oracle.ref_attention(*p.call_args(p.Q.storage, p.K.storage, p.V.storage, O))
    return O


def out(p, storage):
    return np.array(view4(storage, (p.nb_outer, p.nb_inner, p.tq, p.d), p.O.strides))


def tolerance(p):
    hk = -(-p.nb_inner // p.g)
    rows = lambda s, shape, st: np.array(view4(s, shape, st), dtype=np.float64)
    q = rows(p.Q.storage, (p.nb_outer, p.nb_inner, p.tq, p.d), p.Q.strides)
    k = rows(p.K.storage, (p.nb_outer, hk, p.tk, p.d), p.K.strides)
    v = rows(p.V.storage, (p.nb_outer, hk, p.tk, p.d), p.V.strides)
    qn = np.sqrt((q * q).sum(-1)).max(initial=0.0)
    kn = np.sqrt((k * k).sum(-1)).max(initial=0.0)
    delta = (p.d + 3) * U * abs(p.alpha) * qn * kn
    return 2.0 * np.abs(v).max(initial=0.0) * (2.0 * delta + (5 * p.tk + 16) * U)


def check(p, **kw):
    got, plan = split_call(p, **kw)
    ref = out(p, oracle_call(p))
    err = float(np.abs(out(p, got).astype(np.float64) - ref).max(initial=0.0))
    assert err <= tolerance(p), (p.name, plan, err, tolerance(p))
    return got, plan


DECODE = [  # (nb_outer, nb_inner, g, tq, tk, causal, order)
    (2, 6, 3, 1, 200, True, "tokens"),
    (1, 4, 1, 1, 1000, False, "heads"),
    (2, 8, 4, 2, 333, True, "tokens"),
    (1, 15, 3, 4, 517, True, "heads"),     # 12 rows per tile
    (1, 16, 16, 1, 4096, True, "tokens"),  # 16 query heads on one KV head
    (3, 5, 5, 3, 64, False, "heads"),      # 15 rows
    (1, 7, 3, 1, 300, True, "tokens"),     # groups of 3, 3 and 1 query heads
    (2, 4, 2, 8, 129, True, "tokens"),     # 16 rows, causal within the last 8 positions
    (1, 2, 1, 1, 17, False, "heads"),      # fewer keys than a block
    (2, 8, 8, 4, 700, True, "tokens"),     # 32 rows: two tiles
    (1, 12, 4, 16, 1000, True, "heads"),   # 64 rows: four tiles, causal over the last 16 positions
    (2, 6, 3, 7, 300, False, "tokens"),    # 21 rows: a partial second tile
    (1, 7, 7, 9, 257, True, "tokens"),     # 63 rows
    (3, 10, 4, 5, 400, True, "tokens"),    # groups of 4, 4, 2 heads: the last group's second tile is empty
]


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_decode_shapes(case):
    no, h, g, tq, tk, causal, order = case
    p = wl.random_attention(sum(case[:5]), no, h, tq, tk, 64, g=g, causal=causal, order=order)
    got, plan = check(p)
    assert plan["chunks"] > 0, plan
    assert np.array_equal(got, split_call(p, poison=False)[0])


@pytest.mark.parametrize("chunks", [1, 2, 7, 64])
def test_forced_chunk_counts(chunks, monkeypatch):
    """Chunk counts forced from one (a single partial per group) to more
    chunks than 32-key blocks allow (capped), with chunk edges inside the
    causal band of several queries."""
    monkeypatch.setenv("SGEMM_ATTN_CHUNKS", str(chunks))
    p = wl.random_attention(61 + chunks, 2, 6, 4, 777, 64, g=3, causal=True, order="tokens")
    _, plan = check(p)
    assert 1 <= plan["chunks"] <= chunks, plan


def test_large_scores_move_the_reference():
    """Scores in the hundreds (Q and K scaled by 4): each chunk's reference
    maximum moves past its slack, and the merge rescales chunks whose maxima
    differ by far more than the weights' range."""
    p = wl.random_attention(71, 2, 4, 1, 2000, 64, g=2, causal=True, order="heads", scale=4.0)
    check(p)


def test_unsplit_calls_run_as_sgemm_attention():
    """A prefill (g * tq above 64) and a decode without a workspace are not
    split: the same bits as sgemm_attention."""
    pre = wl.random_attention(81, 1, 4, 96, 96, 64, g=2, causal=True, order="tokens")
    assert describe(pre)["chunks"] == 0
    assert np.array_equal(split_call(pre)[0], fused_call(pre))
    dec = wl.random_attention(82, 2, 6, 1, 500, 64, g=3, causal=True, order="tokens")
    assert np.array_equal(split_call(dec, ws=0)[0], fused_call(dec))


def test_workspace_cap_gives_fewer_chunks():
    p = wl.random_attention(91, 1, 8, 1, 8192, 64, g=4, causal=True, order="tokens")
    best = describe(p)
    groups = 2
    cap = 5 * groups * (16 * 64 + 32)
    capped = describe(p, ws=cap)
    assert best["chunks"] > 5 and capped["chunks"] == 5 and capped["workspace_floats"] <= cap, (best, capped)
    check(p, ws=cap)


@pytest.mark.parametrize("name", [w for w in wl.WORKLOADS if wl.kind(w) == "attention_splitkv"])
def test_workload_full_size(name):
    """The decode workload at full size, in the configuration the benchmark
    times (the planned split and its workspace), against the oracle on
    every output; two calls give the same bits."""
    p = wl.workload(name)
    got, plan = check(p)
    assert plan["chunks"] > 1, plan
    assert np.array_equal(got, split_call(p, poison=False)[0])


@pytest.mark.parametrize("tq,causal", [(1, True), (4, True), (96, True), (3, False)])
def test_torch_attention_helper(tq, causal):
    """sg.attention on torch views of token-major buffers ([outer, t, heads,
    d] passed as .transpose(1, 2), no copy), grouped KV heads, on a side
    stream: decode-shaped calls take the split (workspace allocated by the
    helper), a prefill the fused kernel; both within the fused kernel's
    bound against the oracle."""
    no, h, g, tk, d = 2, 6, 3, 700, 64
    p = wl.random_attention(300 + tq, no, h, tq, tk, d, g=g, causal=causal, order="tokens")
    hk = h // g
    Q = dev(p.Q.storage).view(no, tq, h, d).transpose(1, 2)
    K = dev(p.K.storage).view(no, tk, hk, d).transpose(1, 2)
    V = dev(p.V.storage).view(no, tk, hk, d).transpose(1, 2)
    Ot = dev(p.O.storage)
    O = Ot.view(no, tq, h, d).transpose(1, 2)
    split = describe(p)["chunks"] > 0
    assert split == (tq * g <= 64), describe(p)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sg.attention(Q, K, V, O, alpha=p.alpha, causal=causal)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    got, ref = out(p, Ot.cpu().numpy()), out(p, oracle_call(p))
    err = float(np.abs(got.astype(np.float64) - ref).max())
    assert err <= tolerance(p), (tq, causal, err, tolerance(p))
