"""The entry points under HIP graph capture: a strided batched product that
accumulates, a fused causal attention, the allocation-free distance entry
point, a split-k product (its partial products, a shorter last
partition and the reduction: three launches through a caller workspace) and
a split-KV decode attention (chunks and merge through a workspace),
captured together on one stream and replayed several times, with eager work
(resetting C, a host round trip) between the replays.  Every replay must
give the eager results bit for bit: the library enqueues only kernels (no
allocation, no memset), so a replay is the same launches on the same bytes.
"""
import numpy as np
import pytest

import strided_fp32_gemm_amd as sg
from strided_fp32_gemm_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def test_graph_replays_match_eager_calls():
    gemm = wl.random_problem(5101, 3, 200, 170, 96, a_major="col", b_major="row", dist="normal",
                             alpha=0.75, accumulate=True)
    attn = wl.random_attention(5102, 2, 6, 150, 150, 64, g=3, causal=True, order="tokens")
    rng = np.random.default_rng(5103)
    batch, m, n, k = 2, 120, 90, 48
    X = rng.standard_normal(batch * m * k).astype(np.float32)
    Y = rng.standard_normal(batch * n * k).astype(np.float32)
    sX, sY, sD = (m * k, k, 1), (n * k, k, 1), (m * n, n, 1)

    dA, dB, C0 = dev(gemm.A.storage), dev(gemm.B.storage), dev(gemm.C.storage)
    dC = C0.clone()
    dq, dk, dv = dev(attn.Q.storage), dev(attn.K.storage), dev(attn.V.storage)
    do = dev(attn.O.storage)
    dX, dY = dev(X), dev(Y)
    dD = torch.zeros(batch * m * n, device="cuda")
    deep = wl.random_problem(5104, 1, 96, 96, 16284, a_major="col", b_major="row", dist="normal",
                             alpha=0.5, accumulate=True)
    plan = sg.sgemm_splitk_describe(*deep.call_args(1 << 40, 1 << 41, 1 << 42))
    assert plan["splits"] > 1 and plan["launches"] == 3, plan
    dA2, dB2, E0 = dev(deep.A.storage), dev(deep.B.storage), dev(deep.C.storage)
    dE = E0.clone()
    W = torch.empty(plan["workspace_floats"], device="cuda")
    dec = wl.random_attention(5105, 2, 6, 1, 700, 64, g=3, causal=True, order="tokens")
    dplan = sg.sgemm_attention_splitkv_describe(*dec.call_args(1 << 40, 1 << 41, 1 << 42, 1 << 43))
    assert dplan["chunks"] > 1, dplan
    eq, ek, ev, eo = dev(dec.Q.storage), dev(dec.K.storage), dev(dec.V.storage), dev(dec.O.storage)
    W2 = torch.empty(dplan["workspace_floats"], device="cuda")

    def enqueue(stream):
        sg.sgemm_strided_batched(*gemm.call_args(dA, dB, dC), stream=stream)
        sg.sgemm_attention(*attn.call_args(dq, dk, dv, do), stream=stream)
        sg.sgemm_pairwise_sqdist_noalloc(batch, m, n, k, dX, *sX, dY, *sY, dD, *sD, stream=stream)
        sg.sgemm_strided_batched_splitk(*deep.call_args(dA2, dB2, dE), W, W.numel(), stream=stream)
        sg.sgemm_attention_splitkv(*dec.call_args(eq, ek, ev, eo), W2, W2.numel(), stream=stream)

    # Eager results (this also does any one-time set-up outside the capture).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enqueue(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = [dC.cpu().numpy(), do.cpu().numpy(), dD.cpu().numpy(), dE.cpu().numpy(), eo.cpu().numpy()]

    graph = torch.cuda.CUDAGraph()
    dC.copy_(C0)
    dE.copy_(E0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        enqueue(torch.cuda.current_stream())
    for replay in range(4):
        # Eager work between replays: C back to its initial values (the
        # product accumulates), the other outputs poisoned, a host round trip.
        dC.copy_(C0)
        dE.copy_(E0)
        do.fill_(float("nan"))
        dD.fill_(float("nan"))
        W.fill_(float("nan"))
        W2.fill_(float("nan"))
        eo.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [dC.cpu().numpy(), do.cpu().numpy(), dD.cpu().numpy(), dE.cpu().numpy(), eo.cpu().numpy()]
        for name, g_, w_ in zip(("product", "attention", "distances", "split-k product", "split-KV decode"),
                                got, want):
            assert np.array_equal(g_, w_), (replay, name)
