"""GPU parity of fused attention (sgemm_attention) through the C ABI, against
the CPU oracle's attention on the same host bytes.

Tolerance, derived from the fp32 arithmetic (u = 2^-24):
  * each score alpha*<q, k> carries an error of at most
    Delta = (d + 3) * u * |alpha| * |q|_2 * |k|_2 (the d-term sum, the scale,
    the subtraction of the reference maximum and exp2's argument; the
    matrix-core kernel scales Q once and starts the d-term sum from minus the
    reference, which is itself one of the row's scaled scores, so its terms
    are the same ones);
  * logits perturbed by at most Delta move the softmax weights by at most
    2*Delta in the 1-norm, so the output moves by at most 2*Delta*max|V|;
  * the weights' own rounding, the rescaling of the running sums (at most
    once per key; weights may reach 2^8 between rescalings, which changes no
    relative error) and the tk-term sums of the weights and of P V add at
    most (5*tk + 16)*u relative to max|V|.
  max |O_gpu - O_ref| <= 2 * max|V| * (2*Delta + (5*tk + 16)*u), with the
  largest row norms of Q and K; the outer factor 2 covers second-order terms.
Bitwise checks cover what must not depend on the launch: two calls, grouped
KV heads against repeated ones, and a query row against the same row computed
as a decode over its own context.  A missing GPU is a failure, not a skip.
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
PATHS = [sg.PATH_AUTO, sg.PATH_MFMA, sg.PATH_GENERIC]
PATH_IDS = ["auto", "mfma", "generic"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible: GPU parity cannot pass without one"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def gpu_call(p, path=sg.PATH_AUTO, O0=None):
    dq, dk, dv = dev(p.Q.storage), dev(p.K.storage), dev(p.V.storage)
    do = dev(p.O.storage if O0 is None else O0)
    sg.sgemm_attention_path(*p.call_args(dq, dk, dv, do), path=path, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    return do.cpu().numpy()


def oracle_call(p):
    O = p.O.storage.copy()
    oracle.ref_attention(*p.call_args(p.Q.storage, p.K.storage, p.V.storage, O))
    return O


def describe(p, path=sg.PATH_AUTO):
    return sg.sgemm_attention_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42, 1 << 43), path=path)


def out(p, storage):
    return np.array(view4(storage, (p.nb_outer, p.nb_inner, p.tq, p.d), p.O.strides))


def _rows(storage, shape, strides):
    return np.array(view4(storage, shape, strides), dtype=np.float64)


def tolerance(p):
    hk = -(-p.nb_inner // p.g)
    q = _rows(p.Q.storage, (p.nb_outer, p.nb_inner, p.tq, p.d), p.Q.strides)
    k = _rows(p.K.storage, (p.nb_outer, hk, p.tk, p.d), p.K.strides)
    v = _rows(p.V.storage, (p.nb_outer, hk, p.tk, p.d), p.V.strides)
    qn = np.sqrt((q * q).sum(-1)).max(initial=0.0)
    kn = np.sqrt((k * k).sum(-1)).max(initial=0.0)
    delta = (p.d + 3) * U * abs(p.alpha) * qn * kn
    return 2.0 * np.abs(v).max(initial=0.0) * (2.0 * delta + (5 * p.tk + 16) * U)


def check(p, path=sg.PATH_AUTO):
    got, ref = out(p, gpu_call(p, path)), out(p, oracle_call(p))
    err = float(np.abs(got.astype(np.float64) - ref).max(initial=0.0))
    tol = tolerance(p)
    assert err <= tol, (p.name, path, describe(p, path)["kernel"], err, tol)
    return got


CASES = [  # (nb_outer, nb_inner, g, tq, tk, d, causal, order)
    (2, 6, 3, 77, 77, 64, True, "tokens"),     # ragged prefill, grouped KV heads
    (1, 4, 1, 64, 64, 64, False, "heads"),     # exactly one block
    (2, 2, 2, 1, 200, 64, True, "tokens"),     # one decode query per head
    (1, 3, 1, 130, 300, 64, True, "heads"),    # a chunk of queries at the end of a longer context
    (2, 5, 5, 33, 130, 64, False, "tokens"),   # every query head on one KV head
    (1, 2, 1, 200, 17, 64, False, "heads"),    # fewer keys than a block
    (3, 1, 1, 129, 129, 64, True, "heads"),    # 128-query workgroups plus one row
    (1, 16, 4, 256, 256, 64, True, "tokens"),
]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_attention_every_path(path):
    """Each kernel, forced, on prefill, decode and chunked shapes, causal and
    not, with grouped KV heads, ragged query and key counts, both layouts."""
    for no, h, g, tq, tk, d, causal, order in CASES:
        p = wl.random_attention(no * 100 + h * 10 + tq + tk, no, h, tq, tk, d, g=g, causal=causal,
                                order=order)
        if path != sg.PATH_GENERIC:
            assert describe(p, path)["kernel"].startswith("attn_mfma_d64"), describe(p, path)
        check(p, path)


def test_attention_four_wave_workgroups(monkeypatch):
    """The matrix-core kernel with 4 wavefronts (64 query rows) per
    workgroup, forced, on the same shapes (odd and even counts of causal
    half-blocks)."""
    monkeypatch.setenv("SGEMM_ATTN_WAVES", "4")
    for no, h, g, tq, tk, d, causal, order in CASES:
        p = wl.random_attention(no * 100 + h * 10 + tq + tk + 1, no, h, tq, tk, d, g=g, causal=causal,
                                order=order)
        assert describe(p)["kernel"].startswith("attn_mfma_d64_w4"), describe(p)
        check(p)


@pytest.mark.parametrize("d", [1, 7, 32, 100, 256])
def test_attention_generic_head_dims(d):
    """Head dimensions the matrix-core kernel does not take run on the
    generic kernel (chosen automatically) within the same bound."""
    for causal in (False, True):
        p = wl.random_attention(d + causal, 2, 3, 45, 70, d, g=3, causal=causal, order="tokens")
        assert describe(p)["kernel"].startswith("attn_generic"), describe(p)
        check(p)


def test_attention_unaligned_layouts_take_the_generic_kernel():
    """Rows that are not 16-byte aligned, or a non-unit column stride, are
    served by the generic kernel; the result still meets the bound."""
    p = wl.random_attention(5, 2, 2, 40, 50, 64, order="heads")
    rng = np.random.default_rng(5)
    no, h, tq, d = p.nb_outer, p.nb_inner, p.tq, p.d
    p.Q = wl.Operand2(rng.standard_normal(no * h * tq * (d + 1)).astype(np.float32),
                      (h * tq * (d + 1), tq * (d + 1), d + 1, 1))     # rows 65 floats apart
    q = wl.random_attention(6, 1, 2, 30, 40, 64, order="heads")
    q.K = wl.Operand2(np.ascontiguousarray(np.repeat(q.K.storage, 2)),
                      tuple(2 * s for s in q.K.strides))    # column stride 2
    for prob in (p, q):
        assert describe(prob)["kernel"].startswith("attn_generic"), describe(prob)
        check(prob)


def test_attention_bitwise_invariants():
    """On the matrix-core kernel: two calls agree bit for bit; grouped KV
    heads give the bits of each KV head copied for its query heads; every
    row of a causal prefill equals the decode of that row over its own
    context (keys 0..q), whatever workgroup computed it."""
    p = wl.random_attention(31, 2, 6, 150, 150, 64, g=3, causal=True, order="tokens")
    a = gpu_call(p)
    assert np.array_equal(a, gpu_call(p))
    no, h, tk, d = p.nb_outer, p.nb_inner, p.tk, p.d
    K = view4(p.K.storage, (no, 2, tk, d), p.K.strides)
    V = view4(p.V.storage, (no, 2, tk, d), p.V.strides)

    def token_major(X):      # [o][head][t][d] -> stored [o][t][head][d]
        return np.ascontiguousarray(X.transpose(0, 2, 1, 3)).ravel()
    sk = (tk * h * d, d, h * d, 1)
    rep = wl.AttnProblem("rep", no, h, p.tq, tk, d, 1, p.alpha, True, p.Q,
                         wl.Operand2(token_major(np.repeat(K, 3, 1)), sk),
                         wl.Operand2(token_major(np.repeat(V, 3, 1)), sk), p.O)
    assert describe(rep)["kernel"] == describe(p)["kernel"]
    assert np.array_equal(gpu_call(rep), a)
    full = out(p, a)
    for q in (0, 63, 64, 100, 149):
        dec = wl.AttnProblem("dec", no, h, 1, q + 1, d, p.g, p.alpha, True,
                             wl.Operand2(p.Q.storage[q * p.Q.strides[2]:], p.Q.strides), p.K, p.V,
                             wl.Operand2(np.zeros(no * h * d * 4, np.float32), (h * d, d, 0, 1)))
        got = out(dec, gpu_call(dec))
        assert np.array_equal(got[:, :, 0], full[:, :, q]), q


def test_attention_large_scores():
    """Scores in the hundreds (Q and K scaled by 4, alpha 1): only a softmax
    that subtracts the running maximum stays finite and within the bound."""
    for causal in (False, True):
        p = wl.random_attention(41 + causal, 1, 4, 96, 96, 64, g=2, causal=causal, alpha=1.0, scale=4.0)
        got = check(p)
        assert np.all(np.isfinite(got))


def _block_trend_problem(seed, step, causal):
    """Scores that move by `step` (log2 units, alpha*log2(e)*score) from one
    64-key block to the next: Q rows are a shared unit vector u plus a little
    noise, K row j is u scaled to put its score near step * (j // 64), plus
    the same noise.  Rising scores move the matrix-core kernel's reference
    maximum on every block (each move well past its 2^8 slack); falling ones
    leave it at the first block and drive the later weights to zero."""
    p = wl.random_attention(seed, 1, 4, 200, 320, 64, g=2, causal=causal, alpha=0.125, scale=0.05)
    c2 = p.alpha * 1.4426950408889634
    u = np.ones(p.d) / np.sqrt(p.d)
    hk = -(-p.nb_inner // p.g)
    def flat(shape, strides):   # storage index of every element
        grids = np.meshgrid(*[np.arange(n) for n in shape], indexing="ij")
        return sum(gr * st for gr, st in zip(grids, strides))
    iq = flat((p.nb_outer, p.nb_inner, p.tq, p.d), p.Q.strides)
    ik = flat((p.nb_outer, hk, p.tk, p.d), p.K.strides)
    target = step * (np.arange(p.tk) // 64) / c2            # score wanted for key j
    p.Q.storage[iq] = (p.Q.storage[iq] + u).astype(np.float32)
    p.K.storage[ik] = (p.K.storage[ik] + target[None, None, :, None] * u).astype(np.float32)
    return p


@pytest.mark.parametrize("step", [10.0, -10.0, 3.0], ids=["rising", "falling", "within_slack"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_attention_reference_moves(step, causal):
    """The online softmax against the oracle when the row maxima rise past
    the matrix-core kernel's slack on every key block, fall after the first,
    or rise within the slack (the reference stays put and weights exceed 1)."""
    p = _block_trend_problem(61, step, causal)
    assert describe(p)["kernel"].startswith("attn_mfma_d64")
    got = check(p)
    assert np.all(np.isfinite(got))


def test_attention_never_reads_O_and_leaves_gaps():
    """O starts as NaN inside and as a sentinel in the gaps between rows,
    heads and sequences: outputs come out finite and the gaps untouched."""
    for path in PATHS:
        p = wl.random_attention(51, 2, 3, 70, 90, 64, g=3, causal=True, order="heads")
        d, tq, h = p.d, p.tq, p.nb_inner
        so = ((h * (tq * (d + 8) + 4)) + 12, tq * (d + 8) + 4, d + 8, 1)
        store = np.full(2 * so[0], -7.5, np.float32)
        idx = (np.arange(2)[:, None, None, None] * so[0] + np.arange(h)[None, :, None, None] * so[1]
               + np.arange(tq)[None, None, :, None] * so[2] + np.arange(d)[None, None, None, :]).ravel()
        store[idx] = np.nan
        q = wl.AttnProblem(p.name, 2, h, tq, p.tk, d, p.g, p.alpha, True, p.Q, p.K, p.V,
                           wl.Operand2(store, so))
        got = gpu_call(q, path)
        assert np.all(np.isfinite(got[idx])), path
        mask = np.ones(store.size, bool)
        mask[idx] = False
        assert np.all(got[mask] == -7.5), path
        q.O.storage = np.zeros_like(store)
        ref = oracle_call(q)
        assert np.abs(got[idx].astype(np.float64) - ref[idx]).max() <= tolerance(q), path


@pytest.mark.parametrize("name", ["attn_fused", "attn_fused_causal"])
def test_attention_full_size_workload(name):
    """The benchmark's fused attention at full size, in the configuration it
    times, against the oracle on every output; a second call gives the same
    bits."""
    p = wl.workload(name)
    got = check(p)
    assert np.array_equal(out(p, gpu_call(p)), got)
