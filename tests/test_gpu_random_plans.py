"""GPU parity on seeded random products, each on the planner's own choice.

The forced-tile tests cover every kernel configuration on chosen shapes;
this sweep covers what the planner actually picks across shapes drawn at
random: batch 1-4, m and n from 1 to 300 (skinny ones included), k from 1
to 5000 (deep ones included), every storage order of A, B and C, padded
rows, accumulation, alpha.  Each product runs through the plain entry point
and through the split-k entry point (with the workspace its plan asks
for), and both must meet the product's bound against the oracle,
max |C - ref| / (k max|A| max|B|) <= 1e-6.  The drawn cases and the
kernels they ran on are printed, so a failure names its case.
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
CASES = 240


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    sg.load()


def draw_cases(seed=2024_07, count=CASES):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(count):
        batch = int(rng.integers(1, 5))
        dims = []
        for _ in range(2):
            r = rng.random()
            dims.append(int(rng.integers(1, 17)) if r < 0.3 else int(rng.integers(17, 301)))
        r = rng.random()
        k = int(rng.integers(1, 65)) if r < 0.25 else int(rng.integers(65, 1025)) if r < 0.75 else \
            int(rng.integers(1025, 5001))
        cases.append(dict(seed=9000 + c, batch=batch, m=dims[0], n=dims[1], k=k,
                          a_major=str(rng.choice(["row", "col"])), b_major=str(rng.choice(["row", "col"])),
                          c_major=str(rng.choice(["row", "row", "col"])), pad=int(rng.choice([0, 0, 1, 3])),
                          accumulate=bool(rng.random() < 0.5), alpha=float(rng.choice([1.0, -0.5, 0.75]))))
    return cases


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def err_ratio(p, got, ref):
    if p.k == 0:
        return 0.0 if np.array_equal(got, ref) else np.inf
    amax = float(np.abs(view(p.A.storage, p.batch, p.m, p.k, p.A.strides)).max())
    bmax = float(np.abs(view(p.B.storage, p.batch, p.k, p.n, p.B.strides)).max())
    diff = float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max())
    denom = p.k * amax * bmax
    return 0.0 if diff == 0.0 else diff / denom if denom else np.inf


def out(p, C):
    return np.array(view(C, p.batch, p.m, p.n, p.C.strides))


@pytest.mark.parametrize("part", range(4))
def test_random_products_on_the_planner_choice(part):
    cases = draw_cases()[part::4]
    s = torch.cuda.current_stream()
    for c in cases:
        p = wl.random_problem(c["seed"], c["batch"], c["m"], c["n"], c["k"], a_major=c["a_major"],
                              b_major=c["b_major"], c_major=c["c_major"], pad=c["pad"], dist="normal",
                              alpha=c["alpha"], accumulate=c["accumulate"])
        ref = p.C.storage.copy()
        oracle.ref_sgemm(*p.call_args(p.A.storage, p.B.storage, ref))
        plan = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
        split = sg.sgemm_splitk_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
        print(c, plan["kernel"], "split", split["splits"], split["parts"]["kernel"], flush=True)
        dA, dB = dev(p.A.storage), dev(p.B.storage)
        dC = dev(p.C.storage)
        sg.sgemm_strided_batched(*p.call_args(dA, dB, dC), stream=s)
        dC2 = dev(p.C.storage)
        W = torch.full((max(split["workspace_floats"], 1),), float("nan"), device="cuda")
        sg.sgemm_strided_batched_splitk(*p.call_args(dA, dB, dC2), W, split["workspace_floats"], stream=s)
        torch.cuda.synchronize()
        for name, got in (("plain", dC.cpu().numpy()), ("splitk", dC2.cpu().numpy())):
            e = err_ratio(p, out(p, got), out(p, ref))
            assert e <= TOL, (name, c, plan["kernel"], split["splits"], e)
            # Storage outside the logical outputs keeps its initial values.
            mask = np.ones(p.C.storage.size, bool)
            idx = np.arange(p.C.storage.size, dtype=np.int32)
            mask[np.array(view(idx, p.batch, p.m, p.n, p.C.strides)).ravel()] = False
            assert np.array_equal(got[mask], p.C.storage[mask]), (name, c)
