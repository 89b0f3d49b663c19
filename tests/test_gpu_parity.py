"""GPU parity: the HIP library against the CPU oracle on the same host bytes.

Every case goes through the C ABI (via the ctypes binding) and is compared
element by element with the oracle:
  * bitwise where the result is unique -- all-ones operands (C = k*alpha),
    and integer operands whose partial sums are all exact (brute force over
    every m, n, k in 1..8);
  * otherwise within the acceptance bound
        max |C_gpu - C_ref| / (k * max|A| * max|B|) <= 1e-6
    (maxima over all logical elements of the call).
Each kernel family (matrix-core tiles, one-wavefront tiles, generic) is
forced in turn, and every product workload runs at full size in the
configuration the benchmark times, compared with the oracle on every output
(the 4 x 4096^3 product: every 64 x 64 block of every batch entry, plus one
whole batch entry), with properties that hold at any size (determinism,
untouched gaps, no read of C without accumulation).

A missing GPU is a failure here, not a skip.
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
FAMILIES = [sg.PATH_AUTO, sg.PATH_MFMA, sg.PATH_WAVE, sg.PATH_GENERIC]
FAM_IDS = ["auto", "mfma", "wave", "generic"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "no GPU visible: GPU parity cannot pass without one"
    sg.load()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def gpu_call(p, path=sg.PATH_AUTO, C0=None, stream=None):
    """Run problem p through the C ABI; returns the whole C storage."""
    dA, dB = dev(p.A.storage), dev(p.B.storage)
    dC = dev(p.C.storage if C0 is None else C0)
    s = stream or torch.cuda.current_stream()
    sg.sgemm_strided_batched_path(*p.call_args(dA, dB, dC), path=path, stream=s)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def oracle_call(p, C0=None):
    C = (p.C.storage if C0 is None else C0).copy()
    oracle.ref_sgemm(*p.call_args(p.A.storage, p.B.storage, C))
    return C


def out(p, C):
    return np.array(view(C, p.batch, p.m, p.n, p.C.strides))


def err_ratio(p, got, ref):
    """max |got - ref| / (k * max|A| * max|B|) over the logical outputs."""
    if p.k == 0 or p.batch * p.m * p.n == 0:
        return 0.0 if np.array_equal(got, ref) else np.inf
    amax = np.abs(view(p.A.storage, p.batch, p.m, p.k, p.A.strides)).max()
    bmax = np.abs(view(p.B.storage, p.batch, p.k, p.n, p.B.strides)).max()
    denom = p.k * float(amax) * float(bmax)
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()
    if denom == 0.0:
        return 0.0 if diff == 0.0 else np.inf
    return diff / denom


# --------------------------------------------------------------- bitwise pins

@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_all_ones_bitwise(path):
    """A = B = 1 gives k*alpha (+ C_old) exactly, in every transpose case."""
    for a_major, b_major in LAYOUTS:
        for k in (1, 7, 64, 960, 4096):
            for alpha in (1.0, 0.5):
                for acc in (False, True):
                    p = wl.random_problem(k, 2, 37, 45, k, a_major=a_major, b_major=b_major,
                                          alpha=alpha, accumulate=acc, dist="ones")
                    got, ref = out(p, gpu_call(p, path)), out(p, oracle_call(p))
                    assert np.array_equal(got, ref), (a_major, b_major, k, alpha, acc)


def _packed_cases(a_major, b_major, batch, variant, sizes):
    """All (m, n, k) in sizes^3 packed into shared storages at 16-byte
    aligned offsets; integer data in [-3, 3]."""
    rng = np.random.default_rng([int(a_major == "row"), int(b_major == "row"), batch, variant])
    cases, offs = [], [0, 0, 0]
    for m in sizes:
        for n in sizes:
            for k in sizes:
                acc = (m + n + k + batch + variant) % 2 == 0
                alpha = 0.5 if (m * n * k + variant) % 2 else 1.0
                per_a, sa = wl.layout_strides(m, k, a_major)
                per_b, sb = wl.layout_strides(k, n, b_major)
                per_c, sc = wl.layout_strides(m, n, "row")
                cases.append((m, n, k, acc, alpha, sa, sb, sc, tuple(offs)))
                for i, per in enumerate((per_a, per_b, per_c)):
                    offs[i] += -(-per * batch // 4) * 4
    A = rng.integers(-3, 4, offs[0]).astype(np.float32)
    B = rng.integers(-3, 4, offs[1]).astype(np.float32)
    C = rng.integers(-3, 4, offs[2]).astype(np.float32)
    return cases, A, B, C


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_exact_bruteforce_bitwise(path):
    """Every m, n, k in 1..8, all four transpose cases, batch 1 and 3,
    accumulate on and off, alpha 1 and 0.5, integer data: the exact result
    is unique, so the GPU must match the oracle bit for bit."""
    sizes = range(1, 9)
    for a_major, b_major in LAYOUTS:
        for batch in (1, 3):
            for variant in (0, 1):
                cases, A, B, C = _packed_cases(a_major, b_major, batch, variant, sizes)
                dA, dB, dC = dev(A), dev(B), dev(C)
                ref = C.copy()
                s = torch.cuda.current_stream()
                for (m, n, k, acc, alpha, sa, sb, sc, (oa, ob, oc)) in cases:
                    sg.sgemm_strided_batched_path(
                        batch, m, n, k, alpha, dA.data_ptr() + 4 * oa, *sa,
                        dB.data_ptr() + 4 * ob, *sb, acc, dC.data_ptr() + 4 * oc, *sc,
                        path=path, stream=s)
                    oracle.ref_sgemm(batch, m, n, k, alpha, A[oa:], *sa, B[ob:], *sb, acc,
                                     ref[oc:], *sc)
                torch.cuda.synchronize()
                got = dC.cpu().numpy()
                if not np.array_equal(got, ref):
                    for (m, n, k, acc, alpha, sa, sb, sc, (oa, ob, oc)) in cases:
                        g = view(got[oc:], batch, m, n, sc)
                        r = view(ref[oc:], batch, m, n, sc)
                        assert np.array_equal(g, r), (a_major, b_major, batch, m, n, k, acc, alpha)


# ------------------------------------------------------------ tolerance cases

AWKWARD = [(17, 33, 9), (5, 129, 31), (1, 1, 1), (4, 4, 4), (5, 3, 9), (8, 16, 7),
           (33, 20, 65), (64, 1, 64), (1, 64, 1), (127, 129, 128), (129, 127, 257),
           (3, 514, 70), (200, 9, 300)]


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_awkward_shapes(path):
    """The pages' awkward sizes (StaleyNET "Testing the kernels": 17 x 33 x 9,
    5 x 129 x 31; kael ch. 09 "How it is tested": 1x1x1 ... 1x64x1, as rows
    x inner x columns) plus tile-boundary sizes, every transpose case, with
    padding between lines and accumulation."""
    for idx, (m, k, n) in enumerate(AWKWARD):
        for a_major, b_major in LAYOUTS:
            p = wl.random_problem(300 + idx, 2, m, n, k, a_major=a_major, b_major=b_major,
                                  alpha=0.75, accumulate=bool(idx % 2), pad=3)
            got, ref = out(p, gpu_call(p, path)), out(p, oracle_call(p))
            e = err_ratio(p, got, ref)
            assert e <= TOL, (m, n, k, a_major, b_major, e)


@pytest.mark.parametrize("mnk", [(128, 128, 32), (129, 127, 33), (255, 257, 96),
                                 (256, 128, 512), (384, 514, 200), (96, 640, 1000)])
@pytest.mark.parametrize("path", [sg.PATH_AUTO, sg.PATH_MFMA], ids=["auto", "mfma"])
def test_tile_boundaries(mnk, path):
    """Sizes at, just below and just above the matrix-core tile edges, with
    several tiles and a ragged tail, in all four transpose cases."""
    m, n, k = mnk
    for a_major, b_major in LAYOUTS:
        p = wl.random_problem(m * 7 + n, 3, m, n, k, a_major=a_major, b_major=b_major,
                              dist="normal", alpha=-0.5, accumulate=True)
        got, ref = out(p, gpu_call(p, path)), out(p, oracle_call(p))
        assert err_ratio(p, got, ref) <= TOL, (mnk, a_major, b_major)


TILE_NAMES = ["t128x128", "t128x64", "t64x128", "t64x64", "t256x128", "t128x160", "t128x80m16",
              "t64x176m16", "t64x64m16", "t128x128m16", "t128x64m16", "t64x128m16", "t64x32m16",
              "w32x32", "w32x64", "w64x32", "w64x64", "w16x32", "w16x64", "w32x16", "w64x16"]
# Most wavefronts per workgroup each wave tile's split variant allows.
WAVE_MAX_SPLIT = {"w32x32": 16, "w32x64": 8, "w64x32": 8, "w64x64": 8,
                  "w16x32": 16, "w16x64": 16, "w32x16": 16, "w64x16": 16}


@pytest.mark.parametrize("tile", TILE_NAMES)
def test_every_tile(tile, monkeypatch):
    """Each matrix-core tile configuration, forced, on ragged multi-tile
    shapes in all four transpose cases, with 16-byte loads (aligned shape)
    and element loads (padded lines), accumulating and not.  Wave tiles run
    unsplit here (one wavefront per tile); test_wave_split covers the split."""
    monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
    if tile.startswith("w"):
        monkeypatch.setenv("SGEMM_WAVE_SPLIT", "1")
    # k slices of 32: 3, 3, 2, 7, 2, 1 (the main loop never runs), 4 and 5.
    shapes = [(2, 300, 260, 96, 0), (2, 150, 190, 70, 3), (1, 33, 520, 40, 1), (3, 70, 100, 200, 0),
              (2, 64, 96, 64, 0), (2, 100, 90, 20, 0), (1, 70, 80, 128, 0), (1, 130, 140, 160, 2)]
    for batch, m, n, k, pad in shapes:
        for a_major, b_major in LAYOUTS:
            for acc in (False, True):
                p = wl.random_problem(m + n + k + pad, batch, m, n, k, a_major=a_major,
                                      b_major=b_major, dist="normal", alpha=0.625,
                                      accumulate=acc, pad=pad)
                info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
                assert tile in info["kernel"], info
                got, ref = out(p, gpu_call(p)), out(p, oracle_call(p))
                e = err_ratio(p, got, ref)
                assert e <= TOL, (tile, m, n, k, pad, a_major, b_major, acc, e)


@pytest.mark.parametrize("split", [2, 5, 16])
@pytest.mark.parametrize("tile", [t for t in TILE_NAMES if t.startswith("w")])
def test_wave_split(tile, split, monkeypatch):
    """Each wave tile with k split over several wavefronts of a workgroup
    (5 asks for 4; 16 is capped at the tile's limit), forced, on ragged
    shapes in all four transpose cases, 16-byte and element loads,
    accumulating and not.  k = 3 and 40 leave some wavefronts no k group at
    all; k = 1000 gives each several, with a ragged last group.  The same
    call twice gives the same bits (the partials are summed in a fixed
    order)."""
    monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
    monkeypatch.setenv("SGEMM_WAVE_SPLIT", str(split))
    want = min(1 << (split.bit_length() - 1), WAVE_MAX_SPLIT[tile])
    shapes = [(2, 70, 90, 3, 0), (1, 33, 50, 40, 1), (3, 50, 40, 1000, 0), (1, 1, 300, 777, 3),
              (2, 130, 2, 520, 0)]
    for batch, m, n, k, pad in shapes:
        for a_major, b_major in LAYOUTS:
            for acc in (False, True):
                p = wl.random_problem(m + 3 * n + k + pad + split, batch, m, n, k, a_major=a_major,
                                      b_major=b_major, dist="normal", alpha=-0.875, accumulate=acc,
                                      pad=pad)
                info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
                assert tile in info["kernel"] and info["waves"] == want, info
                assert info["kernel"].endswith(f"_s{want}"), info
                got = gpu_call(p)
                assert np.array_equal(got, gpu_call(p)), (tile, split, m, n, k)
                e = err_ratio(p, out(p, got), out(p, oracle_call(p)))
                assert e <= TOL, (tile, split, m, n, k, pad, a_major, b_major, acc, e)


@pytest.mark.parametrize("shape", [(1, 1, 4096, 4096, "row", "row"), (1, 4, 8192, 8192, "row", "col"),
                                   (1, 4096, 1, 4096, "row", "row"), (2, 3000, 8, 2000, "col", "row"),
                                   (1, 1, 1000, 16384, "col", "col")])
def test_skinny_products_split_k(shape):
    """Skinny products (one or a few rows or columns, long k) plan the
    wavefront kernel with k split over several wavefronts (planner's own
    choice) and match the oracle on every output."""
    batch, m, n, k, a_major, b_major = shape
    p = wl.random_problem(sum(shape[:4]), batch, m, n, k, a_major=a_major, b_major=b_major, dist="normal",
                          alpha=0.5, accumulate=True)
    info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
    assert info["kernel"].startswith("wave_") and info["waves"] > 1, info
    e = err_ratio(p, out(p, gpu_call(p)), out(p, oracle_call(p)))
    assert e <= TOL, (shape, info["kernel"], e)


@pytest.mark.parametrize("tile", [t for t in TILE_NAMES if t.startswith("t")])
def test_every_tile_8byte_loads(tile, monkeypatch):
    """Each LDS-tiled configuration, forced, with operands whose rows are
    8- but not 16-byte aligned (row strides 2 more than a multiple of 4, even
    extents): the fixed-offset loader reads them 8 bytes at a time, in all
    four transpose cases, with whole k slices and (when both operands run
    across k) a ragged last slice bounded by the buffer size."""
    monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
    shapes = [(2, 130, 146, 96), (1, 66, 210, 64), (3, 98, 70, 130), (2, 34, 514, 32)]
    widths = set()
    for batch, m, n, k in shapes:
        for a_major, b_major in LAYOUTS:
            for acc in (False, True):
                p = wl.random_problem(3 * m + n + k, batch, m, n, k, a_major=a_major, b_major=b_major,
                                      dist="normal", alpha=0.75, accumulate=acc, pad=2)
                info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
                assert tile in info["kernel"], info
                if info["fixed_offsets"]:
                    widths.update((info["vec_a"], info["vec_b"]))
                got, ref = out(p, gpu_call(p)), out(p, oracle_call(p))
                e = err_ratio(p, got, ref)
                assert e <= TOL, (tile, m, n, k, a_major, b_major, acc, info["vec_a"], info["vec_b"], e)
    assert 2 in widths, widths


@pytest.mark.parametrize("tile", ["p64x64k64", "p128x64k64", "p64x128k64"])
@pytest.mark.parametrize("wgs", [None, "8", "7", "1"])
def test_persistent_tile(tile, wgs, monkeypatch):
    """Each persistent short-k tile, forced, on ragged shapes with k <= 64
    in all four transpose cases, accumulating and not; a capped grid makes
    each workgroup loop over many tiles (odd and even counts)."""
    monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
    if wgs:
        monkeypatch.setenv("SGEMM_PERSIST_WGS", wgs)
    shapes = [(3, 300, 260, 64), (5, 132, 68, 40), (2, 64, 64, 4), (9, 128, 192, 60), (1, 4, 8, 12)]
    for batch, m, n, k in shapes:
        for a_major, b_major in LAYOUTS:
            for acc in (False, True):
                p = wl.random_problem(m * 7 + n + k, batch, m, n, k, a_major=a_major,
                                      b_major=b_major, dist="normal", alpha=-1.25,
                                      accumulate=acc)
                info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
                assert info["kernel"].startswith("persist_" + tile), info
                got, ref = out(p, gpu_call(p)), out(p, oracle_call(p))
                e = err_ratio(p, got, ref)
                assert e <= TOL, (tile, wgs, m, n, k, a_major, b_major, acc, e)


@pytest.mark.parametrize("tile", ["s64k64", "s128k64", "s128r2k64", "s64r2k64"])
def test_strip_tile(tile, monkeypatch):
    """Each short-k strip tile, forced, on ragged shapes with k in 4..64 and
    A, B both contiguous along k (the only layout it serves), accumulating
    and not; its k order is that of the other 16x16 kernels, so it must give
    the persistent kernel's bits."""
    shapes = [(3, 300, 260, 64), (5, 132, 68, 40), (2, 64, 64, 4), (9, 128, 192, 60), (1, 4, 8, 12),
              (2, 77, 1000, 64)]
    for batch, m, n, k in shapes:
        for acc in (False, True):
            p = wl.random_problem(m * 5 + n + k, batch, m, n, k, a_major="row", b_major="col",
                                  dist="normal", alpha=0.375, accumulate=acc)
            monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
            info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
            assert info["kernel"].startswith("strip_" + tile), info
            got = gpu_call(p)
            monkeypatch.setenv("SGEMM_FORCE_TILE", "p64x64k64")
            assert sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))["kernel"].startswith("persist_")
            assert np.array_equal(got, gpu_call(p)), (tile, batch, m, n, k, acc)
            e = err_ratio(p, out(p, got), out(p, oracle_call(p)))
            assert e <= TOL, (tile, m, n, k, acc, e)


def _denormal_problem(kind, seed, batch, m, n, k, a_major="row", b_major="row"):
    """Small integers scaled by powers of two, so every partial sum is exact
    and the result is unique: kind "in" makes A's entries denormal (2^-130
    scale), "out" keeps A and B normal but every product denormal (2^-70
    each), "c" multiplies zeros and adds a denormal C_old (accumulating)."""
    p = wl.random_problem(seed, batch, m, n, k, a_major=a_major, b_major=b_major, dist="int",
                          accumulate=kind == "c")
    if kind == "in":
        p.A.storage[:] = p.A.storage * np.float32(2.0 ** -130)
    elif kind == "out":
        p.A.storage[:] = p.A.storage * np.float32(2.0 ** -70)
        p.B.storage[:] = p.B.storage * np.float32(2.0 ** -70)
    else:
        p.A.storage[:] = 0.0
        p.C.storage[:] = (np.arange(p.C.storage.size) % 7 + 1).astype(np.float32) * np.float32(2.0 ** -135)
    return p


@pytest.mark.parametrize("kind", ["in", "out", "c"])
def test_denormals_are_kept(kind, monkeypatch):
    """Denormal inputs, denormal products and a denormal C_old come out of
    every kernel family (the matrix-core tiles, the short-k strip and
    persistent kernels, the direct wavefront and generic kernels) exactly
    as the oracle computes them: nothing is flushed to zero."""
    for fam in FAMILIES:
        p = _denormal_problem(kind, 91, 2, 96, 80, 40)
        got, ref = out(p, gpu_call(p, fam)), out(p, oracle_call(p))
        assert np.count_nonzero(ref) > 0
        assert np.array_equal(got, ref), (kind, fam)
    for tile in ("s64k64", "p64x64k64"):
        monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
        p = _denormal_problem(kind, 92, 2, 96, 80, 40, a_major="row", b_major="col")
        assert tile in sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))["kernel"]
        assert np.array_equal(out(p, gpu_call(p)), out(p, oracle_call(p))), (kind, tile)


def test_column_major_output():
    """C stored column-major is served as C^T = B^T A^T."""
    for a_major, b_major in LAYOUTS:
        p = wl.random_problem(41, 2, 150, 90, 77, a_major=a_major, b_major=b_major,
                              c_major="col", accumulate=True, alpha=1.5)
        got, ref = out(p, gpu_call(p)), out(p, oracle_call(p))
        assert err_ratio(p, got, ref) <= TOL, (a_major, b_major)


def test_broadcast_batch_stride_zero():
    p = wl.random_problem(42, 5, 70, 130, 96, b_broadcast=True, dist="normal")
    got, ref = out(p, gpu_call(p)), out(p, oracle_call(p))
    assert err_ratio(p, got, ref) <= TOL


def test_general_strides_and_misalignment():
    """Neither stride of A is 1, and B starts one float past 16-byte
    alignment: the loaders fall back to element and 4-byte loads."""
    rng = np.random.default_rng(43)
    m, n, k, batch = 70, 90, 50, 2
    A = rng.uniform(-1, 1, batch * m * k * 2).astype(np.float32)
    B = rng.uniform(-1, 1, batch * k * n + 1).astype(np.float32)
    sa, sb, sc = (m * k * 2, 2 * k, 2), (k * n, n, 1), (m * n, n, 1)
    dA, dB = dev(A), dev(B)
    dC = torch.zeros(batch * m * n, device="cuda")
    info = sg.sgemm_plan_describe(batch, m, n, k, 1.0, dA.data_ptr(), *sa, dB.data_ptr() + 4, *sb,
                                  0, dC.data_ptr(), *sc)
    assert info["path_name"] in ("mfma", "wave") and info["vec_a"] == 1 and info["vec_b"] == 1
    sg.sgemm_strided_batched(batch, m, n, k, 1.0, dA.data_ptr(), *sa, dB.data_ptr() + 4, *sb,
                             0, dC.data_ptr(), *sc, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = np.zeros(batch * m * n, np.float32)
    oracle.ref_sgemm(batch, m, n, k, 1.0, A, *sa, B[1:], *sb, 0, ref, *sc)
    p = wl.Problem("strided", batch, m, n, k, 1.0, False, wl.Operand(A, sa), wl.Operand(B[1:], sb),
                   wl.Operand(ref, sc))
    assert err_ratio(p, dC.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_k_zero_and_empty(path):
    for acc in (False, True):
        p = wl.random_problem(44, 2, 33, 17, 0, accumulate=acc, alpha=3.0)
        got, ref = out(p, gpu_call(p, path)), out(p, oracle_call(p))
        assert np.array_equal(got, ref), acc
    p = wl.random_problem(45, 0, 33, 17, 5)
    gpu_call(p, path)


@pytest.mark.parametrize("path", FAMILIES, ids=FAM_IDS)
def test_canaries_nan_and_gaps(path):
    """With accumulate = 0, a NaN-filled C is never read; the gaps between C's
    rows and matrices keep their NaN sentinel; a NaN in A[0, 2, 1] poisons row
    2 of batch 0 only."""
    p = wl.random_problem(46, 2, 45, 70, 40, pad=5, dist="normal")
    C0 = np.full_like(p.C.storage, np.nan)
    got = gpu_call(p, path, C0=C0)
    ref = oracle_call(p, C0=C0)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert not np.isnan(out(p, got)).any()
    assert err_ratio(p, out(p, got), out(p, ref)) <= TOL
    A = p.A.storage.copy()
    sa = p.A.strides
    A[2 * sa[1] + 1 * sa[2]] = np.nan
    q = wl.Problem("nan", p.batch, p.m, p.n, p.k, 1.0, False, wl.Operand(A, sa), p.B, p.C)
    g = out(q, gpu_call(q, path))
    mask = np.zeros(g.shape, bool)
    mask[0, 2, :] = True
    assert np.array_equal(np.isnan(g), mask)


def test_offsets_beyond_32_bits():
    """Operands whose rows or batch entries lie more than 2 GiB apart.  Rows
    that far apart exceed a workgroup's 32-bit buffer window, so the planner
    takes the 64-bit generic kernel; batch entries that far apart only move
    each workgroup's 64-bit base, so the matrix-core kernel still serves.
    Both match the oracle run on compact copies of the same logical values."""
    far = (1 << 29) + 128                      # floats: 2 GiB + 512 bytes
    rng = np.random.default_rng(77)
    for (batch, m, n, k, where, family) in ((1, 5, 40, 70, "A rows", "generic"),
                                            (2, 33, 20, 16, "C batch", "mfma")):
        A = rng.standard_normal((batch, m, k)).astype(np.float32)
        B = rng.standard_normal((batch, k, n)).astype(np.float32)
        if where == "A rows":
            sa = (0, far, 1)
            dA = torch.zeros((m - 1) * far + k, device="cuda")
            dA.as_strided((m, k), (far, 1)).copy_(torch.from_numpy(A[0]))
            sc = (m * n, n, 1)
            dC = torch.zeros(batch * m * n, device="cuda")
        else:
            sa = (m * k, k, 1)
            dA = torch.from_numpy(A.ravel()).cuda()
            sc = (far, n, 1)
            dC = torch.zeros(far + m * n, device="cuda")
        dB = torch.from_numpy(B.ravel()).cuda()
        sb = (k * n, n, 1)
        args = [batch, m, n, k, 1.5, dA, *sa, dB, *sb, 0, dC, *sc]
        info = sg.sgemm_plan_describe(*[a.data_ptr() if isinstance(a, torch.Tensor) else a for a in args])
        assert info["kernel"].startswith(family), info
        sg.sgemm_strided_batched(*args, stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        got = dC.as_strided((batch, m, n), sc).cpu().numpy()
        ref = np.zeros(batch * m * n, np.float32)
        oracle.ref_sgemm(batch, m, n, k, 1.5, A.ravel(), m * k, k, 1, B.ravel(), k * n, n, 1, 0,
                         ref, m * n, n, 1)
        scale = k * np.abs(A).max() * np.abs(B).max()
        e = np.abs(got.astype(np.float64) - ref.reshape(batch, m, n)).max() / scale
        assert e <= TOL, (where, e)
        del dA, dB, dC
        torch.cuda.empty_cache()


def test_k1_with_huge_k_stride():
    """k = 1 with a k stride of 2^30 floats on A, B or both (irrelevant for a
    single k row, and past what the fixed-offset loader's 32-bit buffer size
    can hold): every family gives the oracle's result, bit for bit (alpha 1:
    each output is one product, rounded once on both sides)."""
    rng = np.random.default_rng(1301)
    m, n = 130, 70
    A = rng.standard_normal(m).astype(np.float32)
    B = rng.standard_normal(n).astype(np.float32)
    huge = 1 << 30
    for sA, sB in (((0, 1, huge), (0, huge, 1)), ((0, 1, huge), (0, n, 1)), ((0, 1, m), (0, huge, 1))):
        for path in FAMILIES:
            dA, dB = dev(A), dev(B)
            dC = torch.zeros(m * n, device="cuda")
            sg.sgemm_strided_batched_path(1, m, n, 1, 1.0, dA, *sA, dB, *sB, 0, dC, 0, n, 1,
                                          path=path, stream=torch.cuda.current_stream())
            torch.cuda.synchronize()
            got = dC.cpu().numpy()
            ref = np.zeros(m * n, np.float32)
            oracle.ref_sgemm(1, m, n, 1, 1.0, A, *sA, B, *sB, 0, ref, 0, n, 1)
            assert np.array_equal(got, ref), (sA, sB, path, float(np.abs(got - ref).max()))


def test_determinism_repeated_calls():
    p = wl.random_problem(47, 4, 300, 260, 500, a_major="col", b_major="col", dist="normal")
    first = gpu_call(p)
    for _ in range(3):
        assert np.array_equal(first, gpu_call(p))


def test_torch_wrapper_and_side_stream():
    """sgemm() on torch views: W.t() passes exchanged strides, a 2-D operand
    broadcasts over the batch, and work runs on a caller-chosen stream."""
    g = torch.Generator().manual_seed(48)
    x = torch.randn(3, 100, 64, generator=g)
    W = torch.randn(80, 64, generator=g)
    y = torch.zeros(3, 100, 80)
    xd, Wd, yd = x.cuda(), W.cuda(), y.cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sg.sgemm(xd, Wd.t(), yd, alpha=2.0)
    s.synchronize()
    ref = np.zeros(3 * 100 * 80, np.float32)
    oracle.ref_sgemm(3, 100, 80, 64, 2.0, x.numpy().ravel(), 6400, 64, 1,
                     W.numpy().ravel(), 0, 1, 64, 0, ref, 8000, 80, 1)
    denom = 64 * float(x.abs().max()) * float(W.abs().max())
    assert np.abs(yd.cpu().numpy().ravel() - ref).max() / denom <= TOL


# --------------------------------------------------- full-size workloads

# The largest product (4 x 4096^3, 5.5e11 FLOP) is the one workload whose
# whole output the oracle cannot recompute in test time; every other product
# workload is compared on every output.
STRATIFIED = "square4096_acc"
CELL = 64          # stratification cell: every 64 x 64 block of every batch entry
PER_CELL = 8       # its 4 corners plus 4 random outputs


def _stratified_indices(p, rng):
    """At least PER_CELL outputs of every CELL x CELL block of every batch
    entry (its four corners and PER_CELL - 4 random ones), so no output tile
    of any kernel tile size (all are multiples of 16 and at most 256 wide)
    goes unchecked."""
    idx = []
    for b in range(p.batch):
        for i0 in range(0, p.m, CELL):
            i1 = min(p.m, i0 + CELL) - 1
            for j0 in range(0, p.n, CELL):
                j1 = min(p.n, j0 + CELL) - 1
                cell = [(b, i0, j0), (b, i0, j1), (b, i1, j0), (b, i1, j1)]
                ri = rng.integers(i0, i1 + 1, PER_CELL - 4)
                rj = rng.integers(j0, j1 + 1, PER_CELL - 4)
                cell += [(b, int(x), int(y)) for x, y in zip(ri, rj)]
                idx.extend(cell)
    return np.array(idx, dtype=np.int64)


@pytest.mark.parametrize("name", [w for w in wl.WORKLOADS if wl.kind(w) == "plain"])
def test_workload_full_size(name):
    """Each workload at its full size, in the launch configuration the
    benchmark times (planner's choice, torch's current stream), against the
    oracle: every output, except for the 4 x 4096^3 product, where every
    64 x 64 block of every batch entry is checked at its corners and 4 random
    points and the last batch entry is checked whole (StaleyNET "GPU
    Implementation", section "Testing the kernels": each kernel's output is
    compared with a plain CPU computation).  Two calls give the same bits."""
    p = wl.workload(name)
    info = sg.sgemm_plan_describe(*p.call_args(1 << 40, 1 << 41, 1 << 42))
    assert info["path_name"] in ("mfma", "wave"), info
    dA, dB = dev(p.A.storage), dev(p.B.storage)
    dC = dev(p.C.storage)
    s = torch.cuda.current_stream()
    sg.sgemm_strided_batched(*p.call_args(dA, dB, dC), stream=s)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    print(f"[full-size] {name}: kernel {info['kernel']}, {p.batch} x {p.m}x{p.n}x{p.k}", flush=True)
    if name != STRATIFIED:
        ref = oracle_call(p)
        e = err_ratio(p, out(p, got), out(p, ref))
        assert e <= TOL, (name, e)
    else:
        idx = _stratified_indices(p, np.random.default_rng(49))
        assert len(idx) == p.batch * -(-p.m // CELL) * -(-p.n // CELL) * PER_CELL
        refv = oracle.ref_entries(*p.call_args(p.A.storage, p.B.storage, p.C.storage), idx=idx)
        gv = view(got, p.batch, p.m, p.n, p.C.strides)[idx[:, 0], idx[:, 1], idx[:, 2]]
        e = err_ratio(p, gv, refv)
        assert e <= TOL, (name, "stratified", e)
        # The last batch entry, whole: the same call restricted to it.
        b = p.batch - 1
        (sAb, sAr, sAc), (sBb, sBr, sBc), (sCb, sCr, sCc) = p.A.strides, p.B.strides, p.C.strides
        ref_b = p.C.storage[b * sCb:].copy()
        oracle.ref_sgemm(1, p.m, p.n, p.k, p.alpha, p.A.storage[b * sAb:], 0, sAr, sAc,
                         p.B.storage[b * sBb:], 0, sBr, sBc, int(p.accumulate), ref_b, 0, sCr, sCc)
        got_b = view(got[b * sCb:], 1, p.m, p.n, (0, sCr, sCc))
        want_b = view(ref_b, 1, p.m, p.n, (0, sCr, sCc))
        e = err_ratio(p, got_b, want_b)
        assert e <= TOL, (name, "batch entry", b, e)
    dC2 = dev(p.C.storage)
    sg.sgemm_strided_batched(*p.call_args(dA, dB, dC2), stream=s)
    torch.cuda.synchronize()
    assert torch.equal(dC, dC2)
