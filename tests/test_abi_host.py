"""Host-side checks of the C ABI: symbols, validation and planning.

These run without a GPU: the library is loaded, every symbol the header
declares must be exported, every invalid-argument path must return its
status before any HIP call, and sgemm_plan_describe (given a CU count) never
touches a device.
"""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import strided_fp32_gemm_amd as sg
from strided_fp32_gemm_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "strided_fp32_gemm_amd", "csrc")
HEADER = os.path.join(ROOT, "include", "sgemm_strided.h")

# Fake, suitably aligned device addresses: the planner reads alignment only.
PA, PB, PC = 0x7F0000000000, 0x7F1000000000, 0x7F2000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sgemm_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = sg.load()
    names = declared_functions()
    assert names == sorted(sg.EXPORTS)
    for name in names:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr), name


def test_status_strings():
    for code, name in sg._binding.STATUS.items():
        assert sg.sgemm_status_string(code).startswith(name)
    assert sg.sgemm_status_string(12345) == "unknown sgemm status"


def plan(batch, m, n, k, sa, sb, sc, acc=0, path=0, ptrs=(PA, PB, PC), alpha=1.0):
    return sg.sgemm_plan_describe(batch, m, n, k, alpha, ptrs[0], *sa, ptrs[1], *sb, acc,
                                  ptrs[2], *sc, path=path, num_cus=256)


def status_of(fn):
    with pytest.raises(sg.SgemmError) as e:
        fn()
    return e.value.status


def test_validation_errors_never_reach_the_device():
    rm = lambda r, c: (r * c, c, 1)  # noqa: E731
    # negative sizes
    assert status_of(lambda: sg.sgemm_strided_batched(1, -1, 4, 4, 1.0, PA, *rm(4, 4), PB, *rm(4, 4),
                                                     0, PC, *rm(4, 4))) == -1
    # negative stride
    assert status_of(lambda: sg.sgemm_strided_batched(1, 4, 4, 4, 1.0, PA, 16, -4, 1, PB, *rm(4, 4),
                                                     0, PC, *rm(4, 4))) == -2
    # null C with work; null A with k > 0
    assert status_of(lambda: sg.sgemm_strided_batched(1, 4, 4, 4, 1.0, PA, *rm(4, 4), PB, *rm(4, 4),
                                                     0, 0, *rm(4, 4))) == -3
    assert status_of(lambda: sg.sgemm_strided_batched(1, 4, 4, 4, 1.0, 0, *rm(4, 4), PB, *rm(4, 4),
                                                     0, PC, *rm(4, 4))) == -3
    # C rows overlap each other (row stride smaller than the row length)
    assert status_of(lambda: sg.sgemm_strided_batched(1, 4, 4, 4, 1.0, PA, *rm(4, 4), PB, *rm(4, 4),
                                                     0, PC, 16, 3, 1)) == -4
    # batch stride 0 on C with batch > 1
    assert status_of(lambda: sg.sgemm_strided_batched(2, 4, 4, 4, 1.0, PA, *rm(4, 4), PB, *rm(4, 4),
                                                     0, PC, 0, 4, 1)) == -4
    # C overlaps A
    assert status_of(lambda: sg.sgemm_strided_batched(1, 4, 4, 4, 1.0, PA, *rm(4, 4), PB, *rm(4, 4),
                                                     0, PA + 8, *rm(4, 4))) == -4
    # extent * stride overflows int64
    assert status_of(lambda: sg.sgemm_strided_batched(1, 4, 4, 4, 1.0, PA, *rm(4, 4), PB, *rm(4, 4),
                                                     0, PC, 0, 1 << 62, 1)) == -5
    # unknown path
    assert status_of(lambda: sg.sgemm_strided_batched_path(1, 4, 4, 4, 1.0, PA, *rm(4, 4), PB,
                                                          *rm(4, 4), 0, PC, *rm(4, 4), path=9)) == -7
    assert "negative stride sA_row" in sg.sgemm_last_error() or sg.sgemm_last_error()


def test_empty_products_are_accepted_without_a_device():
    # batch, m or n == 0: OK, nothing enqueued, pointers may be NULL.
    sg.sgemm_strided_batched(0, 4, 4, 4, 1.0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    sg.sgemm_strided_batched(3, 0, 4, 4, 1.0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    sg.sgemm_strided_batched(3, 4, 0, 4, 1.0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    p = plan(3, 4, 0, 4, (0, 0, 0), (0, 0, 0), (0, 0, 0), ptrs=(0, 0, 0))
    assert p["launches"] == 0 and p["workgroups"] == 0


def test_k_zero_needs_no_operands():
    p = plan(2, 5, 7, 0, (0, 0, 0), (0, 0, 0), (35, 7, 1), ptrs=(0, 0, PC))
    assert p["launches"] == 1


def _cfg_plan(name):
    prob = wl.workload(name) if name != "square4096_acc" else None
    if prob is None:
        s2 = 4096 * 4096
        return plan(4, 4096, 4096, 4096, (s2, 1, 4096), (s2, 4096, 1), (s2, 4096, 1), acc=1, alpha=0.5)
    return plan(prob.batch, prob.m, prob.n, prob.k, prob.A.strides, prob.B.strides, prob.C.strides,
                acc=int(prob.accumulate), alpha=prob.alpha)


@pytest.mark.parametrize("name,path,a_kfast,b_kfast,vec_b", [
    ("square64", "mfma", 1, 0, 4),
    ("linear_xWt", "mfma", 1, 1, 4),
    ("attn_qk", "mfma", 1, 1, 4),
    ("attn_pv", "mfma", 1, 0, 4),
    ("spectrogram", "mfma", 1, 0, 2),
    ("square4096_acc", "mfma", 0, 0, 4),
])
def test_workload_plans(name, path, a_kfast, b_kfast, vec_b):
    """Each workload reaches the matrix-core family with the loader its
    layout calls for (the four transpose cases map to k-fast or m/n-fast
    loaders; the spectrogram basis rows of 514 floats are 8-byte aligned and
    read 8 bytes at a time)."""
    p = _cfg_plan(name)
    assert p["path_name"] == path, p
    assert (p["a_kfast"], p["b_kfast"], p["vec_b"]) == (a_kfast, b_kfast, vec_b), p
    assert p["vec_a"] == 4
    assert p["transposed"] == 0


def test_column_major_output_is_solved_transposed():
    # C stored column-major (row stride 1): computed as C^T = B^T A^T.
    p = plan(1, 3000, 2000, 640, (0, 640, 1), (0, 2000, 1), (0, 1, 3000))
    assert p["transposed"] == 1 and p["path_name"] == "mfma"


def test_offsets_beyond_32_bits_use_the_generic_path():
    huge = 1 << 27  # row stride of 2^27 floats: even 16 rows span > 2^31 bytes
    p = plan(1, 256, 256, 64, (0, huge, 1), (0, 256, 1), (0, 256, 1))
    assert p["path_name"] == "generic"
    forced = plan(1, 256, 256, 64, (0, huge, 1), (0, 256, 1), (0, 256, 1), path=sg.PATH_MFMA)
    assert forced["path_name"] == "generic"


def test_forced_families():
    args = (1, 100, 90, 70, (0, 70, 1), (0, 90, 1), (0, 90, 1))
    assert plan(*args, path=sg.PATH_WAVE)["path_name"] == "wave"
    assert plan(*args, path=sg.PATH_MFMA)["path_name"] == "mfma"
    assert plan(*args, path=sg.PATH_GENERIC)["path_name"] == "generic"


def test_vector_width_follows_alignment():
    # Misaligned base pointer (4 bytes past 16-byte alignment) forces scalar loads.
    p = plan(1, 128, 128, 128, (0, 128, 1), (0, 128, 1), (0, 128, 1), ptrs=(PA + 4, PB, PC))
    assert p["vec_a"] == 1 and p["vec_b"] == 4
    # Fast extent and row stride even but not multiples of 4: 8-byte loads
    # (LDS-tiled kernel with fixed offsets only), odd: element loads.
    p = plan(1, 128, 130, 128, (0, 128, 1), (0, 130, 1), (0, 130, 1))
    assert p["vec_b"] == 2 and p["fixed_offsets"] == 1
    p = plan(1, 128, 130, 128, (0, 128, 1), (0, 130, 1), (0, 130, 1), path=sg.PATH_WAVE)
    assert p["vec_b"] == 1
    p = plan(1, 128, 131, 128, (0, 128, 1), (0, 131, 1), (0, 131, 1))
    assert p["vec_b"] == 1
    # A misaligned by 8 bytes: 8-byte loads of A.
    p = plan(1, 128, 128, 128, (0, 128, 1), (0, 128, 1), (0, 128, 1), ptrs=(PA + 8, PB, PC))
    assert p["vec_a"] == 2
    # Neither stride 1: element loads along the smaller stride.
    p = plan(1, 64, 64, 64, (0, 128, 2), (0, 64, 1), (0, 64, 1))
    assert p["vec_a"] == 1


def test_tile_map_example_shape_is_planned():
    """kael ch. 09 "Matmul" worked example: rows 5, inner 3, columns 9 is a
    single clipped tile for every family here."""
    from helpers import load_golden
    g = load_golden("kael_tile_map.txt")
    rows, inner, cols = int(g["rows"]), int(g["inner"]), int(g["columns"])
    for path in (sg.PATH_WAVE, sg.PATH_MFMA, sg.PATH_GENERIC):
        p = plan(1, rows, cols, inner, (0, inner, 1), (0, cols, 1), (0, cols, 1), path=path)
        assert p["workgroups"] == 1


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
@pytest.mark.parametrize("batches", [1, 3])
def test_tile_order_on_the_worked_example(tmp_path, batches):
    """The library's own tile-order code (plan.hpp's tile_coords, compiled
    with g++) driven over the 4 x 4 decomposition of kael ch. 09 "Matmul"'s
    worked example (rows 5, columns 9): 2 x 3 tiles per batch entry, each
    output covered exactly once, and the page's tile 4 (first row (4 / 3) * 4,
    first column (4 % 3) * 4) clipped to out[4][4..7].  The library visits the
    tiles in its own order (grouped tile rows, column by column), so the
    page's tile number is located by its (tile row, tile column); with 6
    tiles per launch the XCD remap is off (6 is not a multiple of 8), and
    with 3 batch entries (18 tiles) it is off too."""
    from helpers import load_golden
    g = load_golden("kael_tile_map.txt")
    rows, cols, edge = int(g["rows"]), int(g["columns"]), 4
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, os.path.join(HERE, "plan_check.cpp"), "-o",
                    str(exe)], check=True)
    r = subprocess.run([str(exe), "tiles", str(batches), str(rows), str(cols), str(edge)],
                       capture_output=True, text=True, check=True, timeout=60)
    lines = [tuple(int(t) for t in ln.split()) for ln in r.stdout.split("\n") if ln.strip()]
    assert len(lines) == batches * int(g["tiles"])
    assert [ln[0] for ln in lines] == list(range(len(lines)))
    assert max(ln[2] for ln in lines) + 1 == int(g["tile_rows"])
    assert max(ln[3] for ln in lines) + 1 == int(g["tile_columns"])
    cover = np.zeros((batches, rows, cols), np.int64)
    for _, b, tm, tn, r0, rc, c0, cc in lines:
        assert (r0, c0) == (tm * edge, tn * edge)
        cover[b, r0:r0 + rc, c0:c0 + cc] += 1
    assert (cover == 1).all()
    tile = int(g["tile"])
    want = (tile // int(g["tile_columns"]), tile % int(g["tile_columns"]))
    for b in range(batches):
        (hit,) = [ln for ln in lines if ln[1] == b and (ln[2], ln[3]) == want]
        assert hit[4:] == (int(g["tile4_first_row"]), int(g["tile4_row_count"]),
                           int(g["tile4_first_column"]), int(g["tile4_column_count"]))


def test_short_k_kernels_serve_short_k_only(monkeypatch):
    """The attention-score shape (k = 64, A and B contiguous along k) goes to
    the strip kernel, 128 rows per workgroup across all 512 columns; with B
    contiguous along n the persistent kernel takes it (one workgroup per
    LDS-resident pair of slabs on each CU).  Neither is used where it cannot
    serve: k above 64, element loads, or C rows without 16-byte stores."""
    qk = _cfg_plan("attn_qk")
    assert qk["kernel"] == "strip_s128k64_ak_bk", qk
    assert qk["tile_m"] == 128 and qk["tile_k"] == 64 and qk["workgroups"] == 120 * 4
    bn = plan(120, 512, 512, 64, (512 * 64, 64, 1), (512 * 64, 512, 1), (512 * 512, 512, 1))
    assert bn["kernel"].startswith("persist_p64x64k64"), bn
    assert bn["workgroups"] == 2 * 256
    for tile in ("s64k64", "s128k64"):
        monkeypatch.setenv("SGEMM_FORCE_TILE", tile)
        assert not plan(120, 512, 512, 64, (512 * 64, 64, 1), (512 * 64, 512, 1),
                        (512 * 512, 512, 1))["kernel"].startswith("strip_")     # B n-fast
        assert not plan(120, 512, 512, 68, (512 * 68, 68, 1), (512 * 68, 1, 68),
                        (512 * 512, 512, 1))["kernel"].startswith("strip_")     # k above 64
        assert not plan(120, 512, 510, 64, (512 * 64, 64, 1), (510 * 64, 1, 64),
                        (512 * 510, 510, 1))["kernel"].startswith("strip_")     # C rows not 16-byte
    monkeypatch.setenv("SGEMM_FORCE_TILE", "p64x64k64")
    ok = plan(120, 512, 512, 64, (512 * 64, 64, 1), (512 * 64, 1, 64), (512 * 512, 512, 1))
    assert ok["kernel"].startswith("persist_"), ok
    deep = plan(120, 512, 512, 68, (512 * 68, 68, 1), (512 * 68, 1, 68), (512 * 512, 512, 1))
    assert not deep["kernel"].startswith("persist_"), deep
    ragged = plan(120, 512, 512, 62, (512 * 62, 62, 1), (512 * 62, 1, 62), (512 * 512, 512, 1))
    assert not ragged["kernel"].startswith("persist_"), ragged
    odd_c = plan(120, 512, 510, 64, (512 * 64, 64, 1), (510 * 64, 1, 64), (512 * 510, 510, 1))
    assert not odd_c["kernel"].startswith("persist_"), odd_c
    # A grid cap (for sweeps and tests) bounds the workgroups, never above the tiles.
    monkeypatch.setenv("SGEMM_PERSIST_WGS", "7")
    assert plan(120, 512, 512, 64, (512 * 64, 64, 1), (512 * 64, 1, 64), (512 * 512, 512, 1))["workgroups"] == 7
    monkeypatch.setenv("SGEMM_PERSIST_WGS", "100000")
    assert plan(1, 64, 128, 64, (0, 64, 1), (0, 1, 64), (0, 128, 1))["workgroups"] == 2


def test_extended_entry_points_validate_before_the_device():
    """The general epilogue, the squared norms and the distance table reject
    bad arguments with a status before any device call (no GPU here)."""
    ex = lambda **kw: sg.sgemm_strided_batched_ex(
        kw.get("batch", 1), 8, 8, 4, 1.0, PA, 0, 4, 1, PB, 0, 8, 1, kw.get("beta", 0.0),
        PC, 0, 8, 1, kw.get("row"), *kw.get("sR", (0, 1)), kw.get("col"), *kw.get("sL", (0, 1)))
    assert status_of(lambda: ex(row=PA + (1 << 20), sR=(0, -1))) == -2
    assert status_of(lambda: ex(col=PC + 4, sL=(0, 1))) == -4          # column term inside C
    assert status_of(lambda: ex(row=PC - 16, sR=(0, 1))) == -4         # row term reaching into C
    assert status_of(lambda: ex(col=PA, sL=(1 << 62, 1), batch=4)) == -5
    sq = lambda *a: sg.sgemm_sqnorms(*a)
    assert status_of(lambda: sq(1, 4, -1, PA, 0, 4, 1, PC, 0, 1)) == -1
    assert status_of(lambda: sq(1, 4, 4, PA, 0, -4, 1, PC, 0, 1)) == -2
    assert status_of(lambda: sq(1, 4, 4, None, 0, 4, 1, PC, 0, 1)) == -3
    assert status_of(lambda: sq(2, 4, 4, PA, 16, 4, 1, PC, 2, 1)) == -4   # outputs collide
    assert status_of(lambda: sq(1, 4, 4, PA, 0, 4, 1, PA + 8, 0, 1)) == -4  # out inside X
    sg.sgemm_sqnorms(0, 4, 4, None, 0, 4, 1, None, 0, 1)                # empty: nothing to do
    dist = lambda ws, floats: sg.sgemm_pairwise_sqdist(2, 8, 8, 4, PA, 32, 4, 1, PB, 0, 4, 1,
                                                       PC, 64, 8, 1, ws, floats)
    assert status_of(lambda: dist(None, 100)) == -8
    assert status_of(lambda: dist(PA + (1 << 24), 2 * 8 + 8 - 1)) == -8  # needs batch*m + 1*n
    assert status_of(lambda: dist(PC + 4, 24)) == -4                      # workspace inside D
    assert sg.sgemm_status_string(-8).startswith("SGEMM_ERR_WORKSPACE")



def test_splitkv_chunk_count_is_the_cheapest_by_exhaustive_search(monkeypatch):
    """The planner visits only the distinct chunk counts (jumping over block
    counts that give the same number of chunks); an exhaustive search over
    every count 1..blocks with the same rule (the busiest CU's workgroups
    times the blocks of the longest chunk, plus 0.1 per chunk; the cheapest
    count giving each of the 256 CUs a workgroup, else the cheapest overall;
    ties to the most chunks, as the planner meets them first) must agree on
    random decode shapes (1 to 64 rows per group, so 1 to 4 row tiles), with
    and without a workspace cap."""
    monkeypatch.delenv("SGEMM_ATTN_CHUNKS", raising=False)
    rng = np.random.default_rng(404)
    cus, item = 256, 16 * 64 + 32
    for _ in range(60):
        no, hk, g = int(rng.integers(1, 65)), int(rng.integers(1, 9)), int(rng.integers(1, 9))
        tq = int(rng.integers(1, 64 // g + 1))
        tk = int(rng.choice([int(rng.integers(tq, 600)), int(rng.integers(600, 70000))]))
        h = hk * g
        tiles = -(-(g * tq) // 16)                  # 16-row tiles per (outer, KV head)
        groups, blocks = no * hk * tiles, -(-tk // 32)
        cap = blocks
        ws = -1
        if rng.random() < 0.3:
            ws = int(rng.integers(groups * item, groups * item * (blocks + 1)))
            cap = min(cap, ws // (groups * item))
        best = {}
        for n in sorted({-(-blocks // b) for b in range(1, blocks + 1)}, reverse=True):
            if n > cap:
                continue
            per = -(-blocks // n)
            wgs = -(-(groups * n) // 4)
            cost = -(-wgs // cus) * 4.0 * per + 0.1 * n
            for key, ok in (("fill", wgs >= cus), ("any", True)):
                if ok and (key not in best or cost < best[key][0]):
                    best[key] = (cost, n)
        want = (best.get("fill") or best["any"])[1]
        keys = -(-(-(-tk // want)) // 32) * 32
        want = -(-tk // keys)
        sQ, sK = (tq * h * 64, 64, h * 64, 1), (tk * hk * 64, 64, hk * 64, 1)
        got = sg.sgemm_attention_splitkv_describe(no, h, tq, tk, 64, 0.125, 1, PA, *sQ, PB, sK[0], sK[1], g, sK[2],
                                                  sK[3], PB + (1 << 35), *sK, PC, *sQ, workspace_floats=ws)
        assert (got["chunks"], got["chunk_keys"]) == (want, keys), (no, hk, g, tq, tk, ws, got, want, keys)
        assert got["workspace_floats"] == groups * want * item and (want - 1) * keys < tk <= want * keys


def test_splitkv_attention_validates_and_plans_before_the_device(monkeypatch):
    """Split-KV attention checks the attention arguments and its workspace
    (size >= 0, NULL only when empty, no overlap with Q, K, V or O) before
    any device call, and plans without a device: a decode step (one query,
    g = 3 query heads per KV head, 4096 keys, 8 x 5 groups) takes 43 chunks of
    96 keys, 1056 floats of workspace per chunk; 20 rows per group (g = 5,
    tq = 4) take two 16-row tiles, so twice the partials per chunk; a
    prefill, g * tq above 64, a head dimension other than 64 and a workspace
    below one chunk per group and tile are not split; SGEMM_ATTN_CHUNKS fixes
    the count.  Other chunk counts
    worked by hand from the planner's rule (the busiest CU's workgroups times
    their blocks, plus 0.1 per chunk, over the counts that give each of the
    256 CUs a workgroup): 16384 keys over 40 groups take 74 chunks of 224
    keys (740 workgroups, 3 on the busiest CU: 84 + 7.4, where 128 chunks
    cost 80 + 12.8); 32 x 4 groups over 4096 keys take 8 of 512 (64 + 0.8);
    2 groups over 8192 keys fill no CU count and take the cheapest overall,
    86 chunks of 96 keys (12 + 8.6, against 8 + 12.8 for 128 chunks)."""
    def args(no=8, h=15, tq=1, tk=4096, d=64, g=3, V=PB + (1 << 26), O=PC):
        hk = -(-h // g)
        sQ, sK = (tq * h * d, d, h * d, 1), (tk * hk * d, d, hk * d, 1)
        return [no, h, tq, tk, d, 0.125, 1, PA, *sQ, PB, sK[0], sK[1], g, sK[2], sK[3], V, *sK, O, *sQ]
    d = lambda ws=-1, **kw: sg.sgemm_attention_splitkv_describe(*args(**kw), workspace_floats=ws)
    assert d() == {"chunks": 43, "chunk_keys": 96, "workspace_floats": 43 * 40 * 1056}
    assert d(tq=512, tk=512)["chunks"] == 0                                   # prefill
    two = d(g=5, tq=4)                                                        # 20 rows: 2 tiles
    assert two["workspace_floats"] == two["chunks"] * 8 * 3 * 2 * 1056, two
    assert d(g=5, tq=13)["chunks"] == 0 and d(g=5, tq=12)["chunks"] > 0     # 65 rows, 60 rows
    assert d(d=32)["chunks"] == 0
    assert d(ws=40 * 1056 - 1)["chunks"] == 0 and d(ws=3 * 40 * 1056)["chunks"] == 3
    assert (d(tk=16384)["chunks"], d(tk=16384)["chunk_keys"]) == (74, 224)
    assert (d(no=32, h=32, g=8)["chunks"], d(no=32, h=32, g=8)["chunk_keys"]) == (8, 512)
    assert (d(no=1, h=8, g=4, tk=8192)["chunks"], d(no=1, h=8, g=4, tk=8192)["chunk_keys"]) == (86, 96)
    monkeypatch.setenv("SGEMM_ATTN_CHUNKS", "7")
    assert d()["chunks"] == 7
    run = lambda ws, floats: sg.sgemm_attention_splitkv(*args(), ws, floats)
    assert status_of(lambda: run(None, -1)) == -1
    assert status_of(lambda: run(None, 10)) == -3
    assert status_of(lambda: run(PB + 64, 1 << 12)) == -4      # inside K
    assert status_of(lambda: run(PC - 16, 1 << 12)) == -4      # reaching into O


def test_splitk_validates_and_plans_before_the_device(monkeypatch):
    """The split-k entry point checks the product's arguments and its
    workspace (size >= 0, NULL only when empty, no overlap with A, B or C)
    before any device call, and its describe call plans without a device:
    deep contractions into small outputs are split (1 x 128 x 128 x 65536
    into 64 partitions of 1024, 64x64 tiles, the reduction as the second
    launch), large outputs and short k are not, a shorter last partition
    adds a launch, and a workspace cap gives the largest split that fits
    (the partials take splits * batch * m * n floats)."""
    run = lambda ws, floats, **kw: sg.sgemm_strided_batched_splitk(
        1, 64, 64, kw.get("k", 4096), 1.0, PA, 0, 4096, 1, PB, 0, 64, 1, 0, PC, 0, 64, 1, ws, floats)
    assert status_of(lambda: run(None, -1)) == -1
    assert status_of(lambda: run(None, 100)) == -3
    assert status_of(lambda: run(PA + 64, 1 << 16)) == -4      # workspace inside A
    assert status_of(lambda: run(PB - 64, 1 << 16)) == -4      # reaching into B
    assert status_of(lambda: run(PC, 4096)) == -4              # on C
    assert status_of(lambda: run(PA + (1 << 30), 100, k=-1)) == -1
    sg.sgemm_strided_batched_splitk(0, 64, 64, 64, 1.0, None, 0, 64, 1, None, 0, 64, 1, 0, None, 0, 64, 1,
                                    None, 0)                      # empty: nothing to do

    def d(batch, m, n, k, ws=-1, acc=0):
        return sg.sgemm_splitk_describe(batch, m, n, k, 1.0, PA, m * k, k, 1, PB, k * n, 1, k, acc,
                                        PC, m * n, n, 1, workspace=(1 << 44) if ws >= 0 else None,
                                        workspace_floats=ws)
    deep = d(1, 128, 128, 65536)
    assert (deep["splits"], deep["kc"], deep["k_last"], deep["launches"]) == (64, 1024, 1024, 2), deep
    assert deep["workspace_floats"] == 64 * 128 * 128
    assert deep["parts"]["kernel"].startswith("mfma_t64x64m16_"), deep
    assert deep["parts"]["workgroups"] == 64 * 4
    for big in (d(4, 4096, 4096, 4096), d(1, 256, 256, 200)):
        assert big["splits"] == 1 and big["launches"] == 1 and big["workspace_floats"] == 0, big
    ragged = d(1, 128, 128, 65536 - 100)
    assert ragged["splits"] > 1 and ragged["k_last"] < ragged["kc"] and ragged["launches"] == 3, ragged
    capped = d(1, 128, 128, 65536, ws=5 * 128 * 128)
    assert capped["splits"] == 4 and capped["workspace_floats"] == 4 * 128 * 128, capped
    assert d(1, 128, 128, 65536, ws=0)["splits"] == 1
    monkeypatch.setenv("SGEMM_SPLITK", "3")
    forced = d(2, 70, 96, 1000)
    assert (forced["splits"], forced["kc"], forced["k_last"], forced["launches"]) == (3, 384, 232, 3), forced
    monkeypatch.setenv("SGEMM_SPLITK", "1")
    assert d(1, 128, 128, 65536)["splits"] == 1


def test_two_level_batch_validates_before_the_device():
    """Two batch levels with groups: sizes, groups, strides, C's distinctness
    across both levels and overlap with the inputs are checked before any
    device call (no GPU here)."""
    def b2(no=2, ni=4, gA=1, gB=2, sA=(256, 64, 8, 1), sB=(128, 64, 1, 8), sC=(512, 128, 16, 1),
           A=PA, B=PB, C=PC):
        return sg.sgemm_strided_batched2(no, ni, 8, 16, 8, 1.0, A, sA[0], sA[1], gA, sA[2], sA[3],
                                         B, sB[0], sB[1], gB, sB[2], sB[3], 0,
                                         C, sC[0], sC[1], sC[2], sC[3])
    assert status_of(lambda: b2(ni=0)) == -1
    assert status_of(lambda: b2(gA=0)) == -1
    assert status_of(lambda: b2(no=-1)) == -1
    assert status_of(lambda: b2(sB=(128, -64, 1, 8))) == -2
    assert status_of(lambda: b2(sC=(512, 0, 16, 1))) == -4          # every head writes one block
    assert status_of(lambda: b2(sC=(256, 128, 16, 1))) == -4        # sequences overlap heads
    assert status_of(lambda: b2(C=PA + 4 * 100)) == -4              # C inside A
    assert status_of(lambda: b2(no=1 << 40, ni=1 << 30)) == -5      # batch overflows int64
    assert status_of(lambda: b2(sA=(1 << 61, 64, 8, 1), no=8)) == -5
    b2(no=0)                                                        # empty: nothing to do
    # Groups larger than the inner count are accepted (every entry maps to the first).
    b2(no=0, gB=1 << 40)


def test_attention_validates_and_plans_before_the_device():
    """Fused attention rejects bad sizes, strides, pointers, aliasing and
    paths with a status before any device call, and plans the matrix-core
    kernel only for d = 64 with unit column strides and aligned rows."""
    def args(no=2, h=6, tq=32, tk=32, d=64, causal=0, g=3, sQ=None, sK=None, sO=None,
             Q=PA, K=PB, V=PB + (1 << 24), O=PC):
        sQ = sQ or (tq * h * d, d, h * d, 1)
        sK = sK or (tk * 2 * d, d, 2 * d, 1)
        sO = sO or sQ
        return [no, h, tq, tk, d, 0.125, causal, Q, *sQ, K, sK[0], sK[1], g, sK[2], sK[3],
                V, *sK, O, *sO]

    def run(**kw):
        path = kw.pop("path", 0)
        return sg.sgemm_attention_path(*args(**kw), path=path)

    def plan(**kw):
        path = kw.pop("path", 0)
        return sg.sgemm_attention_describe(*args(**kw), path=path)

    assert status_of(lambda: run(h=0)) == -1
    assert status_of(lambda: run(g=0)) == -1
    assert status_of(lambda: run(tk=0)) == -1                       # a query with no key
    assert status_of(lambda: run(tq=40, tk=32, causal=1)) == -1     # causal, first queries see nothing
    assert status_of(lambda: run(d=300, sQ=(0, 300, 300, 1), sK=(0, 300, 300, 1))) == -5
    assert status_of(lambda: run(sK=(0, 64, -128, 1))) == -2
    assert status_of(lambda: run(Q=None)) == -3
    assert status_of(lambda: run(O=PA + 4 * 64)) == -4              # O inside Q
    assert status_of(lambda: run(sO=(0, 64, 384, 1))) == -4         # sequences collide in O
    assert status_of(lambda: run(path=2)) == -7                     # no wavefront family here
    assert status_of(lambda: run(d=32, sQ=(32 * 192, 32, 192, 1), sK=(32 * 64, 32, 64, 1), path=1)) == -5
    run(no=0)                                                        # nothing to do
    run(tq=0, tk=0)
    assert plan()["kernel"] == "attn_mfma_d64_w8"
    assert plan(causal=1)["kernel"] == "attn_mfma_d64_w8_causal"
    assert plan()["workgroups"] == 2 * 6 * 1
    assert plan(path=3)["kernel"] == "attn_generic"
    assert plan(d=32, sQ=(32 * 192, 32, 192, 1), sK=(32 * 64, 32, 64, 1))["kernel"] == "attn_generic"
    assert plan(sQ=(32 * 6 * 66, 66, 6 * 66, 1))["kernel"] == "attn_generic"     # rows 8-byte aligned only
    assert plan(Q=PA + 8)["kernel"] == "attn_generic"
    assert plan(sK=(32 * 2 * 128, 128, 256, 2))["kernel"] == "attn_generic"     # column stride 2


@pytest.mark.parametrize("name,tile", [("linear_bwd_dw", "t64x32m16"), ("linear_bwd_dx", "t64x128m16"),
                                       ("attn_pv", "t64x64m16"), ("square4096_acc", "t128x128m16"),
                                       ("spectrogram", "t64x64m16"), ("linear_xWt", "t128x160"),
                                       ("linear_bias", "t128x160")])
def test_measured_tile_choices(name, tile):
    """The planner's cost model keeps the tile choices that measured fastest
    on MI355X when every tile was forced in turn (with the fixed-offset and
    8-byte loaders): dW (600 tiles of 64x64 on 256 CUs) on the 64x32 tile's
    1200 workgroups, dX on 64x128, P.V and the spectrogram on 64x64, the
    linear layer and its bias-fused form on 128x160, and the 4 x 4096^3
    product on 128x128 (no GPU: planning runs on the host).  The x^T-layout
    linear layer measured 64x64 and 128x160 within 0.3% of each other, so
    either is accepted there."""
    p = _cfg_plan(name) if name != "linear_bias" else _bias_plan()
    assert p["path_name"] == "mfma" and tile in p["kernel"], p


def test_skinny_products_split_k_over_wavefronts(monkeypatch):
    """Products with too few tiles to occupy the SIMDs unsplit and a long k
    plan the wavefront kernel with k split over several wavefronts of a
    workgroup (measured on MI355X: 1 x 4096 x 4096 from 100 us unsplit on
    32 x 32 tiles to 18 us on 16 x 32 tiles split 8 ways); 16-wide tiles
    compete on any shape (4096 x 1 x 4096 on 16 x 32 split 8: 15.7 us
    against 20.0 on 32 x 16; 24 x 4096 x 4096 on 16 x 32: 21.2 against 27.6
    on 32 x 32); products with enough tiles, or too short a k, stay
    unsplit.  SGEMM_WAVE_SPLIT forces a split (rounded
    down to a power of two, capped by the tile), and the describe call
    reports the wavefronts per workgroup."""
    gemv = plan(1, 1, 4096, 4096, (0, 4096, 1), (0, 4096, 1), (0, 4096, 1))
    assert gemv["kernel"] == "wave_w16x32_ak_bn_s8" and gemv["waves"] == 8, gemv
    assert gemv["tile_m"] == 16 and gemv["tile_n"] == 32 and gemv["workgroups"] == 128
    tall = plan(1, 4096, 1, 4096, (0, 4096, 1), (0, 1, 1), (0, 1, 1))
    assert tall["kernel"] == "wave_w16x32_ak_bk_s8", tall
    few = plan(1, 1, 1000, 16384, (0, 16384, 1), (0, 1, 16384), (0, 1000, 1))
    assert few["waves"] == 8 and few["workgroups"] == 32, few
    # Enough tiles to give every SIMD a wavefront: no split.
    wide = plan(64, 1, 4096, 512, (512, 512, 1), (512 * 4096, 4096, 1), (4096, 4096, 1))
    assert not re.search(r"_s\d+$", wide["kernel"]), wide
    # k of 64 is four 16-deep groups: too short to split.
    short = plan(1, 1, 4096, 64, (0, 64, 1), (0, 4096, 1), (0, 4096, 1))
    assert not re.search(r"_s\d+$", short["kernel"]), short
    # 16-wide tiles beyond 16 rows where they measured faster.
    p = plan(1, 24, 4096, 4096, (0, 4096, 1), (0, 4096, 1), (0, 4096, 1))
    assert p["kernel"] == "wave_w16x32_ak_bn_s8", p
    # Forced splits.
    monkeypatch.setenv("SGEMM_FORCE_TILE", "w32x64")
    monkeypatch.setenv("SGEMM_WAVE_SPLIT", "16")
    p = plan(2, 70, 96, 300, (70 * 300, 300, 1), (300 * 96, 96, 1), (70 * 96, 96, 1))
    assert p["kernel"] == "wave_w32x64_ak_bn_s8" and p["waves"] == 8, p          # capped at 8
    monkeypatch.setenv("SGEMM_FORCE_TILE", "w16x32")
    monkeypatch.setenv("SGEMM_WAVE_SPLIT", "5")
    p = plan(2, 70, 96, 3, (70 * 3, 3, 1), (3 * 96, 96, 1), (70 * 96, 96, 1))
    assert p["kernel"] == "wave_w16x32_ak_bn_s4" and p["waves"] == 4, p          # rounded down; k of 3
    monkeypatch.setenv("SGEMM_WAVE_SPLIT", "1")
    assert plan(1, 1, 4096, 4096, (0, 4096, 1), (0, 4096, 1), (0, 4096, 1))["waves"] == 1


def test_accepted_regret_on_the_xT_linear_layer():
    p = _cfg_plan("linear_xT")
    assert p["kernel"].startswith(("mfma_t64x64m16_", "mfma_t128x160_")), p


def _bias_plan():
    prob = wl.workload("linear_bias")
    return sg.sgemm_plan_describe(prob.batch, prob.m, prob.n, prob.k, prob.alpha, PA, *prob.A.strides, PB,
                                  *prob.B.strides, 0, PC, *prob.C.strides, num_cus=256)


def test_noalloc_distance_checks_before_the_device():
    """The allocation-free distance entry point validates exactly like the
    workspace one and refuses a call whose norms exceed its fixed scratch,
    both before any HIP call (this host has no GPU); its capacity is the
    header's SGEMM_SCRATCH_FLOATS."""
    text = open(HEADER).read()
    (cap,) = re.findall(r"#define\s+SGEMM_SCRATCH_FLOATS\s+\(1 << (\d+)\)", text)
    assert sg.SCRATCH_FLOATS == 1 << int(cap)
    f = sg.sgemm_pairwise_sqdist_noalloc
    assert status_of(lambda: f(1, -1, 4, 4, PA, 16, 4, 1, PB, 16, 4, 1, PC, 16, 4, 1)) == -1
    assert status_of(lambda: f(1, 4, 4, 4, PA, 16, -4, 1, PB, 16, 4, 1, PC, 16, 4, 1)) == -2
    assert status_of(lambda: f(1, 4, 4, 4, 0, 16, 4, 1, PB, 16, 4, 1, PC, 16, 4, 1)) == -3
    m = sg.SCRATCH_FLOATS      # batch*m + n exceeds the scratch by n
    with pytest.raises(sg.SgemmError) as e:
        f(1, m, 8, 4, PA, m * 4, 4, 1, PB, 0, 4, 1, PC, m * 8, 8, 1)
    assert e.value.status == -8 and "fixed device scratch" in str(e.value)
    # Empty calls return OK without touching anything.
    f(0, 4, 4, 4, PA, 16, 4, 1, PB, 16, 4, 1, PC, 16, 4, 1)


def test_fixed_offsets_where_the_buffer_size_bounds_k():
    """The LDS-tiled kernel keeps its load offsets for the whole k loop when
    the buffer resource alone can bound k: every benchmark product does; a
    k-fast operand with a partial last slice, or a k-slow one whose rows
    overlap, takes the per-slice loader."""
    for name in ("linear_xWt", "attn_pv", "spectrogram", "square4096_acc", "linear_bwd_dx", "linear_bwd_dw",
                 "linear_xT"):
        p = _cfg_plan(name)
        assert p["fixed_offsets"] == 1 and p["kernel"].startswith("mfma_"), (name, p)
    mfma = sg.PATH_MFMA
    # k-fast A and B, k = 100 (not a multiple of the 32-deep slice): per slice.
    assert plan(2, 128, 128, 100, (128 * 100, 100, 1), (128 * 100, 1, 100), (128 * 128, 128, 1),
                path=mfma)["fixed_offsets"] == 0
    # k-slow A and B with the same ragged k: the buffer size bounds the rows.
    assert plan(2, 128, 128, 100, (128 * 100, 1, 128), (128 * 100, 128, 1), (128 * 128, 128, 1),
                path=mfma)["fixed_offsets"] == 1
    # k-slow B whose rows overlap (row stride 64 < 128 columns): per slice.
    assert plan(1, 128, 128, 96, (0, 96, 1), (0, 64, 1), (0, 128, 1), path=mfma)["fixed_offsets"] == 0
    # k = 1 with a k stride whose one-slice size would pass 2 GiB (the stride of
    # an extent-1 axis is otherwise irrelevant): per slice.
    assert plan(1, 128, 128, 1, (0, 1, 1 << 30), (0, 128, 1), (0, 128, 1), path=mfma)["fixed_offsets"] == 0
    # Other kernel families never use it.
    assert plan(1, 100, 90, 70, (0, 70, 1), (0, 90, 1), (0, 90, 1), path=sg.PATH_WAVE)["fixed_offsets"] == 0


def test_torch_attention_helper_checks_its_arguments():
    """sg.attention refuses non-tensors and tensors off the GPU before any
    device call."""
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 3, 64)
    with pytest.raises(TypeError):
        sg.attention(x.numpy(), x, x, x)
    with pytest.raises(ValueError, match="on the GPU"):
        sg.attention(x, x, x, x)
