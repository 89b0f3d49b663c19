"""Register budget of the compiled kernels (hipcc cross-compiles gfx950 device
code on the CPU; no GPU): no kernel instantiation spills registers to scratch
memory, and the 128 x 128 tile with 16-wide blocks keeps two wavefronts per
SIMD on its 16-byte-load layouts (two workgroups per CU, the occupancy its
schedule is built for).  A register cap on a tile whose accumulators do not
fit it shows up here as scratch, long before a timing does."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from strided_fp32_gemm_amd import build as b

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")

# Every HIP source but scratch.hip, which holds only the allocation-free entry
# point's device array.
KERNEL_SOURCES = [s for s in b.SOURCES if s.endswith(".hip") and s != "scratch.hip"]


def kernel_stats(asm: str):
    """(kernel symbol, scratch bytes, occupancy) for every kernel in one
    device assembly file, from the compiler's per-function summary."""
    out, name = [], None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            scratch = occ = None
            continue
        m = re.match(r"^\s*; ScratchSize: (\d+)", line)
        if m and name:
            scratch = int(m.group(1))
        m = re.match(r"^\s*; Occupancy: (\d+)", line)
        if m and name:
            occ = int(m.group(1))
            out.append((name, scratch, occ))
            name = None
    return out


@pytest.fixture(scope="module")
def stats(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("asm")

    def one(src):
        path = tmp / (src + ".s")
        r = subprocess.run([b._hipcc(), "-x", "hip", *b.common_flags(), "--cuda-device-only", "-S",
                            os.path.join(b.CSRC, src), "-o", str(path)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, kernel_stats(path.read_text())

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(one, KERNEL_SOURCES))


def test_every_source_has_kernels(stats):
    for src, ks in stats.items():
        assert ks, f"no kernel summary found in {src}"


def test_no_kernel_spills(stats):
    spills = [(src, name, s) for src, ks in stats.items() for name, s, _ in ks if s]
    assert not spills, spills


def test_square_tile_keeps_two_wavefronts_per_simd(stats):
    # sgemm_mfma<9, AK, BKF, AW = 4, BW = 4, FX>: tile 9 is t128x128m16;
    # both the per-slice and the fixed-offset loaders.
    vec4 = [(n, occ) for n, _, occ in stats["mfma_t9.hip"] if re.search(r"ELi4ELi4ELb[01]EEEvNS_8MfmaArgsE$", n)]
    assert len(vec4) == 8, vec4
    assert all(occ >= 2 for _, occ in vec4), vec4


def _wave_table():
    """kWaveTiles of the planner header: {bm, bn, waves_per_simd, name, rate, max_split}."""
    text = open(os.path.join(b.CSRC, "plan.hpp")).read()
    body = text[text.index("kWaveTiles[kNumWaveTiles] = {"):]
    body = body[:body.index("};")]
    rows = re.findall(r'\{(\d+), (\d+), (\d+), "(\w+)", ([\d.]+), (\d+)\}', body)
    return [(int(bm), int(bn), int(w), name, int(s)) for bm, bn, w, name, _, s in rows]


def test_wave_tile_table_matches_the_compiled_code(stats):
    """The planner's wavefront tiles state the occupancy their compiled
    code has: the unsplit kernel's resident wavefronts per SIMD (the least
    over its 16 layout instances) is the table's waves_per_simd, and the
    split kernel fits a workgroup of max_split wavefronts on one CU
    (max_split / 4 per SIMD)."""
    table = _wave_table()
    assert len(table) == 8, table
    for w, (bm, bn, wps, name, max_split) in enumerate(table):
        plain, split = [], []
        for n, _, occ in stats[f"wave_w{w}.hip"]:
            m = re.search(r"sgemm_waveILi(\d+)E(?:Lb[01]E){4}Lb([01])EEEv", n)
            if m and int(m.group(1)) == w:
                (split if m.group(2) == "1" else plain).append(occ)
        assert len(plain) == 16 and len(split) == 16, (name, len(plain), len(split))
        assert min(plain) == wps, (name, min(plain), wps)
        assert 4 * min(split) >= max_split, (name, min(split), max_split)
