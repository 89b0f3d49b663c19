"""bench.py's command-line contract on a host without a GPU: it measures one
GPU only (any other count, by flag or by WORLD_SIZE, exits 2 with a message),
rejects meaningless step counts, and without a visible GPU fails with a
message instead of printing a number."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(args, **env):
    e = dict(os.environ)
    e.update(env)
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300, env=e,
                          cwd=ROOT)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = run(args, **env)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("args", [["--steps", "0"], ["--warmup", "-1"]])
def test_bad_step_counts_are_refused(args):
    r = run(args)
    assert r.returncode == 2 and r.stdout == "", (r.returncode, r.stderr)


def test_no_gpu_is_an_error_not_a_number():
    r = run(["--steps", "1"], HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    assert r.returncode != 0 and r.stdout == "", (r.returncode, r.stdout)


def test_traffic_record_hash_covers_every_built_source():
    """The counter record bench.py reports as `roofline.traffic` is only
    trusted while the hash of the library's sources matches the one it was
    taken on; that hash must cover every file the build compiles and every
    header those files include (directly or not), and the public header."""
    import re
    sys.path.insert(0, ROOT)
    import bench
    from strided_fp32_gemm_amd import build
    hashed = set(bench.kernel_sources())
    csrc = os.path.join("strided_fp32_gemm_amd", "csrc")
    todo = [os.path.join(csrc, f) for f in build.SOURCES]
    seen = set()
    while todo:
        rel = todo.pop()
        if rel in seen:
            continue
        seen.add(rel)
        assert rel in hashed, rel
        text = open(os.path.join(ROOT, rel)).read()
        for inc in re.findall(r'#include\s+"([^"]+)"', text):
            local = os.path.join(csrc, inc)
            todo.append(local if os.path.exists(os.path.join(ROOT, local)) else os.path.join("include", inc))
    assert os.path.join("include", "sgemm_strided.h") in seen
    before = bench.kernel_sources_sha256()
    assert before == bench.kernel_sources_sha256() and len(before) == 64


def test_roofline_bound_follows_arithmetic_intensity():
    """A workload at or above the machine balance (157.3 TFLOP/s over
    8 TB/s, ~19.7 flops per byte) is held to the matrix-core peak in
    TFLOP/s; one below it (the skinny product: 2 flops per byte) to the HBM
    peak in GB/s, with achieved = algorithmic bytes over the launch time."""
    sys.path.insert(0, ROOT)
    import bench
    from strided_fp32_gemm_amd import workloads as wl

    sq = wl.workload("square64")
    big = bench._roofline_bound(2.0 * 4 * 4096 ** 3, 4 * 4 * 4 * 4096 ** 2, 3.6)
    assert big["bound"] == "mfma" and big["unit"] == "TFLOP/s" and big["peak"] == 157.3
    assert abs(big["achieved"] - 2.0 * 4 * 4096 ** 3 / 3.6e-3 / 1e12) < 1e-3
    flops, nbytes = 2.0 * 4 * 16384 * 4096, 4 * (4 * 4096 + 16384 * 4096 + 4 * 16384)
    thin = bench._roofline_bound(flops, nbytes, 0.05)
    assert thin["bound"] == "hbm" and thin["unit"] == "GB/s" and thin["peak"] == 8000.0
    assert abs(thin["achieved"] - nbytes / 0.05e-3 / 1e9) < 0.1
    assert abs(thin["frac"] - thin["achieved"] / 8000.0) < 1e-4
    assert bench._roofline_bound(float(sq.flops), wl.algorithmic_bytes(sq), 0.006)["bound"] == "hbm"
