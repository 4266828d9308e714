"""Host-side checks of the benchmark harness: the one-GPU contract, the
roofline arithmetic, operand-set sizing, per-launch percentiles, and that
every workload's committed rocprofv3 summary is the one of the kernel the
automatic plan picks for it (file name and machine-readable line)."""
import os
import subprocess
import sys

import pytest

import bench
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_roofline_fractions():
    r = bench._roofline("mfma", 1250.0, 2500.0, "TFLOP/s", 123, probe_peak=1000.0)
    assert r == {"bound": "mfma", "achieved": 1250.0, "peak": 2500.0, "unit": "TFLOP/s", "frac": 0.5,
                 "traffic": 123, "probe_peak": 1000.0, "frac_of_probe": 1.25}
    assert "probe_peak" not in bench._roofline("hbm", 4000.0, 8000.0, "GB/s", None)


def test_operand_sets_exceed_the_last_level_cache():
    # rotated operand sets together exceed twice the 256 MB cache (within the cap)
    for w in inputs.WORKLOAD_LIST:
        n = bench._n_sets(w, 3)
        assert 3 <= n <= 64
        assert n * w.compulsory_bytes() >= (512 << 20) or n == 64


def test_percentiles():
    p = bench._percentiles([float(i) for i in range(1, 101)])
    assert p["n"] == 100
    assert p["p10_ms"] <= p["median_ms"] <= p["p90_ms"]
    assert abs(p["median_ms"] - 50.5) <= 0.5


@pytest.fixture(scope="module")
def lib():
    return gb.load_library()


@pytest.mark.parametrize("w", inputs.WORKLOAD_LIST, ids=lambda w: w.name)
def test_profile_summary_matches_the_planned_kernel(lib, w):
    h = gb.gemm_epi_plan(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
    try:
        kern, _, name = gb.gemm_epi_plan_describe(h)
    finally:
        gb.gemm_epi_destroy(h)
    path = os.path.join(ROOT, "profiles", f"{name}__{w.name}.txt")
    assert os.path.exists(path), path
    text = open(path).read()
    assert "command: rocprofv3 --kernel-trace --stats" in text
    assert "command: rocprofv3 --pmc FETCH_SIZE" in text and "command: rocprofv3 --pmc WRITE_SIZE" in text
    line = [l for l in text.splitlines() if l.startswith("machine-readable:")]
    assert len(line) == 1
    kv = dict(t.split("=", 1) for t in line[0].split()[1:])
    assert kv["kernel"] == name and kv["workload"] == w.name
    # traffic at least the compulsory bytes (the counters see every byte once at least)
    assert int(kv["traffic_bytes"]) >= 0.95 * w.compulsory_bytes()
