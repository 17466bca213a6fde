"""Host-side pieces of the benchmark that run without a GPU: the percentile
summary and the HIP device attributes it reads the memory clock and bus width
with, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench


def test_stats_percentiles():
    s = bench.stats(np.arange(1, 101, dtype=np.float64))
    assert s["n"] == 100 and s["mean"] == 50.5 and s["p50"] == 50.5
    assert s["p10"] == pytest.approx(np.percentile(np.arange(1, 101), 10))
    assert s["p90"] == pytest.approx(np.percentile(np.arange(1, 101), 90))
    assert bench.stats([7.0])["p10"] == 7.0


def test_device_attribute_numbers_match_the_installed_header():
    """device_peak_gbps asks hipDeviceGetAttribute for attributes 59 and 60;
    the installed HIP header must give those numbers to the memory bus width
    and the memory clock rate."""
    header = "/opt/rocm/include/hip/hip_runtime_api.h"
    if not os.path.exists(header):
        pytest.skip("no HIP headers")
    src = ("#include <hip/hip_runtime_api.h>\n#include <stdio.h>\n"
           "int main(void) { printf(\"%d %d\", (int)hipDeviceAttributeMemoryBusWidth,"
           " (int)hipDeviceAttributeMemoryClockRate); return 0; }\n")
    exe = os.path.join("/tmp", f"lrkv_attr_{os.getpid()}")
    r = subprocess.run(["gcc", "-x", "c", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-", "-o", exe],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    try:
        out = subprocess.run([exe], capture_output=True, text=True).stdout.split()
    finally:
        os.remove(exe)
    assert out == ["59", "60"]


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_with(tmp_path, monkeypatch):
    """measured_traffic returns the profile's bytes per launch while the
    attention kernel's sources hash to the recorded value, and None once any
    of them changes."""
    import json
    import shutil
    csrc = tmp_path / "decode_attention_lrkv_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(bench.ROOT, "decode_attention_lrkv_amd", "csrc", name), csrc / name)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"mean_bytes_per_launch": 12345, "kernel_src_sha256": bench.kernel_sources_sha256()}
    (tmp_path / "profiles" / "split_bf16_kernel_llama8b-b16-32k.txt").write_text(
        "# summary\n\n    TRAFFIC " + json.dumps(rec) + "\n")
    assert bench.measured_traffic() == 12345
    with open(csrc / bench.KERNEL_SOURCES[-1], "a") as f:
        f.write("\n// changed\n")
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    """The decode path runs on one GPU: any other --gpus exits with status 2
    and a message, before torch or the library is imported."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", str(n)], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout and f"--gpus {n}" in r.stdout
