"""The benchmark's command-line contract, checked without a GPU.

bench.py measures one GPU: asked for more it must exit with a message before
it touches torch or the device.  Its counter-traffic figures are tied to the
kernel sources they were measured on, and must read as missing once those
sources change.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    res = subprocess.run([sys.executable, BENCH, "--gpus", str(n)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""  # no JSON line


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    res = subprocess.run([sys.executable, BENCH], capture_output=True, text=True,
                         timeout=120, env=env)
    assert res.returncode == 2 and res.stdout == ""


def test_help_lists_the_modes_and_the_zero_operand_check():
    res = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 0
    for flag in ("--steps", "--warmup", "--mode", "--operand-data",
                 "--fast-baseline", "--lora-rank", "--copy-calibration"):
        assert flag in res.stdout, flag


def test_counter_traffic_is_void_for_other_sources(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    sha = bench.COUNTER_TRAFFIC["sources_sha256"]
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: sha)
    assert bench.counter_traffic("bwd_dw_gemm") > 0
    assert bench.counter_traffic("bwd_dw_gemm", workload="tiny") is None
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.counter_traffic("bwd_dw_gemm") is None


def test_counter_mfma_is_void_for_other_sources(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    sha = bench.COUNTER_TRAFFIC["sources_sha256"]
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: sha)
    c = bench.counter_mfma("bwd_dw_gemm")
    assert 0 < c["mfma_busy"] < 1 and 1.0 < c["clock_ghz"] < 2.5
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.counter_mfma("bwd_dw_gemm") is None

