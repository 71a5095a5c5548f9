"""Host-side checks of bench.py (no GPU): the single-GPU refusal and the rule that a
committed counter record is reported only while the GEMM's sources still match it."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(root):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.ROOT = str(root)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr


@pytest.fixture
def tree(tmp_path):
    """A stand-in repository: two kernel sources and a traffic and a counter record keyed
    to their SHA-256 (concatenated in the listed order)."""
    csrc = tmp_path / "parity_gate_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemm.hip").write_bytes(b"kernel source\n")
    (csrc / "common.h").write_bytes(b"shared header\n")
    sha = hashlib.sha256(b"kernel source\n" + b"shared header\n").hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gemm1_wl_traffic.json").write_text(json.dumps(
        {"kernel_sources": ["gemm.hip", "common.h"], "sources_sha256": sha,
         "fetch_bytes": 3.0e9, "write_bytes": 1.0e9}))
    (prof / "mfma_wl_counters.json").write_text(json.dumps(
        {"kernel_sources": ["gemm.hip", "common.h"], "sources_sha256": sha,
         "kernels": {"moe::grouped_gemm_x<0>": {"mfma_busy": 0.5, "clock_ghz": 2.0, "ops": 1.0e12},
                     "moe::other_kernel": {"mfma_busy": 0.1, "clock_ghz": 2.0, "ops": 1.0}}}))
    return tmp_path


def test_records_reported_while_sources_match(tree):
    b = _bench(tree)
    assert b.measured_traffic("wl") == 4.0e9
    c = b.measured_mfma("wl")
    assert list(c) == ["moe::grouped_gemm_x<0>"]          # only the grouped GEMMs
    assert c["moe::grouped_gemm_x<0>"]["mfma_busy"] == 0.5


@pytest.mark.parametrize("changed", ["gemm.hip", "common.h"])
def test_records_dropped_once_a_source_changes(tree, changed):
    (tree / "parity_gate_gemm_amd" / "csrc" / changed).write_bytes(b"edited\n")
    b = _bench(tree)
    assert b.measured_traffic("wl") is None
    assert b.measured_mfma("wl") is None


def test_no_record_no_figure(tree):
    b = _bench(tree)
    assert b.measured_traffic("other") is None
    assert b.measured_mfma("other") is None
