"""bench.py's host-side contract: one GPU only, its options, and the rule that
the counter-derived traffic is reported only while the kernel sources match
the digest the counters were taken on."""
import os
import subprocess
import sys

import pytest

import bench
from sharded_mixed_precision_step_amd import _build

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--no-placement", "--placement-trials",
                "--no-cpu-baseline", "--calibrate-copy"):
        assert opt in r.stdout, opt


def _summary(tmp_path, digest, fetch="28.0014", write="14.0081"):
    p = tmp_path / "pmc.txt"
    p.write_text(f"header\nfetch_bytes_per_param: {fetch}\nwrite_bytes_per_param: {write}\n"
                 f"kernel_digest_sha256: {digest}\n")
    return str(p)


def test_traffic_read_when_the_digest_matches(tmp_path, monkeypatch):
    digest = _build.kernel_digest()
    monkeypatch.setattr(bench, "PMC_SUMMARY", _summary(tmp_path, digest))
    assert bench.read_traffic(digest, 1000) == pytest.approx((28.0014 + 14.0081) * 1000)


def test_traffic_null_when_the_kernels_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PMC_SUMMARY", _summary(tmp_path, "0" * 64))
    assert bench.read_traffic(_build.kernel_digest(), 1000) is None
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.read_traffic(_build.kernel_digest(), 1000) is None


def test_committed_counter_summary_matches_the_sources():
    """The committed summary was taken on the kernels as they are, so the
    bench reports traffic rather than null."""
    assert bench.read_traffic(_build.kernel_digest(), 1003750000) is not None


def test_digest_ignores_comments_but_not_code():
    a = "int x = 1; // one\n/* block */ int y = 2;"
    b = "int x = 1;   /* other words */\nint y = 2; // two"
    c = "int x = 1; int y = 3;"
    assert _build.code_text(a) == _build.code_text(b) != _build.code_text(c)
