"""bench.py's host-side contract: one GPU only, its options, and the rule that
the counter-derived traffic is reported only while the kernel sources match
the digest the counters were taken on."""
import json
import os
import re
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


def test_every_committed_counter_summary_was_taken_on_these_kernels():
    """Each hardware-counter summary under profiles/ records the digest of
    the kernel sources it was taken on, and that is the digest of the
    sources as they are."""
    import glob
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.txt")))
    assert paths
    digest = _build.kernel_digest()
    for path in paths:
        m = re.search(r"^kernel_digest_sha256:\s*([0-9a-f]+)", open(path).read(), re.M)
        assert m and m.group(1) == digest, os.path.basename(path)


def test_ulp_line_counts_representable_values():
    import numpy as np
    one, m1 = np.float32(1.0), np.float32(-1.0)
    a = np.array([one, m1, 0.0, -0.0, one, 2.0], np.float32)
    b = np.array([np.nextafter(one, np.float32(2)), np.nextafter(m1, np.float32(0)),
                  np.float32(1e-45), np.float32(-1e-45), one, np.nextafter(np.float32(2), 0,
                                                                             dtype=np.float32)],
                 np.float32)
    d = np.abs(bench.ulp_line(a, np.int32) - bench.ulp_line(b, np.int32))
    assert list(d) == [1, 1, 1, 1, 0, 1]
    assert bench.ulp_line(np.array([0.0, -0.0], np.float32), np.int32).tolist() == [0, 0]
    h = np.array([1.0, -2.0, 65504.0], np.float16)
    g = np.array([np.nextafter(np.float16(1), np.float16(2)), -2.0, np.inf], np.float16)
    assert list(np.abs(bench.ulp_line(h, np.int16) - bench.ulp_line(g, np.int16))) == [1, 0, 1]


def test_digest_ignores_comments_but_not_code():
    a = "int x = 1; // one\n/* block */ int y = 2;"
    b = "int x = 1;   /* other words */\nint y = 2; // two"
    c = "int x = 1; int y = 3;"
    assert _build.code_text(a) == _build.code_text(b) != _build.code_text(c)


STATS = os.path.join(ROOT, "profiles", "shard_step_kernel_llama3_8b_shard_stats.txt")


def _fields(path):
    text = open(path).read()
    vals = dict(re.findall(r"^(\w+): (.+)$", text, re.M))
    line = json.loads(vals.pop("bench_line"))
    return vals, line


def test_committed_profile_agrees_with_its_bench_line():
    """The kernel-trace summary and the JSON line of the same profiled
    bench.py run tell the same story: the timed kernel's average over the
    timed dispatches is within 2 % of the line's HIP-event average, no
    longer than the line's whole step, and the roofline fraction recomputed
    from it is the one the summary states and within 0.02 of the line's."""
    vals, line = _fields(STATS)
    avg = float(vals["timed_kernel_average_ms"])
    assert vals["timed_kernel"] == "ctl_step_kernel<8, true>"
    assert int(vals["timed_dispatches"]) == line["steps"]
    assert line["config"]["workload"] == "llama3_8b_shard"
    n, bpp = int(vals["params"]), int(vals["bytes_per_param"])
    assert n == line["config"]["shard_params"] and bpp == line["config"]["bytes_per_param_fused_step"]
    fused = line["extra"]["fused_step_ms"]
    assert abs(avg - fused) <= 0.02 * fused, (avg, fused)
    assert avg <= line["ms_per_step"], (avg, line["ms_per_step"])
    frac = bpp * n / (avg * 1e-3) / 1e9 / 8000.0
    assert abs(frac - float(vals["roofline_frac_from_trace"].split()[0])) < 1e-4
    assert abs(frac - line["roofline"]["frac"]) <= 0.02
