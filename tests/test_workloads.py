"""Workload recipes: sizes, bucket plan and generator properties."""
import numpy as np
import pytest

import oracle.accounting as acc
import oracle.flatten as fl
import workloads as wl

pytestmark = pytest.mark.cpu


def test_shard_sizes():
    assert wl.TINY.n == 1_000_003 and wl.TINY.n_replicas == 3
    assert wl.LLAMA3_8B_SHARD.n == 1_003_750_000
    assert wl.OVERFLOW.n == 125_468_750 and wl.OVERFLOW.n % 8 != 0
    assert wl.OVERFLOW.n_inject == 100_375
    assert wl.LLAMA70B_SHARD.n == 4_412_500_000
    assert sum(wl.LLAMA70B_SHARD.buckets) == wl.LLAMA70B_SHARD.n
    assert len(wl.LLAMA70B_SHARD.buckets) == 23


def test_byte_model_matches_accounting():
    for w in (wl.TINY, wl.LLAMA3_8B_SHARD, wl.LLAMA70B_SHARD):
        assert w.bytes_per_param_step() == acc.step_bytes_per_param(w.n_replicas)


def test_zero2_bucket_plan():
    tensors = wl.zero2_tensors()
    assert len(tensors) == 32 * 9
    sizes = [int(np.prod(s)) for _, s in tensors]
    assert sum(sizes) == 7_784_890_368
    plan = wl.zero2_bucket_plan()
    assert len(plan) == 160
    assert sorted(k for b in plan for k in b) == list(range(len(tensors)))
    lengths = [fl.bucket_layout([sizes[k] for k in b], 256, 256 * 8)[-1] for b in plan]
    assert lengths.count(58_720_256) == 96 and lengths.count(33_558_528) == 64
    assert sum(L // 8 for L in lengths) == 973_111_296
    first = [tensors[k][0] for k in plan[3]]
    assert first == ["layers.31.ffn_norm", "layers.31.attn.o", "layers.31.attn.v"]


def test_generators_are_seeded():
    a = wl.host_shard(wl.TINY, n=1000)
    b = wl.host_shard(wl.TINY, n=1000)
    for k in ("master", "m", "v"):
        assert np.array_equal(a[k], b[k])
    for x, y in zip(a["chunks"], b["chunks"]):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    c = wl.host_shard(wl.TINY, n=1000, offset_seed=1)
    assert not np.array_equal(a["master"], c["master"])


def test_distributions():
    s = wl.host_shard(wl.LLAMA3_8B_SHARD, n=200_000)
    g = s["chunks"][3].astype(np.float64) / wl.LLAMA3_8B_SHARD.loss_scale
    assert abs(g.std() / 1e-4 - 1) < 0.02
    assert abs(s["master"].std() / 0.02 - 1) < 0.02
    assert np.all(s["m"] >= 0) and np.all(s["v"] >= 0)
    assert abs(s["m"].mean() / (1e-4 * np.sqrt(2 / np.pi)) - 1) < 0.02
    t = wl.host_shard(wl.TINY, n=1000)
    assert not t["m"].any() and not t["v"].any()


def test_exactly_summable():
    x = wl.exactly_summable_fp16(5, 100_000).astype(np.float64)
    assert np.all(np.abs(x) <= 256)
    assert np.array_equal(x * 1024, np.round(x * 1024))


def test_injection_sites():
    ci, ei, vals = wl.injection_sites(wl.OVERFLOW, n=1000, count=300)
    q = ci * 1000 + ei
    assert len(np.unique(q)) == 300 and q.max() < 8000
    assert np.isposinf(vals[0]) and np.isneginf(vals[1]) and np.isnan(vals[2])
