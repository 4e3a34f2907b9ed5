"""The device side of the seeded input generators (workloads/libzerogen.so):
Philox-4x32-10 against its published known-answer vectors, the normal draws'
distribution and reproducibility, the fp16 cast against numpy's binary16
rounding, and the scatter of non-finite entries."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "philox4x32_10_kat.json")


def test_philox_known_answers():
    dev = device()
    for case in json.load(open(GOLDEN))["cases"]:
        words = [int(x, 16) for x in case["counter"] + case["key"]]
        print(f"case: philox KAT {case['counter']} {case['key']}", flush=True)
        assert wl.device_philox(words, dev) == [int(x, 16) for x in case["out"]]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("absolute", [False, True])
def test_normal_draws(dtype, absolute):
    dev = device()
    n, sigma = 1_000_003, 6.5536
    print(f"case: normal draws {dtype} absolute={absolute}", flush=True)
    a = torch.empty(n, dtype=dtype, device=dev)
    b = torch.empty(n, dtype=dtype, device=dev)
    c = torch.empty(n, dtype=dtype, device=dev)
    wl.device_fill_normal(a, 12345, sigma, absolute)
    wl.device_fill_normal(b, 12345, sigma, absolute)
    wl.device_fill_normal(c, 12346, sigma, absolute)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16 if dtype == torch.float16 else torch.int32),
                       b.view(torch.int16 if dtype == torch.float16 else torch.int32))
    assert not torch.equal(a, c)
    x = a.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(x))
    if absolute:
        assert np.all(x >= 0)
        assert abs(x.mean() / (sigma * np.sqrt(2 / np.pi)) - 1) < 0.01
        assert abs(np.sqrt((x ** 2).mean()) / sigma - 1) < 0.01
    else:
        assert abs(x.mean()) < 0.01 * sigma
        assert abs(x.std() / sigma - 1) < 0.01
        # the tails of a normal: about 4.55 % beyond 2 sigma, 0.27 % beyond 3
        assert abs((np.abs(x) > 2 * sigma).mean() - 0.0455) < 0.002
        assert abs((np.abs(x) > 3 * sigma).mean() - 0.0027) < 0.0005
    # a prefix is the same draws as the start of a longer fill
    d = torch.empty(1001, dtype=dtype, device=dev)
    wl.device_fill_normal(d, 12345, sigma, absolute)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), a[:1001].cpu().numpy())


def test_fp16_cast_and_scatter():
    dev = device()
    print("case: generator fp16 cast and scatter", flush=True)
    st = wl.device_state(wl.LLAMA3_8B_SHARD, dev, n=100_003)
    master = st["master"].cpu().numpy()
    assert np.array_equal(st["p16"].cpu().numpy().view(np.uint16),
                          master.astype(np.float16).view(np.uint16))
    chunks = wl.device_chunks(wl.OVERFLOW, dev, n=5_000)
    before = [c.cpu().numpy() for c in chunks]
    sites = wl.injection_sites(wl.OVERFLOW, n=5_000, count=900)
    wl.device_inject(chunks, sites)
    torch.cuda.synchronize()
    ci, ei, vals = sites
    for k, (c, b) in enumerate(zip(chunks, before)):
        got = c.cpu().numpy()
        want = b.copy()
        want[ei[ci == k]] = vals[ci == k]
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), k
