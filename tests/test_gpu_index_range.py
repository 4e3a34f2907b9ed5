"""One call over more than 2^31 elements.  Every element index in the kernels
is 64-bit, so a shard longer than a signed 32-bit count is stepped, checked,
averaged and packed like any other: n = 2^31 + 4099 (the last tile partial,
3 params after the last full pack), N = 2, drawn like the Llama-3-8B
shard's inputs.

* the device-controlled single pass against the oracle at every element,
  its flag and squared norm against the oracle's;
* the two-pass check-then-step in place, and a two-slice bucket table whose
  second slice holds 2^31 + 3075 params, equal to it bit for bit;
* the fp16 mean against the oracle's at every element, and the same mean
  folded arrival by arrival equal to it;
* a bucket flatten whose second tensor holds all n elements, against the
  oracle's layout (the contents are a copy, checked on the device).
"""
import dataclasses
import gc
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle.flatten as ofl
import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from fullsize_util import compare_with_oracle, rel_close, threads
from gpu_util import device, flags

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_BIG = (1 << 31) + 4099


def _workload():
    return dataclasses.replace(wl.LLAMA3_8B_SHARD, name="index_range", n=N_BIG, n_replicas=2)


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _same_bits(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_step_beyond_2g_elements():
    dev = device()
    w = _workload()
    print(f"case: index range, n={w.n} N={w.n_replicas}: inputs", flush=True)
    d = wl.device_shard(w, dev)
    cur = (d["master"], d["m"], d["v"], d["p16"])
    out = tuple(torch.empty_like(t) for t in cur)
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    print("case: index range, device-controlled single pass", flush=True)
    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).single_pass(d["chunks"], (cur, out))
    c = zs.control_read(ctl)
    assert c.error == 0 and c.overflow == 0 and c.skip == 0 and c.cur == 1
    print(f"case: index range, single pass vs oracle on {threads()} threads", flush=True)
    overflow, want_sq, _ = compare_with_oracle(d["chunks"], cur, out, w.hyper, w.loss_scale,
                                               label="index range ")
    assert not overflow
    assert rel_close(c.sqnorm, want_sq), (c.sqnorm, want_sq)

    # a two-slice bucket table into a third copy: slice 1 is longer than 2^31
    split = 1024
    slices = zs.BucketSlices([([ch[:split] for ch in d["chunks"]], 0),
                              ([ch[split:] for ch in d["chunks"]], split)])
    third = tuple(torch.empty_like(t) for t in cur)
    hp = zs.adamw_params(w.hyper)
    fl, sq = flags(dev)
    print("case: index range, two-slice bucket table", flush=True)
    zs.zero_shard_step_buckets(slices, w.loss_scale, *cur[:3], *third, hp, fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == 0 and rel_close(float(sq.item()), want_sq)
    for name, a, b in zip(("master", "m", "v", "p16"), third, out):
        assert _same_bits(a, b), f"bucket table {name}"
    del slices, third

    # the two-pass form in place over the same inputs
    fl, sq = flags(dev)
    print("case: index range, two-pass check then in-place step", flush=True)
    zs.zero_overflow_check(d["chunks"], w.loss_scale, fl, sq)
    zs.zero_shard_step(d["chunks"], w.loss_scale, *cur, hp)
    torch.cuda.synchronize()
    assert int(fl.item()) == 0 and rel_close(float(sq.item()), want_sq)
    for name, a, b in zip(("master", "m", "v", "p16"), cur, out):
        assert _same_bits(a, b), f"two-pass {name}"


def test_mean_and_fold_beyond_2g_elements():
    dev = device()
    w = _workload()
    print(f"case: index range fp16 mean, n={w.n} N={w.n_replicas}: inputs", flush=True)
    chunks = wl.device_chunks(w, dev)
    mean16 = torch.empty(w.n, dtype=torch.float16, device=dev)
    fl, sq = flags(dev)
    print("case: index range, zero_reduce_mean_fp16", flush=True)
    zs.zero_reduce_mean_fp16(chunks, mean16, w.loss_scale, fl, sq)
    torch.cuda.synchronize()
    print(f"case: index range, fp16 mean vs oracle on {threads()} threads", flush=True)
    piece = 1 << 24

    def work(k):
        a, b = k * piece, min(w.n, (k + 1) * piece)
        want = ozs.replica_mean_fp16([c[a:b].cpu().numpy() for c in chunks])
        got = mean16[a:b].cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"mean16[{a}:{b}]"
        g = ozs.unscale(ozs.widen(want), w.loss_scale)
        return ozs.nonfinite(g), ozs.grad_sqnorm(g)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(work, range((w.n + piece - 1) // piece)))
    assert int(fl.item()) == int(any(r[0] for r in res)) == 0
    want_sq = float(np.sum(np.array([r[1] for r in res], np.float64)))
    assert rel_close(float(sq.item()), want_sq), (float(sq.item()), want_sq)

    acc = torch.empty(w.n, dtype=torch.float32, device=dev)
    folded = torch.empty_like(mean16)
    print("case: index range, fold arrival by arrival", flush=True)
    for i, ch in enumerate(chunks):
        zs.zero_accumulate_chunk(ch, i, len(chunks), acc, folded)
    torch.cuda.synchronize()
    assert _same_bits(folded, mean16)


def test_flatten_beyond_2g_elements():
    dev = device()
    w = _workload()
    print(f"case: index range flatten, second tensor of {w.n} elements: inputs", flush=True)
    src = wl.device_chunks(w, dev)
    small = src[0][:1001]
    big = src[1]
    align, pad = 256, 8 * 256
    layout = ofl.bucket_layout([small.numel(), big.numel()], align, pad)
    bucket = torch.full((layout[-1],), float("nan"), dtype=torch.float16, device=dev)
    print("case: index range, zero_bucket_flatten", flush=True)
    offs = zs.zero_bucket_flatten([small, big], bucket, align, pad)
    torch.cuda.synchronize()
    assert list(offs) == list(layout)
    o0, o1, end = layout
    assert _same_bits(bucket[o0:o0 + small.numel()], small)
    assert _same_bits(bucket[o1:o1 + big.numel()], big)
    zero_gap = bucket[o0 + small.numel():o1]
    zero_tail = bucket[o1 + big.numel():end]
    assert _same_bits(zero_gap, torch.zeros_like(zero_gap))
    assert _same_bits(zero_tail, torch.zeros_like(zero_tail))
