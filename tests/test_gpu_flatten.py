"""Bucket flatten kernel against the oracle's layout and copy, bit for bit."""
import numpy as np
import pytest
import torch

import oracle.flatten as ofl
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import device

pytestmark = pytest.mark.gpu

GUARD = 0x7777      # fp16 bits written past the bucket end; must survive


def _run(host_tensors, align, pad, dev, misalign=False, extra=4096):
    want, want_offs = ofl.flatten(host_tensors, align, pad)
    srcs = []
    for t in host_tensors:
        flat = torch.from_numpy(t.reshape(-1).view(np.int16)).to(dev)
        if misalign and flat.numel():
            big = torch.empty(flat.numel() + 1, dtype=torch.int16, device=dev)
            big[1:].copy_(flat)
            flat = big[1:]                      # 2-byte aligned, not 16-byte aligned
        srcs.append(flat.view(torch.float16))
    cap = want.size + extra
    bucket = torch.full((cap,), GUARD, dtype=torch.int16, device=dev).view(torch.float16)
    offs = zs.zero_bucket_flatten(srcs, bucket, align=align, pad_multiple=pad)
    torch.cuda.synchronize()
    assert offs == want_offs
    got = bucket.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:want.size], want.view(np.uint16))
    assert np.all(got[want.size:] == GUARD)


@pytest.mark.parametrize("numel", [1, 255, 256, 257, 1_000_003])
@pytest.mark.parametrize("misalign", [False, True])
def test_single_tensor(numel, misalign):
    dev = device()
    t = wl.host_fp16_grad(wl.seed_of(70, numel), numel, 1e-4, 65536.0)
    print(f"case: flatten numel={numel} misalign={misalign}", flush=True)
    _run([t], 256, 2048, dev, misalign=misalign)


@pytest.mark.parametrize("align,pad", [(256, 2048), (8, 24), (3, 0), (1, 1), (256, 0)])
def test_several_tensors(align, pad):
    dev = device()
    rng = np.random.default_rng(align * 100 + pad)
    sizes = [5, 300, 0, 1, 4096, 777, 255, 257]
    ts = [wl.host_fp16_grad(wl.seed_of(71, i), k, 1e-3, 1024.0) for i, k in enumerate(sizes)]
    rng.shuffle(ts)
    print(f"case: flatten several align={align} pad={pad}", flush=True)
    _run(ts, align, pad, dev)
    _run(ts, align, pad, dev, misalign=True)


def test_many_tensors_cross_the_launch_batch():
    dev = device()
    rng = np.random.default_rng(72)
    sizes = rng.integers(0, 3000, 75)
    ts = [wl.host_fp16_grad(wl.seed_of(72, i), int(k), 1e-3, 1024.0) for i, k in enumerate(sizes)]
    _run(ts, 256, 256 * 8, dev)


def test_copies_bits_exactly():
    """NaN payloads, signed zeros and infinities are copied unchanged."""
    dev = device()
    bits = np.array([0x7e01, 0xfd55, 0x8000, 0x0000, 0x7c00, 0xfc00, 0x0001, 0x7bff] * 37,
                    np.uint16)
    _run([bits.view(np.float16)], 256, 512, dev)
    _run([bits.view(np.float16)], 256, 512, dev, misalign=True)


@pytest.mark.parametrize("bucket", [0, 3, 4])
def test_zero2_workload_buckets(bucket):
    """Real buckets of the ZeRO-2 workload: one MLP tensor (58,720,256
    elements), {ffn_norm, o, v} and {k, q, attn_norm} (33,558,528)."""
    dev = device()
    tensors = wl.zero2_tensors()
    plan = wl.zero2_bucket_plan()
    ts = []
    for k in plan[bucket]:
        name, shape = tensors[k]
        numel = int(np.prod(shape))
        ts.append(wl.host_fp16_grad(wl.seed_of(73, k), numel, 1e-4, 65536.0).reshape(shape))
    print(f"case: zero2 bucket {bucket}: {[tensors[k][0] for k in plan[bucket]]}", flush=True)
    _run(ts, wl.ZERO2_ALIGN, wl.ZERO2_ALIGN * wl.ZERO2_REPLICAS, dev, extra=256)


@pytest.mark.parametrize("align,pad", [(256, 2048), (8, 24), (3, 0)])
def test_batch_matches_oracle_per_bucket(align, pad):
    """Many buckets in one zero_bucket_flatten_batch call (their slots span
    several launches, some sources 2-byte aligned only): every bucket equals
    the oracle's flatten of its own tensors, bit for bit, and nothing past
    any bucket's padded end is written."""
    dev = device()
    rng = np.random.default_rng(74 + align + pad)
    specs = []
    for b in range(37):
        sizes = [int(x) for x in rng.integers(0, 5000, 1 + b % 4)]
        if b == 11:
            sizes = [0]                                  # an empty bucket
        if b == 20:
            sizes = [9_001, 1_000_003]                   # slots of many tiles
        specs.append([wl.host_fp16_grad(wl.seed_of(74, 1000 * b + i), k, 1e-3, 1024.0)
                      for i, k in enumerate(sizes)])
    pairs, wants = [], []
    for b, ts in enumerate(specs):
        want, want_offs = ofl.flatten(ts, align, pad)
        srcs = []
        for i, t in enumerate(ts):
            flat = torch.from_numpy(t.reshape(-1).view(np.int16)).to(dev)
            if (b + i) % 3 == 0 and flat.numel():
                big = torch.empty(flat.numel() + 1, dtype=torch.int16, device=dev)
                big[1:].copy_(flat)
                flat = big[1:]
            srcs.append(flat.view(torch.float16))
        bucket = torch.full((want.size + 64,), GUARD, dtype=torch.int16,
                            device=dev).view(torch.float16)
        pairs.append((srcs, bucket))
        wants.append((want, want_offs))
    print(f"case: flatten batch of {len(pairs)} buckets align={align} pad={pad}", flush=True)
    offs = zs.zero_bucket_flatten_batch(pairs, align=align, pad_multiple=pad)
    torch.cuda.synchronize()
    for b, ((_, bucket), (want, want_offs)) in enumerate(zip(pairs, wants)):
        assert offs[b] == want_offs, b
        got = bucket.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:want.size], want.view(np.uint16)), b
        assert np.all(got[want.size:] == GUARD), b


def test_batch_refuses_a_bad_bucket_and_writes_nothing():
    """A batch with one bucket too small is refused whole: ZERO_ERANGE, and
    no bucket of the batch is written."""
    dev = device()
    ts = [torch.ones(1000, dtype=torch.float16, device=dev) for _ in range(3)]
    good = torch.full((4096,), GUARD, dtype=torch.int16, device=dev).view(torch.float16)
    small = torch.full((1024,), GUARD, dtype=torch.int16, device=dev).view(torch.float16)
    with pytest.raises(zs.ZeroStepError) as e:
        zs.zero_bucket_flatten_batch([(ts[:1], good), (ts, small)], align=256, pad_multiple=256)
    assert e.value.code == zs.ZERO_ERANGE
    torch.cuda.synchronize()
    for bk in (good, small):
        assert bool((bk.view(torch.int16) == GUARD).all())
