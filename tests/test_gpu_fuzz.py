"""Seeded random configurations against the oracle: 160 draws of shard length
(1 .. 50,000), replica count (1 .. 20), loss scale (powers of two and
arbitrary values), t (1 .. 10^6), betas, eps, weight decay, learning rate,
AdamW or L2 Adam, bias correction on or off, gradient magnitudes that
sometimes overflow fp16 or the unscale, and in one draw in six a single
planted inf or NaN.  Each draw runs the single pass
under the device control block and the host-pointer two-pass step; the
flag is the oracle's, and on a clean step every element is the oracle's, bit
for bit; on an overflow the control block skips and the state is
unchanged."""
import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import device, flags

pytestmark = pytest.mark.gpu

CASES = 160


def _draw(case):
    rng = np.random.default_rng(7000 + case)
    N = int(rng.integers(1, 21))
    n = int(rng.integers(1, 50_001))
    kind = rng.integers(0, 3)
    S = float(2.0 ** int(rng.integers(-4, 25))) if kind < 2 else float(rng.uniform(0.5, 1e5))
    hyper = wl.AdamWHyper(lr=float(10 ** rng.uniform(-6, -1)),
                          beta1=float(rng.uniform(0.5, 0.99)),
                          beta2=float(rng.uniform(0.9, 0.99999)),
                          eps=float(10 ** rng.uniform(-12, -3)),
                          weight_decay=float(rng.uniform(0, 0.1)) if rng.random() < 0.8 else 0.0,
                          step=int(rng.integers(1, 1_000_001)),
                          decoupled_wd=bool(rng.random() < 0.7),
                          bias_correction=bool(rng.random() < 0.8))
    sigma = float(10 ** rng.uniform(-7, -1))
    with np.errstate(over="ignore"):
        chunks = [(rng.standard_normal(n, dtype=np.float32) * np.float32(sigma * S))
                  .astype(np.float16) for _ in range(N)]
    if rng.random() < 1 / 6:
        chunks[int(rng.integers(0, N))][int(rng.integers(0, n))] = np.float16(
            [np.inf, -np.inf, np.nan][int(rng.integers(0, 3))])
    master = (rng.standard_normal(n, dtype=np.float32) *
              np.float32(10 ** rng.uniform(-3, 0)))
    m = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    v = np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(sigma * sigma)
    return dict(N=N, n=n, S=S, hyper=hyper, chunks=chunks, master=master, m=m, v=v,
                p16=master.astype(np.float16))


def _same(t, ref):
    bits = np.uint16 if ref.dtype == np.float16 else np.uint32
    return np.array_equal(t.cpu().numpy().view(bits), ref.view(bits))


@pytest.mark.parametrize("case", range(CASES))
def test_random_configuration_matches_oracle(case):
    dev = device()
    c = _draw(case)
    h = c["hyper"]
    print(f"case: fuzz {case}: n={c['n']} N={c['N']} S={c['S']} t={h.step} "
          f"decoupled={h.decoupled_wd} bc={h.bias_correction}", flush=True)
    want = ozs.shard_step(c["chunks"], c["master"], c["m"], c["v"], c["p16"], h, c["S"])
    state = (c["master"], c["m"], c["v"], c["p16"])
    chunks = [torch.from_numpy(x).to(dev) for x in c["chunks"]]

    # the single pass under the control block, its table based at t
    a = tuple(torch.from_numpy(x).to(dev) for x in state)
    copies = (a, tuple(torch.empty_like(x) for x in a))
    ctl = zs.control_new(zs.LossScaler.create(scale=c["S"]), h.step, dev)
    zs.DeviceStepper(ctl, zs.adamw_params(h)).single_pass(chunks, copies)
    cb = zs.control_read(ctl)
    assert cb.error == 0 and cb.overflow == int(want.overflow) and cb.skip == int(want.overflow)
    if want.overflow:
        assert cb.cur == 0 and cb.step == h.step
        for x, ref in zip(copies[0], state):
            assert _same(x, ref)
    else:
        assert cb.cur == 1 and cb.step == h.step + 1
        assert abs(cb.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
        for name, x, ref in zip(("master", "m", "v", "p16"), copies[1],
                                (want.master, want.m, want.v, want.p16)):
            assert _same(x, ref), name

    # the host-pointer two-pass: check, then the in-place step if clean
    d = [torch.from_numpy(x).to(dev) for x in state]
    fl, sq = flags(dev)
    zs.zero_overflow_check(chunks, c["S"], fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == int(want.overflow)
    if not want.overflow:
        zs.zero_shard_step(chunks, c["S"], *d, zs.adamw_params(h))
        torch.cuda.synchronize()
        for name, x, ref in zip(("master", "m", "v", "p16"), d,
                                (want.master, want.m, want.v, want.p16)):
            assert _same(x, ref), name


GUARD = 0x7E01          # a NaN pattern no flatten writes


@pytest.mark.parametrize("case", range(24))
def test_random_flatten_batch_matches_oracle(case):
    """A batch of 1-9 buckets of 0-12 tensors each (0-30,000 elements, some
    sources only 2-byte aligned), with align in 1..1024 and pad_multiple
    0 or a multiple of align: each bucket equals the oracle's flatten bit for
    bit, and nothing past its padded end is written; one call per bucket
    gives the same buckets."""
    import oracle.flatten as ofl
    dev = device()
    rng = np.random.default_rng(8000 + case)
    align = int(rng.integers(1, 1025))
    pad = 0 if rng.random() < 0.25 else align * int(rng.integers(1, 17))
    specs = [[rng.standard_normal(int(rng.integers(0, 30_001))).astype(np.float16)
              for _ in range(int(rng.integers(0, 13)))] for _ in range(int(rng.integers(1, 10)))]
    print(f"case: flatten fuzz {case}: {len(specs)} buckets align={align} pad={pad}", flush=True)
    pairs, wants, singles = [], [], []
    for ts in specs:
        want, want_offs = ofl.flatten(ts, align, pad)
        srcs = []
        for t in ts:
            flat = torch.from_numpy(t.view(np.int16)).to(dev)
            if rng.random() < 0.4 and flat.numel():
                big = torch.empty(flat.numel() + 1, dtype=torch.int16, device=dev)
                big[1:].copy_(flat)
                flat = big[1:]
            srcs.append(flat.view(torch.float16))
        bucket = torch.full((want.size + 64,), GUARD, dtype=torch.int16,
                            device=dev).view(torch.float16)
        single = torch.full_like(bucket, 0).view(torch.int16).fill_(GUARD).view(torch.float16)
        pairs.append((srcs, bucket))
        singles.append(single)
        wants.append((want, want_offs))
    offs = zs.zero_bucket_flatten_batch(pairs, align=align, pad_multiple=pad)
    for (srcs, _), single in zip(pairs, singles):
        zs.zero_bucket_flatten(srcs, single, align, pad)
    torch.cuda.synchronize()
    for b, ((_, bucket), single, (want, want_offs)) in enumerate(zip(pairs, singles, wants)):
        assert offs[b] == want_offs, b
        got = bucket.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:want.size], want.view(np.uint16)), b
        assert np.all(got[want.size:] == GUARD), b
        assert torch.equal(single.view(torch.int16), bucket.view(torch.int16)), b


@pytest.mark.parametrize("case", range(24))
def test_random_bucket_table_matches_oracle(case):
    """A shard tiled by 1-70 slices of random lengths (multiples of 8 apart,
    the last ragged), N in 1..20, in the multi-bucket call and under the
    control block: the state is the oracle's step of the whole shard, bit for
    bit, and the flag is the oracle's."""
    dev = device()
    rng = np.random.default_rng(9000 + case)
    N = int(rng.integers(1, 21))
    k = int(rng.integers(1, 71))
    sizes = [8 * int(x) for x in rng.integers(0, 700, k - 1)]
    sizes.append(int(rng.integers(1, 5000)))
    n = sum(sizes)
    S = float(2.0 ** int(rng.integers(0, 17)))
    hyper = wl.AdamWHyper(step=int(rng.integers(1, 5000)))
    chunks_h = [(rng.standard_normal(n, dtype=np.float32) * np.float32(1e-4 * S))
                .astype(np.float16) for _ in range(N)]
    if rng.random() < 0.2:
        chunks_h[int(rng.integers(0, N))][int(rng.integers(0, n))] = np.float16(np.nan)
    master = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
    m = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-4)
    v = np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(1e-8)
    p16 = master.astype(np.float16)
    print(f"case: bucket table fuzz {case}: {k} slices n={n} N={N} S={S}", flush=True)
    want = ozs.shard_step(chunks_h, master, m, v, p16, hyper, S)
    chunks = [torch.from_numpy(x).to(dev) for x in chunks_h]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int)
    table = zs.BucketSlices([([c[o:o + sz] for c in chunks], int(o))
                             for o, sz in zip(offs, sizes)])
    state = (master, m, v, p16)
    # host-pointer table call
    a = tuple(torch.from_numpy(x).to(dev) for x in state)
    b = tuple(torch.empty_like(x) for x in a)
    fl, sq = flags(dev)
    zs.zero_shard_step_buckets(table, S, *a[:3], *b, zs.adamw_params(hyper), fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == int(want.overflow)
    if not want.overflow:
        for name, x, ref in zip(("master", "m", "v", "p16"), b,
                                (want.master, want.m, want.v, want.p16)):
            assert _same(x, ref), name
    # under the control block
    ctl = zs.control_new(zs.LossScaler.create(scale=S), hyper.step, dev)
    zs.DeviceStepper(ctl, zs.adamw_params(hyper)).single_pass_buckets(table, (a, b))
    c = zs.control_read(ctl)
    assert c.error == 0 and c.overflow == int(want.overflow)
    got = (a, b)[c.cur]
    for name, x, ref in zip(("master", "m", "v", "p16"), got,
                            state if want.overflow else (want.master, want.m, want.v, want.p16)):
        assert _same(x, ref), name
