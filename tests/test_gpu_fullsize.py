"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (the single-pass step; also the two-pass check-then-step), compared
with the CPU oracle element by element wherever the oracle can follow in
seconds on the host's cores, and by properties that hold at any size
elsewhere.

* Llama-3-8B shard (1,003,750,000 params, N = 8): every element, for the
  device-controlled single pass and for the two-pass step; and the
  page-literal split (the fp16 mean, its folds one, two and four arrivals at
  a time, the one-chunk update from it).
* Overflow (125,468,750 params, 100,375 injected inf/NaN): the step is
  skipped, the scale halves, the state stays bit-identical; then a clean
  step at the halved scale matches the oracle everywhere.
* ZeRO-2 bucketed (160 buckets, 973,111,296 params on one rank): every
  bucket flattened for 8 replicas, then all 160 slices stepped by one
  multi-bucket call; every element against the oracle; buckets 0, 3, 4 and
  159 (both bucket shapes, first and last) also from the replicas' tensors
  through the oracle's flatten; and against 160 single-slice calls and the
  device-controlled table call.
* 70B-class shard (4,412,500,000 params, N = 16) streamed in 23 buckets
  through two chunk buffers: every bucket against the oracle element by
  element as it completes, the squared norm against the oracle's sum over
  the buckets, and the fp16 writeback property over the whole shard.
"""
import gc
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle.flatten as ofl
import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from fullsize_util import (compare_with_expected, compare_with_oracle, oracle_check_only,
                           rel_close, threads)
from gpu_util import device, flags

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _bits(t):
    return t.view(torch.uint8)


def _assert_writeback_property(master, p16, label, piece=1 << 24):
    """p16 == fp16 round-to-nearest-even of master, and master finite, at
    every element: the last step of the update, at any size."""
    n = master.numel()

    def work(k):
        a, b = k * piece, min(n, (k + 1) * piece)
        mh = master[a:b].cpu().numpy()
        ph = p16[a:b].cpu().numpy()
        assert np.isfinite(mh).all(), f"{label}: non-finite master in [{a}:{b}]"
        assert np.array_equal(mh.astype(np.float16).view(np.uint16), ph.view(np.uint16)), \
            f"{label}: p16 is not the rounded master in [{a}:{b}]"

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(work, range((n + piece - 1) // piece)))


def test_llama3_8b_shard_full():
    """The step bench.py times (single pass under the device control block)
    against the oracle at every element; then the two-pass check-then-step
    on the same inputs against the same expected state."""
    dev = device()
    w = wl.LLAMA3_8B_SHARD
    print(f"case: full {w.name} n={w.n} N={w.n_replicas}", flush=True)
    d = wl.device_shard(w, dev)
    cur = (d["master"], d["m"], d["v"], d["p16"])
    out = tuple(torch.empty_like(t) for t in cur)
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).single_pass(d["chunks"], (cur, out))
    c = zs.control_read(ctl)
    assert c.error == 0 and c.overflow == 0 and c.skip == 0 and c.cur == 1
    assert c.step == w.hyper.step + 1 and c.scale == w.loss_scale
    print("case: full llama3_8b_shard, device-controlled single pass vs oracle", flush=True)
    overflow, want_sq, expected = compare_with_oracle(d["chunks"], cur, out, w.hyper,
                                                      w.loss_scale, label="single-pass ",
                                                      keep_expected=True)
    assert not overflow
    assert rel_close(c.sqnorm, want_sq), (c.sqnorm, want_sq)
    del out
    hp = zs.adamw_params(w.hyper)
    fl2, sq2 = flags(dev)
    zs.zero_overflow_check(d["chunks"], w.loss_scale, fl2, sq2)
    zs.zero_shard_step(d["chunks"], w.loss_scale, *cur, hp)
    torch.cuda.synchronize()
    print("case: full llama3_8b_shard, two-pass step vs oracle", flush=True)
    assert int(fl2.item()) == 0 and rel_close(float(sq2.item()), want_sq)
    compare_with_expected(cur, expected, label="two-pass ")


def test_llama3_8b_page_literal_full():
    """The page-literal split at the Llama-3-8B shard: the fp16 mean of the 8
    replicas against the oracle's at every element (with its flag and norm);
    the same mean folded arrival by arrival, in pairs and in quads equal to
    it bit for bit; then the one-chunk update from it against the oracle at
    every element."""
    dev = device()
    w = wl.LLAMA3_8B_SHARD
    N, n, S = w.n_replicas, w.n, w.loss_scale
    print(f"case: full {w.name} page-literal split n={n} N={N}", flush=True)
    d = wl.device_shard(w, dev)
    mean = torch.empty(n, dtype=torch.float16, device=dev)
    fl, sq = flags(dev)
    zs.zero_reduce_mean_fp16(d["chunks"], mean, S, fl, sq)
    torch.cuda.synchronize()
    piece = 1 << 24

    def check_mean(k):
        a, b = k * piece, min(n, (k + 1) * piece)
        want = ozs.replica_mean_fp16([c[a:b].cpu().numpy() for c in d["chunks"]])
        got = mean[a:b].cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), (a, b)
        g = ozs.unscale(ozs.widen(want), S)
        return ozs.nonfinite(g), ozs.grad_sqnorm(g)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(check_mean, range((n + piece - 1) // piece)))
    assert not any(r[0] for r in res) and int(fl.item()) == 0
    assert rel_close(float(sq.item()), float(np.sum([r[1] for r in res])))
    acc = torch.empty(n, dtype=torch.float32, device=dev)
    for groups in ([1] * N, [2] * (N // 2), [4] * (N // 4)):
        print(f"case: full page-literal fold in groups {groups}", flush=True)
        folded = torch.full((n,), float("nan"), dtype=torch.float16, device=dev)
        first = 0
        for g in groups:
            last = first + g == N
            if g == 1:
                zs.zero_accumulate_chunk(d["chunks"][first], first, N, acc,
                                         folded if last else None)
            else:
                zs.zero_accumulate_chunks(d["chunks"][first:first + g], first, N, acc,
                                          folded if last else None)
            first += g
        torch.cuda.synchronize()
        assert torch.equal(folded.view(torch.int16), mean.view(torch.int16)), groups
        del folded
    del acc
    cur = (d["master"], d["m"], d["v"], d["p16"])
    out = tuple(torch.empty_like(t) for t in cur)
    zs.zero_shard_step_out([mean], S, *cur[:3], *out, zs.adamw_params(w.hyper))
    torch.cuda.synchronize()
    print("case: full page-literal one-chunk step vs oracle", flush=True)
    overflow, _, _ = compare_with_oracle([mean], cur, out, w.hyper, S, label="split ")
    assert not overflow


def test_overflow_workload_full():
    dev = device()
    w = wl.OVERFLOW
    print(f"case: full {w.name} n={w.n} N={w.n_replicas} inject={w.n_inject}", flush=True)
    d = wl.device_shard(w, dev)
    wl.device_inject(d["chunks"], wl.injection_sites(w))
    shard = zs.DoubleBufferedShard(d["master"], d["m"], d["v"], d["p16"])
    snap = [t.clone() for t in shard.current]
    scaler = zs.LossScaler.create(scale=w.loss_scale)
    hp = zs.adamw_params(w.hyper)
    fl, sq = flags(dev)
    r = zs.committed_step(d["chunks"], shard, hp, scaler, fl, sq)
    torch.cuda.synchronize()
    want_flag, _ = oracle_check_only(d["chunks"], w.loss_scale)
    assert want_flag and r.overflow and r.skipped
    assert scaler.scale == w.loss_scale / 2 and hp.step == w.hyper.step and shard.cur == 0
    for a, b in zip(snap, shard.current):
        assert torch.equal(_bits(a), _bits(b))
    fl2, _ = flags(dev)
    zs.zero_overflow_check(d["chunks"], w.loss_scale, fl2, None)
    torch.cuda.synchronize()
    assert int(fl2.item()) == 1
    # the retry: clean gradients drawn at the halved scale, same t
    S2 = scaler.scale
    wl.device_chunks(w, dev, offset_seed=1, loss_scale=S2, out=d["chunks"])
    state_in = shard.current
    r2 = zs.committed_step(d["chunks"], shard, hp, scaler, fl, sq)
    torch.cuda.synchronize()
    assert not r2.overflow and not r2.skipped and hp.step == w.hyper.step + 1
    print("case: full overflow workload, clean retry vs oracle", flush=True)
    overflow, want_sq, _ = compare_with_oracle(d["chunks"], state_in, shard.current, w.hyper,
                                               S2, label="retry ")
    assert not overflow and rel_close(r2.sqnorm, want_sq)


ZERO2_SAMPLED = (0, 3, 4, 159)


def test_zero2_bucketed_full():
    """Every bucket is flattened for the 8 replicas and this rank's slice of
    each replica's bucket is kept (what the per-bucket reduce-scatter would
    deliver); then one zero_shard_step_buckets call updates all 160 slices,
    as a ZeRO-2 rank steps after backward.  Every element of the step is
    checked against the oracle; sampled buckets are also checked from the
    replicas' tensors through the oracle's flatten; 160 per-bucket
    zero_shard_step_out calls and the device-controlled table call must give
    the same bits."""
    dev = device()
    w = wl.ZERO2
    N, r, S = w.n_replicas, wl.ZERO2_RANK, w.loss_scale
    align, pad = wl.ZERO2_ALIGN, wl.ZERO2_ALIGN * w.n_replicas
    sizes = [int(np.prod(s)) for _, s in wl.zero2_tensors()]
    plan = wl.zero2_bucket_plan()
    layouts = [ofl.bucket_layout([sizes[k] for k in idx], align, pad) for idx in plan]
    assert len(plan) == 160 and sum(lay[-1] for lay in layouts) // N == w.n
    print(f"case: full {w.name} buckets={len(plan)} rank={r} n={w.n}", flush=True)
    lmax = max(lay[-1] for lay in layouts)
    buckets = [torch.empty(lmax, dtype=torch.float16, device=dev) for _ in range(N)]
    owned = [torch.empty(w.n, dtype=torch.float16, device=dev) for _ in range(N)]
    host_reps, offsets = {}, []
    off = 0
    for b, idx in enumerate(plan):
        L = layouts[b][-1]
        sl = L // N
        reps = [[wl.zero2_device_tensor(i, k, dev) for k in idx] for i in range(N)]
        for i in range(N):
            offs = zs.zero_bucket_flatten(reps[i], buckets[i], align=align, pad_multiple=pad)
            assert offs == layouts[b], (b, offs, layouts[b])
            owned[i][off:off + sl].copy_(buckets[i][r * sl:(r + 1) * sl])
        if b in ZERO2_SAMPLED:
            torch.cuda.synchronize()
            host_reps[b] = [[t.cpu().numpy() for t in reps[i]] for i in range(N)]
            for i in range(N):
                got = buckets[i][:L].cpu().numpy()
                want_b = ofl.flatten(host_reps[b][i], align, pad)[0]
                assert np.array_equal(got.view(np.uint16), want_b.view(np.uint16)), (b, i)
        del reps
        offsets.append((off, sl))
        off += sl
    assert off == w.n
    del buckets
    st = wl.device_state(w, dev)
    cur = (st["master"], st["m"], st["v"], st["p16"])
    out = tuple(torch.empty_like(t) for t in cur)
    table = zs.BucketSlices([([o[a:a + n] for o in owned], a) for a, n in offsets])
    hp = zs.adamw_params(w.hyper)
    fl, sq = flags(dev)
    zs.zero_shard_step_buckets(table, S, *cur[:3], *out, hp, fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == 0
    for b in ZERO2_SAMPLED:
        a, n = offsets[b]
        L = layouts[b][-1]
        print(f"case: zero2 bucket {b} (L={L}) step vs oracle", flush=True)
        want_b = [ofl.flatten(host_reps[b][i], align, pad)[0] for i in range(N)]
        want = ozs.shard_step([wb[r * n:(r + 1) * n] for wb in want_b],
                              *[t[a:a + n].cpu().numpy() for t in cur], w.hyper, S)
        assert not want.overflow
        fb, sb = flags(dev)
        zs.zero_overflow_check([o[a:a + n] for o in owned], S, fb, sb)
        torch.cuda.synchronize()
        assert int(fb.item()) == 0 and rel_close(float(sb.item()), want.sqnorm)
        for name, t, ref in zip(("master", "m", "v"), out[:3], (want.master, want.m, want.v)):
            assert np.array_equal(t[a:a + n].cpu().numpy().view(np.uint32),
                                  ref.view(np.uint32)), (b, name)
        assert np.array_equal(out[3][a:a + n].cpu().numpy().view(np.uint16),
                              want.p16.view(np.uint16))
    # every element of the rank's 973M-param step against the oracle, from
    # the slices the device flatten produced (checked above for the sampled
    # buckets against the oracle's flatten of the replicas' tensors)
    print("case: full zero2 rank, all 160 slices vs oracle", flush=True)
    overflow, want_sq, _ = compare_with_oracle(owned, cur, out, w.hyper, S, label="zero2 ")
    assert not overflow and rel_close(float(sq.item()), want_sq)
    # the same update as 160 separate calls, and as the whole step under the
    # device control block (what bench.py --workload zero2_bucketed times)
    ref = tuple(torch.empty_like(t) for t in cur)
    for a, n in offsets:
        zs.zero_shard_step_out([o[a:a + n] for o in owned], S, *(t[a:a + n] for t in cur[:3]),
                               *(t[a:a + n] for t in ref), hp)
    torch.cuda.synchronize()
    for x, y in zip(out, ref):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    del ref
    ctl = zs.control_new(zs.LossScaler.create(scale=S), w.hyper.step, dev)
    dst = tuple(torch.empty_like(t) for t in cur)
    zs.DeviceStepper(ctl, hp).single_pass_buckets(table, (cur, dst))
    c = zs.control_read(ctl)
    assert c.error == 0 and c.skip == 0 and c.cur == 1 and c.step == w.hyper.step + 1
    for x, y in zip(out, dst):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_zero2_rank_flatten_batch_full():
    """The rank's own 160 gradient buckets (bench.py's flatten leg) flattened
    by one zero_bucket_flatten_batch call: every bucket equals the one
    zero_bucket_flatten call per bucket gives, bit for bit, and the sampled
    buckets equal the oracle's flatten of the tensors."""
    dev = device()
    w = wl.ZERO2
    r = wl.ZERO2_RANK
    align, pad = wl.ZERO2_ALIGN, wl.ZERO2_ALIGN * w.n_replicas
    sizes = [int(np.prod(s)) for _, s in wl.zero2_tensors()]
    plan = wl.zero2_bucket_plan()
    layouts = [ofl.bucket_layout([sizes[k] for k in idx], align, pad) for idx in plan]
    print(f"case: full zero2 rank flatten batch, {len(plan)} buckets", flush=True)
    grads = [[wl.zero2_device_tensor(r, k, dev) for k in idx] for idx in plan]
    batch = [torch.empty(lay[-1], dtype=torch.float16, device=dev) for lay in layouts]
    single = [torch.empty(lay[-1], dtype=torch.float16, device=dev) for lay in layouts]
    offs = zs.zero_bucket_flatten_batch(list(zip(grads, batch)), align=align, pad_multiple=pad)
    assert offs == layouts
    for ts, bk in zip(grads, single):
        zs.zero_bucket_flatten(ts, bk, align=align, pad_multiple=pad)
    torch.cuda.synchronize()
    for b, (x, y) in enumerate(zip(batch, single)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), b
    for b in ZERO2_SAMPLED:
        want = ofl.flatten([t.cpu().numpy() for t in grads[b]], align, pad)[0]
        assert np.array_equal(batch[b].cpu().numpy().view(np.uint16), want.view(np.uint16)), b


def test_llama70b_shard_streamed():
    """The launch sequence bench.py times for this shard: one step under the
    device control block, each bucket updated as it arrives in one of two
    chunk buffers (the other refilled meanwhile), one decision at the end.
    Every one of the 23 buckets is compared with the oracle element by
    element as soon as its update is done (before its buffer is refilled),
    and the oracle's squared norms, summed over the buckets, must match the
    block's."""
    dev = device()
    w = wl.LLAMA70B_SHARD
    N, S = w.n_replicas, w.loss_scale
    assert sum(w.buckets) == w.n
    print(f"case: full {w.name} n={w.n} N={N} buckets={len(w.buckets)}", flush=True)
    st = wl.device_state(w, dev)
    cur = (st["master"], st["m"], st["v"], st["p16"])
    out = tuple(torch.empty_like(t) for t in cur)
    bmax = max(w.buckets)
    bufs = [[torch.empty(bmax, dtype=torch.float16, device=dev) for _ in range(N)]
            for _ in range(2)]
    ctl = zs.control_new(zs.LossScaler.create(scale=S), w.hyper.step, dev)
    checked = []
    want_sq_total = [0.0]

    def arrivals():
        off = 0
        for b, nb in enumerate(w.buckets):
            chunks = [c[:nb] for c in bufs[b % 2]]
            wl.device_chunks(w, dev, n=nb, offset_seed=100 + b, out=chunks)
            yield chunks, off
            # bucket b's update is enqueued; check it now, before its buffer
            # is refilled
            torch.cuda.synchronize()
            print(f"case: llama70b bucket {b} (n={nb}) step vs oracle", flush=True)
            s_in = tuple(t[off:off + nb] for t in cur)
            s_out = tuple(t[off:off + nb] for t in out)
            overflow, want_sq, _ = compare_with_oracle(chunks, s_in, s_out, w.hyper, S,
                                                       label=f"bucket {b} ")
            assert not overflow
            want_sq_total[0] += want_sq
            checked.append(b)
            off += nb

    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).single_pass_streamed(arrivals(), (cur, out))
    c = zs.control_read(ctl)
    assert checked == list(range(len(w.buckets)))
    assert c.error == 0 and c.overflow == 0 and c.skip == 0 and c.cur == 1
    assert c.step == w.hyper.step + 1 and c.scale == S
    assert rel_close(c.sqnorm, want_sq_total[0]), (c.sqnorm, want_sq_total[0])
    _assert_writeback_property(out[0], out[3], "llama70b")
