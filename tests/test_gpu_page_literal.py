"""The page-literal split against the CPU oracle: the owner's gradient mean
stored as fp16 (all chunks at once, one arriving chunk at a time, or groups
of chunks arriving together), then
the update from it as a one-chunk step, element by element and bit for bit;
also the whole split enqueued under the device control block."""
import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import device, flags

pytestmark = pytest.mark.gpu


def _chunks(n, N, seed, sigma=1e-4, S=65536.0):
    return [wl.host_fp16_grad(wl.seed_of(801, seed, i), n, sigma, S) for i in range(N)]


def _dev(hs, dev):
    return [torch.from_numpy(h).to(dev) for h in hs]


@pytest.mark.parametrize("N", [1, 3, 8, 16, 17, 64])
@pytest.mark.parametrize("n", [1, 7, 9, 2049, 100_003])
def test_reduce_mean_fp16_bit_exact(n, N):
    dev = device()
    ch = _chunks(n, N, seed=n * 100 + N)
    print(f"case: reduce mean fp16 n={n} N={N}", flush=True)
    mean = torch.empty(n, dtype=torch.float16, device=dev)
    fl, sq = flags(dev)
    zs.zero_reduce_mean_fp16(_dev(ch, dev), mean, 65536.0, fl, sq)
    torch.cuda.synchronize()
    want = ozs.replica_mean_fp16(ch)
    assert np.array_equal(mean.cpu().numpy().view(np.uint16), want.view(np.uint16))
    g = ozs.unscale(ozs.widen(want), 65536.0)
    assert int(fl.item()) == int(ozs.nonfinite(g))
    want_sq = ozs.grad_sqnorm(g)
    assert abs(float(sq.item()) - want_sq) <= 1e-6 * want_sq


def test_reduce_mean_fp16_rounding_cases():
    """Means that fall on binary16 ties, in the subnormal range, at the top
    of the range, and from opposite infinities."""
    dev = device()
    n = 4104
    rng = np.random.default_rng(3)
    a = rng.standard_normal(n).astype(np.float16)
    b = a.copy()
    b[:1024] = (a[:1024].astype(np.float32) + np.float32(2.0 ** -11)).astype(np.float16)
    c = rng.standard_normal(n).astype(np.float16)
    c[1024:2048] = np.float16(2.0 ** -24) * rng.integers(-1023, 1024, 1024)   # subnormals
    a[2048:2100] = np.float16(65504.0)
    b[2048:2100] = np.float16(65504.0)
    c[2048:2100] = np.float16(65504.0)
    a[2100], b[2100] = np.float16(np.inf), np.float16(-np.inf)
    for N, chunks in ((2, [a, b]), (3, [a, b, c])):
        mean = torch.empty(n, dtype=torch.float16, device=dev)
        zs.zero_reduce_mean_fp16(_dev(chunks, dev), mean)
        torch.cuda.synchronize()
        want = ozs.replica_mean_fp16(chunks)
        got = mean.cpu().numpy()
        assert np.array_equal(np.isnan(got), np.isnan(want))
        fin = ~np.isnan(want)
        assert np.array_equal(got[fin].view(np.uint16), want[fin].view(np.uint16)), N


@pytest.mark.parametrize("N", [1, 2, 3, 8, 17])
@pytest.mark.parametrize("n", [5, 4096, 20_011])
def test_accumulate_chunks_in_arrival_order(n, N):
    """Folding the chunks in one call per arrival gives the oracle's
    accumulated mean, which also equals the all-at-once mean."""
    dev = device()
    ch = _chunks(n, N, seed=n + 7 * N)
    print(f"case: accumulate n={n} N={N}", flush=True)
    acc = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    mean = torch.empty(n, dtype=torch.float16, device=dev)
    for i, c in enumerate(_dev(ch, dev)):
        zs.zero_accumulate_chunk(c, i, N, acc, mean)
    once = torch.empty_like(mean)
    zs.zero_reduce_mean_fp16(_dev(ch, dev), once)
    torch.cuda.synchronize()
    want = ozs.accumulate_chunks(ch)
    assert np.array_equal(mean.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert torch.equal(mean.view(torch.int16), once.view(torch.int16))


@pytest.mark.parametrize("N,groups", [(1, [1]), (2, [2]), (8, [2, 2, 2, 2]), (8, [3, 1, 4]),
                                      (8, [8]), (8, [7, 1]), (17, [5, 9, 3]),
                                      (64, [16, 16, 16, 16]), (64, [1, 62, 1])])
@pytest.mark.parametrize("n", [7, 4096, 20_011])
def test_fold_groups_equal_single_arrivals(n, N, groups):
    """Chunks folded in groups (zero_accumulate_chunks, one call per group of
    arrivals) leave the same accumulator after every group, bit for bit, as
    one zero_accumulate_chunk call per arrival, and the same fp16 mean, the
    oracle's."""
    dev = device()
    assert sum(groups) == N
    ch = _chunks(n, N, seed=3 * n + N + len(groups))
    d = _dev(ch, dev)
    print(f"case: fold groups n={n} N={N} groups={groups}", flush=True)
    acc_g = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    acc_s = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    mean_g = torch.empty(n, dtype=torch.float16, device=dev)
    mean_s = torch.empty(n, dtype=torch.float16, device=dev)
    first = 0
    for k in groups:
        last = first + k == N
        zs.zero_accumulate_chunks(d[first:first + k], first, N, acc_g, mean_g if last else None)
        for i in range(first, first + k):
            zs.zero_accumulate_chunk(d[i], i, N, acc_s, mean_s if i == N - 1 else None)
        first += k
        if not last:
            torch.cuda.synchronize()
            assert torch.equal(acc_g.view(torch.int32), acc_s.view(torch.int32)), first
    torch.cuda.synchronize()
    want = ozs.accumulate_chunks(ch)
    assert np.array_equal(mean_g.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert torch.equal(mean_g.view(torch.int16), mean_s.view(torch.int16))


@pytest.mark.parametrize("N,S", [(8, 65536.0), (3, 1024.0), (5, 1000.0)])
def test_split_step_matches_oracle(N, S):
    """fp16 mean, then the update as a one-chunk step, out of place with the
    flag: the oracle's split, bit for bit."""
    dev = device()
    n = 50_021
    base = wl.LLAMA3_8B_SHARD
    w = wl.ShardWorkload(name="split", wid=base.wid, n=n, n_replicas=N, grad_sigma=1e-4,
                         loss_scale=S, hyper=base.hyper, m_sigma=1e-4, v_sigma=1e-8)
    h = wl.host_shard(w, n=n, offset_seed=820 + N)
    print(f"case: split step N={N} S={S}", flush=True)
    d = {k: torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16")}
    out = {k: torch.full_like(t, float("nan")) for k, t in d.items()}
    mean = torch.empty(n, dtype=torch.float16, device=dev)
    zs.zero_reduce_mean_fp16(_dev(h["chunks"], dev), mean)
    fl, sq = flags(dev)
    zs.zero_shard_step_out([mean], S, d["master"], d["m"], d["v"], out["master"], out["m"],
                           out["v"], out["p16"], zs.adamw_params(w.hyper), fl, sq)
    torch.cuda.synchronize()
    m16 = ozs.replica_mean_fp16(h["chunks"])
    want = ozs.shard_step_from_fp16_mean(m16, h["master"], h["m"], h["v"], h["p16"], w.hyper, S)
    assert int(fl.item()) == 0 and abs(float(sq.item()) - want.sqnorm) <= 1e-6 * want.sqnorm
    for k, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
        assert np.array_equal(out[k].cpu().numpy().view(np.uint32), ref.view(np.uint32)), k
    assert np.array_equal(out["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))


def test_split_flag_from_planted_nan():
    dev = device()
    n, N = 9000, 8
    ch = _chunks(n, N, seed=830)
    ch[6][8999] = np.float16(np.nan)
    mean = torch.empty(n, dtype=torch.float16, device=dev)
    fl, sq = flags(dev)
    zs.zero_reduce_mean_fp16(_dev(ch, dev), mean, 65536.0, fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == 1
    assert np.isnan(float(mean[8999].item()))


def test_split_under_the_control_block_walks_the_oracle():
    """The page-literal split enqueued under the device control block (fp16
    mean, one-chunk single pass, decision on the device) over clean and
    overflowing steps: the oracle's split, loss scaler and t, bit for bit."""
    import oracle.loss_scale as ols
    dev = device()
    n, N = 30_011, 8
    base = wl.LLAMA3_8B_SHARD
    w = wl.ShardWorkload(name="split_ctl", wid=base.wid, n=n, n_replicas=N, grad_sigma=1e-4,
                         loss_scale=65536.0, hyper=base.hyper.replace(step=20),
                         m_sigma=1e-4, v_sigma=1e-8)
    h = wl.host_shard(w, n=n, offset_seed=840)
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    copies = (a, tuple(torch.full_like(x, float("nan")) for x in a))
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale, growth_interval=2),
                         w.hyper.step, dev)
    os_ = ols.ScalerState(scale=w.loss_scale, growth_interval=2)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    mean16 = torch.empty(n, dtype=torch.float16, device=dev)
    state, t, cur = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step, 0
    for k, plant in enumerate([False, True, False, False, True, False]):
        S = os_.scale
        g = [wl.host_fp16_grad(wl.seed_of(w.wid, 850 + k, i), n, w.grad_sigma, S)
             for i in range(N)]
        if plant:
            g[(3 * k) % N][(101 * k) % n] = np.float16(np.inf if k % 2 else np.nan)
        for c, src in zip(chunks, g):
            c.copy_(torch.from_numpy(src))
        stepper.single_pass_page_literal(chunks, mean16, copies)
        m16 = ozs.replica_mean_fp16(g)
        want = ozs.shard_step_from_fp16_mean(m16, *state, w.hyper.replace(step=t), S)
        skip = ols.update_loss_scale(os_, want.overflow)
        t += 0 if skip else 1
        c = zs.control_read(ctl)
        print(f"case: page-literal split under control, step {k} plant={plant} S={S}",
              flush=True)
        assert np.array_equal(mean16.cpu().numpy().view(np.uint16), m16.view(np.uint16))
        assert c.overflow == int(want.overflow) and c.skip == int(skip) and c.error == 0
        assert c.scale == np.float32(os_.scale) and c.step == t
        if skip:
            assert c.cur == cur
            continue
        assert abs(c.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
        cur = 1 - cur
        assert c.cur == cur
        for x, ref in zip(copies[cur], (want.master, want.m, want.v, want.p16)):
            bits = np.uint16 if ref.dtype == np.float16 else np.uint32
            assert np.array_equal(x.cpu().numpy().view(bits), ref.view(bits)), k
        state = (want.master, want.m, want.v, want.p16)
