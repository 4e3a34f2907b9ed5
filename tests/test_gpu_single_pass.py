"""The single-pass step (zero_shard_step_out) against the CPU oracle: the
out-of-place update equals the oracle's step element by element, leaves its
inputs untouched, fuses the same flag and squared norm as the check, and the
committed step (update, flag read-back, loss scale, commit or drop) walks the
same states as the oracle over clean and overflowing steps."""
import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import assert_matches_oracle, device, flags, to_dev

pytestmark = pytest.mark.gpu


def _shard(n, N, S, seed, base=wl.LLAMA3_8B_SHARD, hyper=None):
    w = wl.ShardWorkload(name=base.name, wid=base.wid, n=n, n_replicas=N,
                         grad_sigma=base.grad_sigma, loss_scale=S, hyper=hyper or base.hyper,
                         m_sigma=base.m_sigma, v_sigma=base.v_sigma)
    return w, wl.host_shard(w, n=n, offset_seed=seed)


def _bits(t):
    return t.view(torch.uint8).clone()


def _out_state(d):
    return dict(master=torch.full_like(d["master"], float("nan")),
                m=torch.full_like(d["m"], float("nan")),
                v=torch.full_like(d["v"], float("nan")),
                p16=torch.full_like(d["p16"], float("nan")))


@pytest.mark.parametrize("N,S", [(8, 65536.0), (3, 1024.0), (5, 1000.0), (16, 65536.0)])
def test_out_of_place_bit_exact_and_inputs_untouched(N, S):
    dev = device()
    w, h = _shard(100_003, N, S, seed=200 + N)
    print(f"case: single-pass N={N} S={S}", flush=True)
    d = to_dev(h, dev)
    before = {k: _bits(d[k]) for k in ("master", "m", "v", "p16")}
    o = _out_state(d)
    fl, sq = flags(dev)
    zs.zero_shard_step_out(d["chunks"], S, d["master"], d["m"], d["v"], o["master"], o["m"],
                           o["v"], o["p16"], zs.adamw_params(w.hyper), fl, sq)
    torch.cuda.synchronize()
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper, S)
    assert int(fl.item()) == 0
    assert abs(float(sq.item()) - want.sqnorm) <= 1e-6 * want.sqnorm
    for k, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
        got = o[k].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k
    assert np.array_equal(o["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))
    for k, b in before.items():
        assert torch.equal(_bits(d[k]), b), f"{k} input changed"


@pytest.mark.parametrize("n", [1, 7, 8, 9, 4095, 4096, 4097, 8191, 12_289])
def test_out_of_place_ragged_sizes(n):
    """Sizes around the 8-param pack and the 4096-param tile."""
    dev = device()
    w, h = _shard(n, 8, 65536.0, seed=300 + n)
    print(f"case: single-pass ragged n={n}", flush=True)
    d = to_dev(h, dev)
    o = _out_state(d)
    fl, sq = flags(dev)
    zs.zero_shard_step_out(d["chunks"], 65536.0, d["master"], d["m"], d["v"], o["master"],
                           o["m"], o["v"], o["p16"], zs.adamw_params(w.hyper), fl, sq)
    torch.cuda.synchronize()
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper, 65536.0)
    assert int(fl.item()) == 0 and abs(float(sq.item()) - want.sqnorm) <= 1e-6 * want.sqnorm
    assert_matches_oracle(o, want)


def test_in_place_through_out_entry_matches_in_place_step():
    """*_out == *_in is the in-place step, bit for bit."""
    dev = device()
    w, h = _shard(50_001, 8, 65536.0, seed=400)
    a, b = to_dev(h, dev), to_dev(h, dev)
    hp = zs.adamw_params(w.hyper)
    zs.zero_shard_step(a["chunks"], 65536.0, a["master"], a["m"], a["v"], a["p16"], hp)
    zs.zero_shard_step_out(b["chunks"], 65536.0, b["master"], b["m"], b["v"], b["master"],
                           b["m"], b["v"], b["p16"], hp)
    torch.cuda.synchronize()
    for k in ("master", "m", "v", "p16"):
        assert torch.equal(_bits(a[k]), _bits(b[k])), k


@pytest.mark.parametrize("plant", ["nan_tail", "inf_first", "none"])
def test_fused_flag_matches_check(plant):
    dev = device()
    n, N, S = 8195, 8, 65536.0
    w, h = _shard(n, N, S, seed=500)
    ch = [c.copy() for c in h["chunks"]]
    if plant == "nan_tail":
        ch[N - 1][n - 1] = np.nan
    elif plant == "inf_first":
        ch[0][0] = np.inf
    print(f"case: single-pass flag plant={plant}", flush=True)
    want_flag, want_sq = ozs.check_only(ch, S)
    d = to_dev(dict(h, chunks=ch), dev)
    o = _out_state(d)
    fl, sq = flags(dev)
    zs.zero_shard_step_out(d["chunks"], S, d["master"], d["m"], d["v"], o["master"], o["m"],
                           o["v"], o["p16"], zs.adamw_params(w.hyper), fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == int(want_flag)
    if not want_flag:
        assert abs(float(sq.item()) - want_sq) <= 1e-6 * want_sq


def test_committed_steps_follow_the_oracle():
    """Clean, overflow, clean, clean: the committed copy matches the oracle's
    state after each step, a skipped step leaves it bit-identical, the scale
    halves on overflow, and t advances only on clean steps."""
    dev = device()
    n, N = 40_009, 8
    w = wl.ShardWorkload(name="committed", wid=wl.LLAMA3_8B_SHARD.wid, n=n, n_replicas=N,
                         grad_sigma=1e-4, loss_scale=65536.0,
                         hyper=wl.LLAMA3_8B_SHARD.hyper, m_sigma=1e-4, v_sigma=1e-8)
    h = wl.host_shard(w, n=n, offset_seed=600)
    d = to_dev(h, dev)
    shard = zs.DoubleBufferedShard(d["master"], d["m"], d["v"], d["p16"])
    scaler = zs.LossScaler.create(scale=w.loss_scale, growth_interval=3)
    hp = zs.adamw_params(w.hyper)
    fl, sq = flags(dev)
    state = (h["master"], h["m"], h["v"], h["p16"])
    t = w.hyper.step
    chunks_dev = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    for k, plant in enumerate([False, True, False, False]):
        S = scaler.scale
        g = [wl.host_fp16_grad(wl.seed_of(w.wid, 600 + k, wl.ARRAY_GRAD, i), n, w.grad_sigma, S)
             for i in range(N)]
        if plant:
            g[3][1234] = np.float16(np.inf)
        for c, src in zip(chunks_dev, g):
            c.copy_(torch.from_numpy(src))
        before = [_bits(x) for x in shard.current]
        r = zs.committed_step(chunks_dev, shard, hp, scaler, fl, sq)
        torch.cuda.synchronize()
        want = ozs.shard_step(g, *state, w.hyper.replace(step=t), S)
        print(f"case: committed step {k} plant={plant} S={S}", flush=True)
        assert r.overflow == want.overflow == plant and r.skipped == plant
        if plant:
            assert scaler.scale == S / 2 and hp.step == t
            for a, b in zip(before, shard.current):
                assert torch.equal(a, _bits(b))
            continue
        assert hp.step == t + 1
        assert abs(r.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
        cur = dict(zip(("master", "m", "v", "p16"), shard.current))
        assert_matches_oracle(cur, want, label=f"step {k} ")
        state = (want.master, want.m, want.v, want.p16)
        t += 1
