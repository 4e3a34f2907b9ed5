"""The multi-bucket step (zero_shard_step_buckets) against the CPU oracle: each
bucket slice updates exactly its own state elements as the oracle's step of
that slice does, elements outside every slice are left alone, the flag and
the squared norm cover all slices, and tables longer than one launch holds
(32 slices, or 256 chunk pointers) are split without loss."""
import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import assert_matches_oracle, device, flags

pytestmark = pytest.mark.gpu


def _layout(sizes, gap):
    """Offsets (multiples of 8) of consecutive slices with `gap` elements
    between them, and the state length."""
    offs, end = [], 0
    for n in sizes:
        offs.append(end)
        end = (end + n + gap + 7) // 8 * 8
    return offs, end


def _run(sizes, N, S=65536.0, gap=24, seed=0, hyper=None, plant=None, in_place=False):
    dev = device()
    base = wl.LLAMA3_8B_SHARD
    hyper = hyper or base.hyper
    offs, n_state = _layout(sizes, gap)
    w = wl.ShardWorkload(name="buckets", wid=base.wid, n=n_state, n_replicas=N,
                         grad_sigma=base.grad_sigma, loss_scale=S, hyper=hyper,
                         m_sigma=base.m_sigma, v_sigma=base.v_sigma)
    h = wl.host_shard(w, n=n_state, offset_seed=700 + seed)
    slices_h = []
    for k, (n, off) in enumerate(zip(sizes, offs)):
        ch = [wl.host_fp16_grad(wl.seed_of(base.wid, 700 + seed, k, i), n, base.grad_sigma, S)
              for i in range(N)]
        slices_h.append((ch, off))
    if plant is not None:
        k, i, j = plant
        slices_h[k][0][i][j] = np.float16(np.nan)
    slices_d = zs.BucketSlices([([torch.from_numpy(c).to(dev) for c in ch], off)
                                for ch, off in slices_h])
    state_in = {k: torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16")}
    if in_place:
        out = state_in
    else:
        out = {k: torch.full_like(t, float("nan")) for k, t in state_in.items()}
    before_out = {k: t.clone() for k, t in out.items()}
    fl, sq = flags(dev)
    zs.zero_shard_step_buckets(slices_d, S, state_in["master"], state_in["m"], state_in["v"],
                               out["master"], out["m"], out["v"], out["p16"],
                               zs.adamw_params(hyper), fl, sq)
    torch.cuda.synchronize()
    return h, slices_h, offs, n_state, out, before_out, int(fl.item()), float(sq.item()), hyper


def _check(h, slices_h, offs, out, before_out, flag, sqnorm, hyper, S):
    covered = np.zeros(out["master"].numel(), bool)
    want_flag, want_sq = False, 0.0
    for (ch, off) in slices_h:
        n = ch[0].size
        sl = slice(off, off + n)
        covered[sl] = True
        want = ozs.shard_step(ch, h["master"][sl], h["m"][sl], h["v"][sl], h["p16"][sl], hyper, S)
        want_flag |= want.overflow
        want_sq += want.sqnorm
        if want.overflow:
            continue
        got = {k: t[sl] for k, t in out.items()}
        assert_matches_oracle(got, want, label=f"slice@{off} ")
    assert flag == int(want_flag)
    if not want_flag:
        assert abs(sqnorm - want_sq) <= 1e-6 * want_sq
    # elements outside every slice keep what the output held before
    idx = torch.from_numpy(np.flatnonzero(~covered)).to(out["master"].device)
    for k, t in out.items():
        assert torch.equal(t[idx].view(torch.uint8), before_out[k][idx].view(torch.uint8)), k


@pytest.mark.parametrize("N", [1, 3, 8, 16, 17, 64])
def test_ragged_slices_many_launches(N):
    """40 slices of ragged sizes: 2 launches at N <= 8, 3 at N = 16, more above."""
    rng = np.random.default_rng(N)
    sizes = [int(x) for x in rng.choice([1, 7, 8, 9, 255, 4095, 4096, 4097, 9000], size=40)]
    print(f"case: buckets N={N} slices={len(sizes)}", flush=True)
    h, sl, offs, n_state, out, before, fl, sq, hyper = _run(sizes, N, seed=N)
    _check(h, sl, offs, out, before, fl, sq, hyper, 65536.0)


def test_in_place_and_non_power_of_two_scale():
    sizes = [4096, 12_345, 64, 8]
    h, sl, offs, n_state, out, before, fl, sq, hyper = _run(sizes, 6, S=1000.0, seed=1,
                                                            in_place=True)
    _check(h, sl, offs, out, before, fl, sq, hyper, 1000.0)


def test_flag_from_any_slice():
    sizes = [4096] * 36
    h, sl, offs, n_state, out, before, fl, sq, hyper = _run(sizes, 8, seed=2,
                                                            plant=(34, 5, 4095))
    assert fl == 1


def test_matches_per_slice_calls():
    """One call over the table equals one zero_shard_step_out per slice, bit for bit."""
    dev = device()
    sizes = [5000, 4096, 17, 8192]
    h, sl, offs, n_state, out, before, fl, sq, hyper = _run(sizes, 8, seed=3)
    ref = {k: torch.full_like(t, float("nan")) for k, t in out.items()}
    st = {k: torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v")}
    hp = zs.adamw_params(hyper)
    for ch, off in sl:
        n = ch[0].size
        s = slice(off, off + n)
        zs.zero_shard_step_out([torch.from_numpy(c).to(dev) for c in ch], 65536.0,
                               st["master"][s], st["m"][s], st["v"][s], ref["master"][s],
                               ref["m"][s], ref["v"][s], ref["p16"][s], hp)
    torch.cuda.synchronize()
    for k in out:
        assert torch.equal(out[k].view(torch.uint8), ref[k].view(torch.uint8)), k
