"""The placement search (sharded_mixed_precision_step_amd.placement): it may
move a shard's arrays to new memory, but it hands back the same contents bit
for bit (the chunks and copy 0, the state), in tensors the step accepts, and
a step over the placed arrays gives the same bits as over the originals and
matches the oracle."""
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import assert_matches_oracle, device, flags, to_dev
from sharded_mixed_precision_step_amd import placement

pytestmark = pytest.mark.gpu

KEYS = ("master", "m", "v", "p16")


def _bits(t):
    return t.view(torch.uint8).clone()


@pytest.mark.parametrize("n,N,trials", [(1_000_003, 3, 4), (4097, 8, 3), (7, 1, 2)])
def test_contents_survive_and_step_matches(n, N, trials):
    dev = device()
    base = wl.LLAMA3_8B_SHARD
    w = wl.ShardWorkload(name=base.name, wid=base.wid, n=n, n_replicas=N,
                         grad_sigma=base.grad_sigma, loss_scale=base.loss_scale,
                         hyper=base.hyper, m_sigma=base.m_sigma, v_sigma=base.v_sigma)
    h = wl.host_shard(w, n=n, offset_seed=31 + N)
    d = to_dev(h, dev)
    print(f"case: placement n={n} N={N} trials={trials}", flush=True)
    spare = tuple(torch.empty_like(d[k]) for k in KEYS)
    ref_chunks = [c.clone() for c in d["chunks"]]
    ref_state = [d[k].clone() for k in KEYS]
    before_chunks = [_bits(c) for c in ref_chunks]
    before_state = [_bits(t) for t in ref_state]
    chunks, copies, rep = placement.place_shard(
        d["chunks"], (tuple(d[k] for k in KEYS), spare), w.hyper, w.loss_scale,
        trials=trials, max_spacer=64 << 20, budget_s=60.0)
    torch.cuda.synchronize()

    assert rep.trials <= trials and rep.final_ms <= rep.initial_ms
    assert all(1 <= k <= rep.trials for k in rep.kept)
    assert len(chunks) == N and len(copies) == 2 and all(len(c) == 4 for c in copies)
    for got, want in zip(chunks, before_chunks):
        assert got.dtype == torch.float16 and got.numel() == n and got.is_contiguous()
        assert torch.equal(_bits(got), want)
    for got, want, k in zip(copies[0], before_state, KEYS):
        assert got.is_contiguous() and got.numel() == n, k
        assert torch.equal(_bits(got), want), f"copy 0 {k} changed"
    for c in copies:
        for t in c:
            assert t.data_ptr() % 16 == 0
    # no array of one copy shares memory with the other copy or with a chunk
    ptrs = [t.data_ptr() for t in chunks] + [t.data_ptr() for c in copies for t in c]
    assert len(set(ptrs)) == len(ptrs)

    # a step over the placed arrays: the oracle's step, bit for bit the same
    # as the same step over copies of the inputs taken before the search (the
    # tensors passed in are scratch to the search)
    fl, sq = flags(dev)
    hp = zs.adamw_params(w.hyper)
    zs.zero_shard_step_out(chunks, w.loss_scale, *copies[0][:3], *copies[1], hp, fl, sq)
    orig_out = tuple(torch.empty_like(t) for t in ref_state)
    fl2, sq2 = flags(dev)
    zs.zero_shard_step_out(ref_chunks, w.loss_scale, *ref_state[:3], *orig_out, hp, fl2, sq2)
    torch.cuda.synchronize()
    for a, b in zip(copies[1], orig_out):
        assert torch.equal(_bits(a), _bits(b))
    # the host-pointer step adds the blocks' partial norms with fp64 atomics,
    # whose order varies from launch to launch
    assert int(fl.item()) == 0
    assert abs(float(sq.item()) - float(sq2.item())) <= 1e-12 * float(sq2.item())
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper,
                          w.loss_scale)
    assert_matches_oracle(dict(zip(KEYS, copies[1])), want)
    assert abs(float(sq.item()) - want.sqnorm) <= 1e-6 * max(want.sqnorm, 1e-300)


def test_lean_search_by_groups_keeps_and_restores_contents():
    """place_groups re-places one group per trial: a group whose contents are
    kept comes back bit for bit, arrays listed for restoring come back as
    they were even though the timing overwrites them, the input list is taken
    over (emptied), and the kept trials follow the times the stand-in timing
    reports (its own count of calls, so the fastest trial is known)."""
    dev = device()
    print("case: lean placement by groups", flush=True)
    src = [torch.randn(10_001, device=dev) for _ in range(6)]
    want = [_bits(t) for t in src]
    arrays = [t.clone() for t in src]
    calls = [0]
    times = [10.0, 9.0, 9.5, 7.0, 8.0, 6.0, 6.5]     # initial, then trials 1..6

    def timed(arrs):
        arrs[0].add_(1.0)                              # the timing overwrites array 0
        t = times[calls[0]]
        calls[0] += 1
        return t

    groups = [([0, 1], True), ([2, 3, 4], True), ([5], False)]
    got, rep = placement.place_groups(arrays, groups, timed, restore=[0], trials=6,
                                      max_spacer=1 << 20, budget_s=60.0)
    torch.cuda.synchronize()
    assert arrays == [] and len(got) == 6
    assert rep.trials == 6 and rep.kept == [1, 3, 5]
    assert rep.initial_ms == 10.0 and rep.final_ms == 6.0
    for i in range(5):                                 # kept contents, and array 0 restored
        assert torch.equal(_bits(got[i]), want[i]), i
    assert got[5].shape == src[5].shape and got[5].dtype == src[5].dtype
