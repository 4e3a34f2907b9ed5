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
