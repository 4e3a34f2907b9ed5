"""The boundary from C alone: tests/c_client/zero_client (host code, gcc,
linked against libzerostep.so and the HIP runtime, no Python or torch in the
process) runs one rank's ZeRO-2 step through the four calls of the C ABI --
zero_bucket_flatten for each replica, zero_overflow_check on the rank's
chunks, zero_update_loss_scale with the flag read back, zero_shard_step on a
clean step -- and its output is compared with the oracle: the bucket layout
and every element bit for bit, the flag, the skip, the scaler's state, the
squared norm within 1e-6 relative.

Inputs: N = 4 replicas of three gradient tensors of ragged sizes (5,000, 1
and 70,001 fp16 values, drawn like the tiny workload's), align 256, the
bucket padded to N shards, rank 2's shard of the state.  Cases: a clean step
that also reaches the growth interval (the scale doubles), and a step with
+inf in one replica inside rank 2's shard (skipped: the scale halves and the
state comes back unchanged)."""
import os
import subprocess

import numpy as np
import pytest

import oracle.flatten as ofl
import oracle.loss_scale as ols
import oracle.zero_step as ozs
import workloads as wl
from c_client.build import BINARY
from c_client.client_io import ClientInput, read_output
from gpu_util import device

pytestmark = pytest.mark.gpu

N, RANK, ALIGN = 4, 2, 256
NUMELS = (5000, 1, 70001)


def _inputs(overflow: bool) -> ClientInput:
    w = wl.TINY
    replicas = [[wl.host_fp16_grad(wl.seed_of(w.wid, 40 + i, k), numel, w.grad_sigma,
                                   w.loss_scale) for k, numel in enumerate(NUMELS)]
                for i in range(N)]
    layout = ofl.bucket_layout(NUMELS, ALIGN, ALIGN * N)
    s = layout[-1] // N
    if overflow:
        # +inf in replica 1 at the first element of the third tensor that
        # falls inside rank 2's shard
        k0 = max(RANK * s - layout[2], 0)
        assert k0 < NUMELS[2] and RANK * s <= layout[2] + k0 < (RANK + 1) * s
        replicas[1][2] = replicas[1][2].copy()
        replicas[1][2][k0] = np.float16(np.inf)
    h = wl.host_shard(w, n=s, offset_seed=41)
    return ClientInput(replicas=replicas, rank=RANK, align=ALIGN, hyper=w.hyper.replace(step=7),
                       loss_scale=w.loss_scale, growth_factor=2.0, backoff_factor=0.5,
                       min_scale=1.0, max_scale=2.0 ** 24, growth_interval=3, good_steps=2,
                       skipped_steps=5, master=h["master"], m=h["m"], v=h["v"], p16=h["p16"])


def _run_client(inp: ClientInput, tmp_path):
    if not os.path.exists(BINARY):
        pytest.fail("the C client is not built: run __graft_entry__.build()")
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    src.write_bytes(inp.to_bytes())
    print(f"case: C client N={N} rank={RANK} numels={NUMELS}", flush=True)
    proc = subprocess.run([BINARY, str(src), str(dst)], capture_output=True, text=True,
                          timeout=120)
    assert proc.returncode == 0, proc.stderr
    return read_output(dst.read_bytes(), len(NUMELS))


def _oracle(inp: ClientInput):
    buckets = [ofl.flatten(rep, inp.align, inp.align * N) for rep in inp.replicas]
    layout = buckets[0][1]
    s = layout[-1] // N
    chunks = [b[RANK * s:(RANK + 1) * s] for b, _ in buckets]
    flag, sqnorm = ozs.check_only(chunks, inp.loss_scale)
    scaler = ols.ScalerState(scale=inp.loss_scale, growth_factor=inp.growth_factor,
                             backoff_factor=inp.backoff_factor, min_scale=inp.min_scale,
                             max_scale=inp.max_scale, growth_interval=inp.growth_interval,
                             good_steps=inp.good_steps, skipped_steps=inp.skipped_steps)
    skip = ols.update_loss_scale(scaler, flag)
    state = (inp.master, inp.m, inp.v, inp.p16)
    if not skip:
        r = ozs.shard_step(chunks, *state, inp.hyper, inp.loss_scale)
        state = (r.master, r.m, r.v, r.p16)
    return layout, flag, sqnorm, skip, scaler, state


def _same_bits(a, b):
    bits = np.uint16 if a.dtype == np.float16 else np.uint32
    return a.shape == b.shape and np.array_equal(a.view(bits), b.view(bits))


@pytest.mark.parametrize("overflow", [False, True], ids=["clean_and_growth", "overflow_skip"])
def test_c_client_matches_oracle(overflow, tmp_path):
    device()  # skips without a GPU
    inp = _inputs(overflow)
    got = _run_client(inp, tmp_path)
    layout, flag, sqnorm, skip, scaler, state = _oracle(inp)
    assert got.offsets == layout and got.L == layout[-1] and got.s == layout[-1] // N
    assert bool(got.overflow) == flag == overflow
    assert bool(got.skip) == skip == overflow
    assert got.scale == scaler.scale == (inp.loss_scale / 2 if overflow else inp.loss_scale * 2)
    assert got.good_steps == scaler.good_steps and got.skipped_steps == scaler.skipped_steps
    if not overflow:
        assert abs(got.sqnorm - sqnorm) <= 1e-6 * sqnorm
    for name, a, b in zip(("master", "m", "v", "p16"), (got.master, got.m, got.v, got.p16),
                          state):
        assert _same_bits(a, b), name
    if overflow:  # the state comes back as it went in
        for a, b in zip((got.master, got.m, got.v, got.p16),
                        (inp.master, inp.m, inp.v, inp.p16)):
            assert _same_bits(a, b)
