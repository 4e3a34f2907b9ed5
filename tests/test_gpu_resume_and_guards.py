"""Checkpoint and resume, and writes confined to the shard.

Resume: K device-controlled steps, a checkpoint of the state and the control
block written to disk and read back into fresh device memory, then K more
steps give bit for bit the state and block of 2K uninterrupted steps (and
that state matches the oracle's 2K steps).

Guard bands: every kernel that writes a shard (in-place and out-of-place
steps, the multi-bucket step, the fp16 mean, the accumulator, the control
steps over a shard and over a bucket table, the traffic twin) leaves the
bytes just before and just after its output arrays as they were, at sizes
with a ragged tail."""
import numpy as np
import pytest
import torch

import oracle.loss_scale as ols
import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import device, flags, guarded, guards_intact
from sharded_mixed_precision_step_amd import twin as zt

pytestmark = pytest.mark.gpu

N, n, K = 8, 20_011, 3


def _workload():
    base = wl.LLAMA3_8B_SHARD
    return wl.ShardWorkload(name="resume", wid=base.wid, n=n, n_replicas=N, grad_sigma=1e-4,
                            loss_scale=65536.0, hyper=base.hyper.replace(step=10),
                            m_sigma=1e-4, v_sigma=1e-8)


def _grads(w, k, S):
    g = [wl.host_fp16_grad(wl.seed_of(w.wid, 1000 + k, wl.ARRAY_GRAD, i), n, w.grad_sigma, S)
         for i in range(N)]
    if k == 1:
        g[2][77] = np.float16(np.inf)          # one skipped step inside the run
    return g


def _run(w, h, dev, steps, start=0, state=None, ctl=None):
    """Device-controlled single-pass steps start..start+steps-1 (gradients
    drawn at the block's current scale); returns (current copy, control)."""
    if state is None:
        a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale, growth_interval=2),
                             w.hyper.step, dev)
    else:
        a = state
    copies = (a, tuple(torch.empty_like(t) for t in a))
    c = zs.control_read(ctl)
    # the loaded block names the current copy; bring it to copy 0 of this run
    if c.cur != 0:
        raise AssertionError("callers pass the current copy as copy 0")
    hp = zs.adamw_params(w.hyper.replace(step=int(c.step)))
    stepper = zs.DeviceStepper(ctl, hp)
    chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    for k in range(start, start + steps):
        S = zs.control_read(ctl).scale
        for t, g in zip(chunks, _grads(w, k, S)):
            t.copy_(torch.from_numpy(g))
        stepper.single_pass(chunks, copies)
    c = zs.control_read(ctl)
    return copies[c.cur & 1], ctl


def _normalised(ctl):
    """The block with cur set to 0: a run that resumes from a checkpoint
    renumbers its copies so that the loaded state is copy 0."""
    c = zs.control_read(ctl)
    cur = c.cur
    c.cur = 0
    return c, cur


def test_resume_from_checkpoint_is_bit_identical(tmp_path):
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=1001)
    # 2K steps in one run
    full, full_ctl = _run(w, h, dev, 2 * K)
    # K steps, checkpoint, K more from the file
    half, half_ctl = _run(w, h, dev, K)
    c, cur = _normalised(half_ctl)
    ctl_bytes = torch.frombuffer(bytearray(bytes(c)), dtype=torch.uint8)
    path = str(tmp_path / "shard.safetensors")
    zs.save_shard_state(path, *half, ctl=ctl_bytes)
    del half, half_ctl
    torch.cuda.synchronize()
    loaded = zs.load_shard_state(path, dev)
    state = (loaded["master"], loaded["exp_avg"], loaded["exp_avg_sq"], loaded["param_fp16"])
    resumed, resumed_ctl = _run(w, h, dev, K, start=K, state=state, ctl=loaded["control"])
    for x, y in zip(full, resumed):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    a, _ = _normalised(full_ctl)
    b, _ = _normalised(resumed_ctl)
    for name, _ in zs.StepControl._fields_:
        if name == "sqnorm":
            assert abs(a.sqnorm - b.sqnorm) <= 1e-12 * a.sqnorm
        elif name in ("sqnorm_part", "check_part"):
            for x, y in zip(getattr(a, name), getattr(b, name)):
                assert abs(x - y) <= 1e-12 * abs(y)
        else:
            assert getattr(a, name) == getattr(b, name), name
    # and the 2K steps are the oracle's 2K steps
    os_ = ols.ScalerState(scale=w.loss_scale, growth_interval=2)
    st, t = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step
    for k in range(2 * K):
        S = os_.scale
        r = ozs.shard_step(_grads(w, k, S), *st, w.hyper.replace(step=t), S)
        if not ols.update_loss_scale(os_, r.overflow):
            st, t = (r.master, r.m, r.v, r.p16), t + 1
    assert a.step == t and a.scale == np.float32(os_.scale) and a.skipped_steps == 1
    for x, ref in zip(full, st):
        bits = np.uint16 if ref.dtype == np.float16 else np.uint32
        assert np.array_equal(x.cpu().numpy().view(bits), ref.view(bits))


def _assert_guards(buf, numel, label):
    assert guards_intact(buf, numel), f"{label}: a write outside the array"


@pytest.mark.parametrize("nn", [1, 7, 4097, 12_345])
def test_no_writes_outside_the_outputs(nn):
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=nn, offset_seed=1100 + nn)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    hp = zs.adamw_params(w.hyper)
    print(f"case: guard bands n={nn}", flush=True)

    def state(dst_nan=False):
        out = {}
        for k in ("master", "m", "v", "p16"):
            src = torch.from_numpy(h[k]).to(dev)
            out[k] = guarded(nn, src.dtype, dev, None if dst_nan else src)
        return out

    # in place
    s = state()
    zs.zero_shard_step(chunks, w.loss_scale, *(s[k][1] for k in ("master", "m", "v", "p16")), hp,
                       *flags(dev))
    # out of place
    src, dst = state(), state(dst_nan=True)
    zs.zero_shard_step_out(chunks, w.loss_scale, *(src[k][1] for k in ("master", "m", "v")),
                           *(dst[k][1] for k in ("master", "m", "v", "p16")), hp, *flags(dev))
    # one bucket slice through the table
    bsrc, bdst = state(), state(dst_nan=True)
    zs.zero_shard_step_buckets(zs.BucketSlices([(chunks, 0)]), w.loss_scale,
                               *(bsrc[k][1] for k in ("master", "m", "v")),
                               *(bdst[k][1] for k in ("master", "m", "v", "p16")), hp,
                               *flags(dev))
    # under the control block, both flows
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    cs = state()
    zs.DeviceStepper(ctl, hp).two_pass(chunks, *(cs[k][1] for k in ("master", "m", "v", "p16")),
                                       max_grad_norm=1e-3)
    ctl2 = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    c0, c1 = state(), state(dst_nan=True)
    zs.DeviceStepper(ctl2, hp).single_pass(
        chunks, (tuple(c0[k][1] for k in ("master", "m", "v", "p16")),
                 tuple(c1[k][1] for k in ("master", "m", "v", "p16"))))
    # the bucket table under the control block, and the traffic twin
    ctl3 = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    t0, t1 = state(), state(dst_nan=True)
    zs.DeviceStepper(ctl3, hp).single_pass_buckets(
        zs.BucketSlices([(chunks, 0)]), (tuple(t0[k][1] for k in ("master", "m", "v", "p16")),
                                         tuple(t1[k][1] for k in ("master", "m", "v", "p16"))))
    tw_src, tw_dst = state(), state(dst_nan=True)
    zt.zero_traffic_twin(chunks, *(tw_src[k][1] for k in ("master", "m", "v")),
                         *(tw_dst[k][1] for k in ("master", "m", "v", "p16")))
    # the fp16 mean and the accumulator
    mbuf, mean = guarded(nn, torch.float16, dev)
    zs.zero_reduce_mean_fp16(chunks, mean, w.loss_scale, *flags(dev))
    abuf, acc = guarded(nn, torch.float32, dev)
    a16buf, amean = guarded(nn, torch.float16, dev)
    for i, c in enumerate(chunks):
        zs.zero_accumulate_chunk(c, i, N, acc, amean)
    torch.cuda.synchronize()
    for label, group in (("in place", s), ("out of place", dst), ("bucket table", bdst),
                         ("control two-pass", cs), ("control single pass", c1),
                         ("control bucket table", t1), ("traffic twin", tw_dst)):
        for k, (buf, _) in group.items():
            _assert_guards(buf, nn, f"{label} {k}")
    _assert_guards(mbuf, nn, "fp16 mean")
    _assert_guards(abuf, nn, "accumulator")
    _assert_guards(a16buf, nn, "accumulated mean")
    # and the outputs are the oracle's
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper,
                          w.loss_scale)
    for k, ref in (("master", want.master), ("m", want.m), ("v", want.v), ("p16", want.p16)):
        bits = np.uint16 if ref.dtype == np.float16 else np.uint32
        for label, group in (("in place", s), ("out of place", dst), ("bucket table", bdst),
                             ("control single pass", c1), ("control bucket table", t1)):
            got = group[k][1].cpu().numpy().view(bits)
            assert np.array_equal(got, ref.view(bits)), (label, k)
