"""A long run: 600 device-controlled single-pass steps on a small ragged
shard (20,011 params, N = 4), fresh gradients every step, an overflow
planted every 97th step, the scale growing every 50 clean steps, and the
bias-correction table rebased every 64 steps, against the oracle's 600
steps of the same inputs: t, the scale, the counters and every bit of the
state agree at every 50th step and at the end."""
import numpy as np
import pytest
import torch

import oracle.loss_scale as ols
import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import device

pytestmark = pytest.mark.gpu

N, n, STEPS = 4, 20_011, 600


def test_six_hundred_steps_follow_the_oracle():
    dev = device()
    base = wl.LLAMA3_8B_SHARD
    w = wl.ShardWorkload(name="long_run", wid=base.wid, n=n, n_replicas=N, grad_sigma=1e-4,
                         loss_scale=1024.0, hyper=base.hyper.replace(step=1), m_sigma=0.0,
                         v_sigma=0.0)
    h = wl.host_shard(w, n=n, offset_seed=970)
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    copies = (a, tuple(torch.empty_like(x) for x in a))
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale, growth_interval=50),
                         w.hyper.step, dev)
    step = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).prepare_single_pass
    chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    run = step(chunks, copies)
    os_ = ols.ScalerState(scale=w.loss_scale, growth_interval=50)
    state, t = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step
    scales = set()
    for k in range(STEPS):
        S = os_.scale
        g = [wl.host_fp16_grad(wl.seed_of(w.wid, 971, k, i), n, w.grad_sigma, S)
             for i in range(N)]
        if k % 97 == 96:
            g[k % N][(31 * k) % n] = np.float16(np.inf)
        for c, src in zip(chunks, g):
            c.copy_(torch.from_numpy(src))
        run()
        want = ozs.shard_step(g, *state, w.hyper.replace(step=t), S)
        if not ols.update_loss_scale(os_, want.overflow):
            t += 1
            state = (want.master, want.m, want.v, want.p16)
        scales.add(os_.scale)
        if k % 50 == 49 or k == STEPS - 1:
            c = zs.control_read(ctl)
            print(f"case: long run step {k + 1}: t={c.step} S={c.scale}", flush=True)
            assert c.error == 0 and c.step == t and c.scale == np.float32(os_.scale)
            assert c.good_steps == os_.good_steps and c.skipped_steps == os_.skipped_steps
            for name, x, ref in zip(("master", "m", "v", "p16"), copies[c.cur], state):
                bits = np.uint16 if ref.dtype == np.float16 else np.uint32
                assert np.array_equal(x.cpu().numpy().view(bits), ref.view(bits)), (k, name)
    assert os_.skipped_steps == STEPS // 97 and t == w.hyper.step + STEPS - STEPS // 97
    assert max(scales) == 2 * w.loss_scale and min(scales) == w.loss_scale  # grew and backed off
