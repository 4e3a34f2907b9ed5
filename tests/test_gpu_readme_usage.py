"""The usage example of README.md runs as written: its Python block is taken
from the file and executed on a small shard (40,009 params, N = 8), and the
state it leaves current is the oracle's step of that shard."""
import os
import re

import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import workloads as wl
from gpu_util import device

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_usage_block_runs_and_matches_the_oracle():
    dev = device()
    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), re.S)
    assert len(blocks) == 1
    w = wl.LLAMA3_8B_SHARD
    n = 40_009
    h = wl.host_shard(w, n=n, offset_seed=960)
    env = {"chunks": [torch.from_numpy(c).to(dev) for c in h["chunks"]]}
    for k, name in (("master", "master"), ("m", "m"), ("v", "v"), ("p16", "p16")):
        env[name] = torch.from_numpy(h[k]).to(dev)
    print("case: README usage block, n=40009 N=8", flush=True)
    exec(blocks[0], env)                       # the example as printed
    torch.cuda.synchronize()
    # the example's hyperparameters: lr 1e-3, betas (0.9, 0.999), eps 1e-8,
    # wd 0.01, t = 1, AdamW with bias correction; S = 65536
    hyper = wl.AdamWHyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
                          step=1)
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], hyper, 65536.0)
    assert not want.overflow
    for name, x, ref in zip(("master", "m", "v", "p16"), env["state"],
                            (want.master, want.m, want.v, want.p16)):
        bits = np.uint16 if ref.dtype == np.float16 else np.uint32
        assert np.array_equal(x.cpu().numpy().view(bits), ref.view(bits)), name
