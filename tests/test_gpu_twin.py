"""The fused step's traffic twin (a bandwidth reference, not part of the
step) writes exactly its definition, bit for bit, at ragged sizes and any N,
and nothing outside its output arrays.  The reference is computed here with
plain integer XORs on the host."""
import numpy as np
import pytest
import torch

import sharded_mixed_precision_step_amd as zs
from gpu_util import device, guarded, guards_intact

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("N", [1, 3, 8, 17])
@pytest.mark.parametrize("n", [1, 7, 8, 4097, 20_011])
def test_twin_writes_its_definition(n, N):
    dev = device()
    rng = np.random.default_rng(1000 * N + n)
    ch = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(N)]
    ins = [rng.integers(0, 1 << 32, n, dtype=np.uint32) for _ in range(3)]
    print(f"case: traffic twin n={n} N={N}", flush=True)
    d_ch = [torch.from_numpy(c.view(np.float16)).to(dev) for c in ch]
    d_in = [torch.from_numpy(x.view(np.float32)).to(dev) for x in ins]
    outs = [guarded(n, torch.float32, dev) for _ in range(3)] + [guarded(n, torch.float16, dev)]
    zs.zero_traffic_twin(d_ch, *d_in, *(t for _, t in outs))
    torch.cuda.synchronize()
    h = np.zeros(n, np.uint16)
    for c in ch:
        h ^= c
    h32 = h.astype(np.uint32)
    p, m, v = ins
    want = (p ^ m ^ v ^ h32, m ^ h32, v ^ h32, h ^ (p & 0xFFFF).astype(np.uint16))
    for k, ((buf, t), ref) in enumerate(zip(outs, want)):
        got = t.cpu().numpy().view(ref.dtype)
        assert np.array_equal(got, ref), k
        assert guards_intact(buf, n), k
