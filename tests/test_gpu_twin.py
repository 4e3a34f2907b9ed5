"""The benchmark's measurement aids (libzerotwin.so): the fused step's
traffic twin writes exactly its definition, bit for bit, at ragged sizes and
any N, and nothing outside its output arrays; the read-only stream folds
every word it reads.  The references are plain integer XORs on the host."""
import numpy as np
import pytest
import torch

from gpu_util import device, guarded, guards_intact
from sharded_mixed_precision_step_amd import twin as zt

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
    zt.zero_traffic_twin(d_ch, *d_in, *(t for _, t in outs))
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


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1_000_003])
def test_stream_read_folds_every_word(nbytes):
    """The read-only stream XORs every 32-bit word it reads into the sink."""
    dev = device()
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    print(f"case: stream read {nbytes} bytes", flush=True)
    src = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    zt.zero_stream_read(src, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
