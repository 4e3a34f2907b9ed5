"""The allocation-free arrival fold (zero_accumulate_chunk_noalloc) against
zero_accumulate_chunk with a caller-owned accumulator: the same fp16 mean,
bit for bit, over two folds in a row on one GPU, the second over fewer
elements than the first (the library's accumulator keeps the first fold's
contents, which the second must not see), for a one-replica fold, and in a
HIP graph replayed with new contents.  The calls go through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import device

pytestmark = pytest.mark.gpu


def _chunks(n, N, seed, dev):
    return [torch.from_numpy(wl.host_fp16_grad(wl.seed_of(980, seed, i), n, 1e-4, 65536.0)).to(dev)
            for i in range(N)]


def _fold_noalloc(chunks, mean):
    N, n = len(chunks), chunks[0].numel()
    stream = torch.cuda.current_stream().cuda_stream
    for i, c in enumerate(chunks):
        rc = zs.lib.zero_accumulate_chunk_noalloc(c.data_ptr(), n, i, N,
                                                  mean.data_ptr() if i == N - 1 else None,
                                                  stream)
        assert rc == zs.ZERO_OK, zs.lib.zero_last_error_string().decode()


def _fold_with_acc(chunks, mean):
    N, n = len(chunks), chunks[0].numel()
    acc = torch.empty(n, dtype=torch.float32, device=chunks[0].device) if N > 1 else None
    for i, c in enumerate(chunks):
        zs.zero_accumulate_chunk(c, i, N, acc, mean if i == N - 1 else None)


@pytest.mark.parametrize("sizes", [((5_000_011, 8), (40_009, 3)),
                                   ((zs.ZERO_FOLD_SCRATCH_ELEMS, 4), (1_003, 8))])
def test_noalloc_fold_equals_the_fold_with_an_accumulator(sizes):
    dev = device()
    for k, (n, N) in enumerate(sizes):
        print(f"case: allocation-free fold n={n} N={N} (call {k} of 2)", flush=True)
        chunks = _chunks(n, N, 10 * k + N, dev)
        got = torch.full((n,), float("nan"), dtype=torch.float16, device=dev)
        want = torch.full((n,), float("nan"), dtype=torch.float16, device=dev)
        _fold_noalloc(chunks, got)
        _fold_with_acc(chunks, want)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        if n < 100_000:
            host = [c.cpu().numpy() for c in chunks]
            ref = ozs.accumulate_chunks(host)
            assert np.array_equal(got.cpu().numpy().view(np.uint16), ref.view(np.uint16))


def test_noalloc_single_replica_and_refusals():
    dev = device()
    c = _chunks(4_099, 1, 7, dev)
    got = torch.empty(4_099, dtype=torch.float16, device=dev)
    print("case: allocation-free fold, one replica", flush=True)
    _fold_noalloc(c, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), c[0].view(torch.int16))     # mean of one = itself
    big = torch.empty(zs.ZERO_FOLD_SCRATCH_ELEMS + 8, dtype=torch.float16, device=dev)
    with pytest.raises(zs.ZeroStepError) as e:
        zs.zero_accumulate_chunk_noalloc(big, 0, 2, None)
    assert e.value.code == zs.ZERO_ERANGE


def test_noalloc_fold_replays_in_a_hip_graph():
    """Code under HIP graph capture is among the callers the allocation-free
    fold is for: the N calls of one fold captured once and replayed three
    times, the chunks' contents redrawn eagerly between replays (with device
    synchronisations and unrelated eager work in between), every replay's
    fp16 mean equal, bit for bit, to the fold with an accumulator of the same
    contents."""
    dev = device()
    n, N = 70_001, 4
    chunks = _chunks(n, N, 300, dev)
    got = torch.empty(n, dtype=torch.float16, device=dev)
    want = torch.empty(n, dtype=torch.float16, device=dev)
    _fold_noalloc(chunks, got)          # the device's accumulator looked up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print(f"case: allocation-free fold n={n} N={N} captured in a HIP graph", flush=True)
    with torch.cuda.graph(graph):
        _fold_noalloc(chunks, got)
    torch.cuda.synchronize()
    for r in range(3):
        for c, f in zip(chunks, _chunks(n, N, 301 + r, dev)):
            c.copy_(f)
        got.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=dev).sum()      # unrelated eager work
        _fold_with_acc(chunks, want)
        torch.cuda.synchronize()
        print(f"case: allocation-free fold, graph replay {r}", flush=True)
        assert torch.isfinite(junk)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
