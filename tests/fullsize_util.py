"""Element-by-element comparison of a device step with the CPU oracle at full
workload sizes: the shard is cut into slices of 2^24 params, each slice is
copied to the host and recomputed by the oracle on a thread pool (numpy
releases the GIL), and the device result must equal the oracle bit for bit
(and so also meet the 1e-6 relative / 1e-9 absolute and 1-ulp fp16 bars).
The oracle's inputs are host copies of the generated inputs, never of a
kernel's output."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle.zero_step as ozs
from gpu_util import assert_fp16_close, assert_fp32_close

PIECE = 1 << 24


def threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _host(t: torch.Tensor, a: int, b: int) -> np.ndarray:
    return t[a:b].cpu().numpy()


def compare_with_oracle(chunks, state_in, state_out, hyper, loss_scale, label="",
                        keep_expected=False, piece=PIECE):
    """chunks: N device fp16 tensors; state_in: (master, m, v, p16) before the
    step; state_out: the same four after it.  Returns (overflow, sqnorm,
    expected) where expected holds the oracle's host arrays if asked for."""
    n = chunks[0].numel()
    count = (n + piece - 1) // piece
    expected = ([np.empty(n, np.float32) for _ in range(3)] + [np.empty(n, np.float16)]
                if keep_expected else None)

    def work(k):
        a, b = k * piece, min(n, (k + 1) * piece)
        ch = [_host(c, a, b) for c in chunks]
        st = [_host(t, a, b) for t in state_in]
        want = ozs.shard_step(ch, *st, hyper, loss_scale)
        got = [_host(t, a, b) for t in state_out]
        tag = f"{label}[{a}:{b}] "
        if not want.overflow:
            for name, g, ref in zip(("master", "m", "v"), got[:3], (want.master, want.m, want.v)):
                if not np.array_equal(g.view(np.uint32), ref.view(np.uint32)):
                    assert_fp32_close(tag + name, g, ref)
                    raise AssertionError(f"{tag}{name}: within tolerance but not bit-exact")
            if not np.array_equal(got[3].view(np.uint16), want.p16.view(np.uint16)):
                assert_fp16_close(tag + "p16", got[3], want.p16)
                raise AssertionError(f"{tag}p16: within 1 ulp but not bit-exact")
        if expected is not None:
            for dst, src in zip(expected, (want.master, want.m, want.v, want.p16)):
                dst[a:b] = src
        return want.overflow, want.sqnorm

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(work, range(count)))
    overflow = any(r[0] for r in res)
    sqnorm = float(np.sum(np.array([r[1] for r in res], np.float64)))
    return overflow, sqnorm, expected


def compare_with_expected(state_out, expected, label="", piece=PIECE):
    """The device state against oracle results kept from an earlier compare."""
    n = state_out[0].numel()
    count = (n + piece - 1) // piece

    def work(k):
        a, b = k * piece, min(n, (k + 1) * piece)
        for name, t, ref in zip(("master", "m", "v", "p16"), state_out, expected):
            g = _host(t, a, b)
            bits = np.uint16 if g.dtype == np.float16 else np.uint32
            assert np.array_equal(g.view(bits), ref[a:b].view(bits)), f"{label}{name}[{a}:{b}]"

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(work, range(count)))


def oracle_check_only(chunks, loss_scale, piece=PIECE):
    """The oracle's overflow flag and squared norm over device chunks."""
    n = chunks[0].numel()
    count = (n + piece - 1) // piece

    def work(k):
        a, b = k * piece, min(n, (k + 1) * piece)
        return ozs.check_only([_host(c, a, b) for c in chunks], loss_scale)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(work, range(count)))
    return any(r[0] for r in res), float(np.sum(np.array([r[1] for r in res], np.float64)))


def rel_close(got: float, want: float, rel: float = 1e-6) -> bool:
    return abs(got - want) <= rel * abs(want)
