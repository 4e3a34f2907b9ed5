"""Helpers of the GPU parity tests: device copies, running the step through
the C ABI, and element-by-element comparison with the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sharded_mixed_precision_step_amd as zs

REL, ABS = 1e-6, 1e-9          # fp32 master/m/v: 1e-6 relative or 1e-9 absolute
MAX_ULP = 16                   # diagnostic bound on fp32 ulp distance


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(h: dict, dev) -> dict:
    return dict(chunks=[torch.from_numpy(c).to(dev) for c in h["chunks"]],
                master=torch.from_numpy(h["master"]).to(dev),
                m=torch.from_numpy(h["m"]).to(dev), v=torch.from_numpy(h["v"]).to(dev),
                p16=torch.from_numpy(h["p16"]).to(dev))


def flags(dev):
    return (torch.zeros(1, dtype=torch.int32, device=dev),
            torch.zeros(1, dtype=torch.float64, device=dev))


def run_check_then_step(d: dict, hyper, loss_scale: float, stream=None):
    """The clean-step launch sequence: the overflow check (flag and squared
    norm), then the fused step without reductions.  Returns (flag, sqnorm)."""
    dev = d["master"].device
    fl, sq = flags(dev)
    zs.zero_overflow_check(d["chunks"], loss_scale, fl, sq, stream=stream)
    zs.zero_shard_step(d["chunks"], loss_scale, d["master"], d["m"], d["v"], d["p16"],
                       zs.adamw_params(hyper), stream=stream)
    torch.cuda.synchronize()
    return int(fl.item()), float(sq.item())


def ordered32(x: np.ndarray) -> np.ndarray:
    b = np.asarray(x, np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7fffffff), b)


def ordered16(x: np.ndarray) -> np.ndarray:
    b = np.asarray(x, np.float16).view(np.int16).astype(np.int64)
    return np.where(b < 0, -(b & 0x7fff), b)


def ulp32(a, b) -> np.ndarray:
    return np.abs(ordered32(a) - ordered32(b))


def ulp16(a, b) -> np.ndarray:
    return np.abs(ordered16(a) - ordered16(b))


def assert_fp32_close(name: str, got: np.ndarray, want: np.ndarray, max_ulp=MAX_ULP) -> int:
    """1e-6 relative or 1e-9 absolute per element, and (unless max_ulp is
    None) at most max_ulp fp32 ulps; returns the largest ulp distance."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, name
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{name}: NaN positions differ"
    fin = ~np.isnan(want)
    g64, w64 = got[fin].astype(np.float64), want[fin].astype(np.float64)
    err = np.abs(g64 - w64)
    bad = ~(err <= np.maximum(REL * np.abs(w64), ABS))
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} outside 1e-6 rel / 1e-9 abs; "
                           f"first at {np.flatnonzero(bad)[:5]}")
    u = int(ulp32(got[fin], want[fin]).max()) if fin.any() else 0
    if max_ulp is not None:
        assert u <= max_ulp, f"{name}: {u} ulp"
    return u


def assert_fp16_close(name: str, got: np.ndarray, want: np.ndarray) -> int:
    u = int(ulp16(got, want).max()) if got.size else 0
    assert u <= 1, f"{name}: fp16 params differ by {u} ulp"
    return u


def assert_matches_oracle(d: dict, want, label: str = "", max_ulp=MAX_ULP) -> dict:
    """Compare the device state after a step with an oracle StepResult."""
    ulps = {}
    for k, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
        ulps[k] = assert_fp32_close(f"{label}{k}", d[k].cpu().numpy(), ref, max_ulp)
    ulps["p16"] = assert_fp16_close(f"{label}p16", d["p16"].cpu().numpy(), want.p16)
    return ulps


GUARD = 4096          # bytes of canary on each side of a guarded array
CANARY = 0xA5


def guarded(numel: int, dtype, dev, fill=None):
    """(buffer, tensor): a tensor of `numel` elements with GUARD bytes of the
    CANARY byte on either side, inside one 16-byte aligned buffer; the tensor
    is filled from `fill` if given."""
    esize = torch.empty(0, dtype=dtype).element_size()
    g = GUARD // esize
    buf = torch.empty(numel + 2 * g, dtype=dtype, device=dev)
    buf.view(torch.uint8).fill_(CANARY)
    t = buf[g:g + numel]
    if fill is not None:
        t.copy_(fill)
    return buf, t


def guards_intact(buf: torch.Tensor, numel: int) -> bool:
    """Both canary bands of a `guarded` buffer still hold CANARY."""
    raw = buf.view(torch.uint8)
    end = GUARD + numel * buf.element_size()
    return bool((raw[:GUARD] == CANARY).all()) and bool((raw[end:] == CANARY).all())

