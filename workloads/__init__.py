"""Seeded synthetic inputs for the per-rank ZeRO-1/2 mixed-precision shard step.

This module holds workload shapes, value distributions and seeds, and nothing
of the step's arithmetic: it draws random numbers, scales them to the stated
standard deviation and rounds fp16 arrays to binary16 on creation.  Both sides
of every parity check take their inputs from here: the CPU oracle gets host
arrays, the GPU path gets the same bits copied to the device (small cases), or
the GPU draws its own with the HIP generator in csrc/zero_gen.hip and the
oracle receives host copies of what it drew (full-size cases).

Workloads (the rank's shard at its real shape; N replicas of the gradient
shard stand in for the N ranks whose gradients are reduced onto this owner):

* ``tiny``              psi = 1,000,003, N = 3, loss scale 1024, first step.
* ``llama3_8b_shard``   8.03e9 params over N = 8 ranks, shard 1,003,750,000,
                        loss scale 65536, t = 1000, non-zero m and v.
* ``zero2_bucketed``    32 decoder layers of q,k,v,o [4096x4096],
                        gate,up,down [4096x14336], two [4096] norms, packed in
                        backward order into buckets of at most 5e7 elements.
* ``overflow``          the Llama-3-8B shard at 1/8 size with 0.01 % of the
                        gradient entries set to +inf, -inf and NaN in turn.
* ``llama70b_shard``    7.06e10 params over N = 16 ranks, shard 4,412,500,000,
                        streamed as 22 buckets of 2e8 and one of 1.25e7.

"N(0, s)" means mean 0 and standard deviation s throughout; m and v are the
absolute values of such draws (v must be non-negative for its square root).
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

ARRAY_GRAD, ARRAY_MASTER, ARRAY_M, ARRAY_V, ARRAY_INJECT = 0, 1, 2, 3, 4


def seed_of(*key: int) -> int:
    """A 63-bit seed from an integer tuple (workload id, array id, indices).

    Tuples map to independent streams, so no two arrays share a seed.
    """
    ss = np.random.SeedSequence([int(k) for k in key])
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


@dataclasses.dataclass(frozen=True)
class AdamWHyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1
    decoupled_wd: bool = True
    bias_correction: bool = True

    def replace(self, **kw) -> "AdamWHyper":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class ShardWorkload:
    """One rank's flat shard: N replica gradient chunks of n fp16 values each,
    and the fp32 master weights, first and second moments of those n params."""
    name: str
    wid: int                 # workload id, used in seeds
    n: int                   # params in this rank's shard
    n_replicas: int          # N, the number of ranks reducing onto the owner
    grad_sigma: float        # std of one replica's unscaled gradient
    loss_scale: float        # S
    hyper: AdamWHyper
    master_sigma: float = 0.02
    m_sigma: float = 0.0     # 0 means m starts at zero
    v_sigma: float = 0.0     # 0 means v starts at zero
    n_inject: int = 0        # entries of the N*n gradient values set non-finite
    buckets: Tuple[int, ...] = ()   # streamed bucket lengths (shard elements)

    def bytes_per_param_step(self) -> int:
        """Algorithmic HBM bytes of the fused step per param: N fp16 chunk reads,
        fp32 master, m, v read and written, fp16 param written."""
        return 2 * self.n_replicas + 24 + 2


TINY = ShardWorkload(
    name="tiny", wid=0, n=1_000_003, n_replicas=3, grad_sigma=1e-3,
    loss_scale=1024.0, hyper=AdamWHyper(step=1))

LLAMA3_8B_SHARD = ShardWorkload(
    name="llama3_8b_shard", wid=1, n=8_030_000_000 // 8, n_replicas=8,
    grad_sigma=1e-4, loss_scale=65536.0, hyper=AdamWHyper(step=1000),
    m_sigma=1e-4, v_sigma=1e-8)

OVERFLOW = ShardWorkload(
    name="overflow", wid=3, n=8_030_000_000 // 64, n_replicas=8,
    grad_sigma=1e-4, loss_scale=65536.0, hyper=AdamWHyper(step=1000),
    m_sigma=1e-4, v_sigma=1e-8, n_inject=8 * (8_030_000_000 // 64) // 10_000)

LLAMA70B_SHARD = ShardWorkload(
    name="llama70b_shard", wid=4, n=70_600_000_000 // 16, n_replicas=16,
    grad_sigma=1e-4, loss_scale=65536.0, hyper=AdamWHyper(step=5000),
    m_sigma=1e-4, v_sigma=1e-8,
    buckets=tuple([200_000_000] * 22 + [12_500_000]))

WORKLOADS = {w.name: w for w in (TINY, LLAMA3_8B_SHARD, OVERFLOW, LLAMA70B_SHARD)}
# (the ZeRO-2 bucketed workload, ZERO2, is defined below with its bucket plan)


# ---------------------------------------------------------------------------
# ZeRO-2 bucketed workload: tensor list in backward order and bucket packing.
# ---------------------------------------------------------------------------

ZERO2_WID = 2
ZERO2_LAYERS = 32
ZERO2_HIDDEN = 4096
ZERO2_FFN = 14336
ZERO2_BUCKET_CAP = 50_000_000
ZERO2_ALIGN = 256
ZERO2_REPLICAS = 8


def zero2_tensors() -> List[Tuple[str, Tuple[int, ...]]]:
    """(name, shape) of every gradient tensor, in the order backward produces
    them: last layer first, and inside a layer the reverse of forward order."""
    h, f = ZERO2_HIDDEN, ZERO2_FFN
    per_layer_backward = [
        ("mlp.down", (h, f)), ("mlp.up", (h, f)), ("mlp.gate", (h, f)),
        ("ffn_norm", (h,)), ("attn.o", (h, h)), ("attn.v", (h, h)),
        ("attn.k", (h, h)), ("attn.q", (h, h)), ("attn_norm", (h,)),
    ]
    out = []
    for layer in reversed(range(ZERO2_LAYERS)):
        for nm, shape in per_layer_backward:
            out.append((f"layers.{layer}.{nm}", shape))
    return out


def _round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def zero2_bucket_plan(cap: int = ZERO2_BUCKET_CAP, align: int = ZERO2_ALIGN
                      ) -> List[List[int]]:
    """Greedy packing of whole tensors, in backward order, into buckets.

    A bucket is closed when the next tensor, started at the next multiple of
    ``align``, would end past ``cap``; a tensor larger than ``cap`` alone
    fills a bucket of its own.  Returns tensor indices per bucket.
    """
    sizes = [int(np.prod(s)) for _, s in zero2_tensors()]
    buckets: List[List[int]] = []
    cur: List[int] = []
    end = 0
    for k, sz in enumerate(sizes):
        start = _round_up(end, align) if cur else 0
        if cur and start + sz > cap:
            buckets.append(cur)
            cur, start = [], 0
        cur.append(k)
        end = start + sz
    if cur:
        buckets.append(cur)
    return buckets


ZERO2_GRAD_SIGMA = 1e-4
ZERO2_LOSS_SCALE = 65536.0
ZERO2_RANK = 3          # the rank whose shard the bucketed workload updates


# One rank's shard of the bucketed workload: slice ZERO2_RANK of every bucket.
# The 160 buckets are 96 of 58,720,256 elements (one MLP gradient each) and
# 64 of 33,558,528 (three attention-side gradients each) once tensor starts
# are aligned to 256 and lengths to 256 * 8, so the shard holds
# (96 * 58,720,256 + 64 * 33,558,528) / 8 = 973,111,296 params.
ZERO2 = ShardWorkload(
    name="zero2_bucketed", wid=ZERO2_WID, n=973_111_296, n_replicas=ZERO2_REPLICAS,
    grad_sigma=ZERO2_GRAD_SIGMA, loss_scale=ZERO2_LOSS_SCALE, hyper=AdamWHyper(step=1000),
    m_sigma=1e-4, v_sigma=1e-8)


def zero2_device_tensor(replica: int, k: int, device):
    """Replica ``replica``'s fp16 gradient of tensor ``k`` (flat), loss-scaled."""
    torch = _torch()
    numel = int(np.prod(zero2_tensors()[k][1]))
    t = torch.empty(numel, dtype=torch.float16, device=device)
    return device_fill_normal(t, seed_of(ZERO2_WID, 100 + replica, ARRAY_GRAD, k),
                              ZERO2_GRAD_SIGMA * ZERO2_LOSS_SCALE)


# ---------------------------------------------------------------------------
# Host (numpy) generators.
# ---------------------------------------------------------------------------

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def host_normal_f32(seed: int, n: int, sigma: float) -> np.ndarray:
    z = _rng(seed).standard_normal(n, dtype=np.float32)
    return z * np.float32(sigma)


def host_fp16_grad(seed: int, n: int, sigma: float, loss_scale: float
                   ) -> np.ndarray:
    """fp16(N(0, sigma) * loss_scale): a loss-scaled replica gradient."""
    z = _rng(seed).standard_normal(n, dtype=np.float32)
    with np.errstate(over="ignore"):
        return (z * np.float32(sigma * loss_scale)).astype(np.float16)


def host_shard(w: ShardWorkload, n: int | None = None, offset_seed: int = 0):
    """Host arrays for workload ``w`` (optionally its first-``n``-style
    miniature with the same distributions).  Returns a dict with
    ``chunks`` (list of N fp16 arrays), ``master``, ``m``, ``v`` (fp32) and
    ``p16`` (fp16 copy of master, the replica's current fp16 params)."""
    n = w.n if n is None else n
    key = (w.wid, offset_seed)
    chunks = [host_fp16_grad(seed_of(*key, ARRAY_GRAD, i), n, w.grad_sigma,
                             w.loss_scale) for i in range(w.n_replicas)]
    master = host_normal_f32(seed_of(*key, ARRAY_MASTER), n, w.master_sigma)
    m = (np.abs(host_normal_f32(seed_of(*key, ARRAY_M), n, w.m_sigma))
         if w.m_sigma else np.zeros(n, np.float32))
    v = (np.abs(host_normal_f32(seed_of(*key, ARRAY_V), n, w.v_sigma))
         if w.v_sigma else np.zeros(n, np.float32))
    return dict(chunks=chunks, master=master, m=m, v=v,
                p16=master.astype(np.float16))


def injection_sites(w: ShardWorkload, n: int | None = None, count: int | None = None,
                    offset_seed: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Seeded distinct positions over the N*n gradient entries, as (chunk,
    element, value) with values +inf, -inf, NaN in turn by draw order."""
    n = w.n if n is None else n
    count = w.n_inject if count is None else count
    total = w.n_replicas * n
    rng = _rng(seed_of(w.wid, offset_seed, ARRAY_INJECT))
    q = rng.choice(total, size=min(count, total), replace=False)
    kinds = np.array([np.inf, -np.inf, np.nan], dtype=np.float16)
    vals = kinds[np.arange(q.size) % 3]
    return (q // n).astype(np.int64), (q % n).astype(np.int64), vals


def exactly_summable_fp16(seed: int, n: int, bound_log2: int = 8) -> np.ndarray:
    """fp16 multiples of 2^-10 in [-2^bound_log2, 2^bound_log2] (with the
    default bound, |k| <= 2^18 units of 2^-10): any sum of up to 64 of them
    is a multiple of 2^-10 below 2^24 units, hence exact in fp32 in any order."""
    k = _rng(seed).integers(-(1 << (bound_log2 + 10)) + 1, 1 << (bound_log2 + 10),
                            size=n)
    return np.ldexp(k.astype(np.float64), -10).astype(np.float16)


# ---------------------------------------------------------------------------
# Device generators for full-size workloads: HIP kernels of their own
# (workloads/csrc/zero_gen.hip, built into workloads/libzerogen.so) draw
# Philox-4x32-10 normals straight into device memory; torch only allocates
# the tensors and supplies the stream.
# ---------------------------------------------------------------------------

_GEN = None


def _torch():
    import torch
    return torch


def _gen():
    """libzerogen.so, loaded on first use (after torch, whose HIP runtime it
    shares)."""
    global _GEN
    if _GEN is None:
        import ctypes
        import os
        _torch()
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzerogen.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        lib.zero_gen_philox.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
        lib.zero_gen_normal.argtypes = [vp, i32, i64, u64, ctypes.c_float, i32, vp]
        lib.zero_gen_to_fp16.argtypes = [vp, vp, i64, vp]
        lib.zero_gen_scatter_fp16.argtypes = [vp, i64, vp, vp, i64, vp]
        for name in ("zero_gen_philox", "zero_gen_normal", "zero_gen_to_fp16",
                     "zero_gen_scatter_fp16"):
            getattr(lib, name).restype = ctypes.c_int
        _GEN = lib
    return _GEN


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def device_philox(ctr_key, device):
    """The four output words of Philox-4x32-10 for counter ctr_key[0:4] and
    key ctr_key[4:6], computed on the device (for known-answer tests)."""
    import ctypes
    torch = _torch()
    out = torch.zeros(4, dtype=torch.int32, device=device)
    words = (ctypes.c_uint32 * 6)(*[int(x) & 0xFFFFFFFF for x in ctr_key])
    _ok(_gen().zero_gen_philox(out.data_ptr(), words, _stream()), "zero_gen_philox")
    return [int(x) & 0xFFFFFFFF for x in out.cpu().tolist()]


def device_fill_normal(out, seed: int, sigma: float, absolute: bool = False):
    """Fill ``out`` (contiguous fp32 or fp16 device tensor) with N(0, sigma)
    draws of stream ``seed`` (their absolute values if ``absolute``), rounded
    to out's dtype."""
    torch = _torch()
    if not out.is_contiguous() or out.dtype not in (torch.float32, torch.float16):
        raise TypeError("out must be a contiguous fp32 or fp16 device tensor")
    _ok(_gen().zero_gen_normal(out.data_ptr(), int(out.dtype == torch.float16), out.numel(),
                               int(seed), float(sigma), int(bool(absolute)), _stream()),
        "zero_gen_normal")
    return out


def device_state(w: ShardWorkload, device, n: int | None = None, offset_seed: int = 0):
    """Device fp32 master, m, v and the fp16 params for workload ``w``."""
    torch = _torch()
    n = w.n if n is None else n
    key = (w.wid, offset_seed)
    master = torch.empty(n, dtype=torch.float32, device=device)
    device_fill_normal(master, seed_of(*key, ARRAY_MASTER), w.master_sigma)
    m = torch.zeros(n, dtype=torch.float32, device=device)
    v = torch.zeros(n, dtype=torch.float32, device=device)
    if w.m_sigma:
        device_fill_normal(m, seed_of(*key, ARRAY_M), w.m_sigma, absolute=True)
    if w.v_sigma:
        device_fill_normal(v, seed_of(*key, ARRAY_V), w.v_sigma, absolute=True)
    p16 = torch.empty(n, dtype=torch.float16, device=device)
    _ok(_gen().zero_gen_to_fp16(master.data_ptr(), p16.data_ptr(), n, _stream()),
        "zero_gen_to_fp16")
    return dict(master=master, m=m, v=v, p16=p16)


def device_chunks(w: ShardWorkload, device, n: int | None = None, offset_seed: int = 0,
                  loss_scale: float | None = None, out=None):
    """The N replica gradient chunks of ``w`` (fp16(N(0, sigma) * S)), drawn
    into ``out`` (a list of N device fp16 tensors) if given."""
    torch = _torch()
    n = w.n if n is None else n
    S = w.loss_scale if loss_scale is None else loss_scale
    key = (w.wid, offset_seed)
    if out is None:
        out = [torch.empty(n, dtype=torch.float16, device=device) for _ in range(w.n_replicas)]
    for i, c in enumerate(out):
        device_fill_normal(c[:n], seed_of(*key, ARRAY_GRAD, i), w.grad_sigma * S)
    return out


def device_shard(w: ShardWorkload, device, n: int | None = None, offset_seed: int = 0):
    """Device tensors for workload ``w``: N fp16 chunks, fp32 master/m/v and
    the fp16 params.  All are separate allocations (16-byte aligned)."""
    d = device_state(w, device, n=n, offset_seed=offset_seed)
    d["chunks"] = device_chunks(w, device, n=n, offset_seed=offset_seed)
    return d


def device_inject(chunks: Sequence, sites) -> None:
    """Write the non-finite values of ``injection_sites`` into device chunks."""
    torch = _torch()
    ci, ei, vals = sites
    for c in range(len(chunks)):
        sel = ci == c
        if not sel.any():
            continue
        idx = torch.from_numpy(np.ascontiguousarray(ei[sel])).to(chunks[c].device)
        val = torch.from_numpy(np.ascontiguousarray(vals[sel]).view(np.int16)).to(
            chunks[c].device)
        _ok(_gen().zero_gen_scatter_fp16(chunks[c].data_ptr(), chunks[c].numel(),
                                         idx.data_ptr(), val.data_ptr(), idx.numel(),
                                         _stream()), "zero_gen_scatter_fp16")
        torch.cuda.current_stream().synchronize()   # idx and val are freed on return
