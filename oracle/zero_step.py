"""CPU oracle of the per-rank ZeRO-1/2 mixed-precision shard step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never does.  It shares no
code with the HIP library and imports nothing from it.

What it computes, in the order the sources give it:

* ZeRO notes (rkmt.cn/news/44736), section "Deepspeed ZeRO-1", step
  "同步" (sync): every owner ends up holding the *mean* of the N replicas'
  gradients for its 1/N of the parameters.
* Same page and section, step "更新" (update): the fp16 mean is taken to fp32
  (not stored), scaled (read: divided by the loss scale), the fp32 first and
  second moments are updated, then the fp32 master weights, then the owner's
  fp16 parameters.  Section "Deepspeed ZeRO-2", step "更新", says the bucketed
  variant updates exactly as ZeRO-1 does.
* DP/DDP/FSDP walkthrough (pswp.cn/web/84187), section "DDP", ring example:
  the reduced value of a chunk is the plain sum a0+a1+a2 of the replicas.
* Same ZeRO notes page, section "Deepspeed ZeRO" (memory): params and grads
  are fp16, and the moments and master copy are fp32.

Readings taken where the pages leave a step open (each one is listed with its
reason in the design notes):

* the replica sum is taken in fp32, in the fixed order 0..N-1, and the mean
  is not rounded to fp16 in between;
* mean = s / N and g = mean / S are two correctly rounded fp32 divisions;
* the non-finite check is made on g, in fp32;
* the optimizer is Adam with Kingma & Ba's bias correction (Adam, Alg. 1),
  eps added after the square root, with decoupled weight decay as in
  Loshchilov & Hutter (AdamW, Alg. 2): p <- p - lr*wd*p, applied before the
  Adam term; ``decoupled_wd=False`` instead folds wd*p into g (L2 Adam);
* bias corrections are 1 - beta^t evaluated in fp64 from the fp32 betas and
  rounded once to fp32; c1 = 1 - beta1 and c2 = 1 - beta2 are fp32 ops;
* every other operation is one IEEE fp32 operation, rounded to nearest even,
  with no fused multiply-add;
* the new fp16 params are the new master rounded to nearest even binary16;
* the squared gradient norm is the sum of the exact fp64 squares of g,
  accumulated in fp64 in ascending index order.

The page-literal split (the owner stores its gradient mean as fp16, then
updates from it) is ``replica_mean_fp16`` / ``accumulate_chunks`` followed by
``shard_step_from_fp16_mean``.

Pins (tests that tie this module to facts outside itself):
replica sum -> brute-force ring simulation and the worked 3-GPU example;
mean and unscale -> identical-replica invariant (exact closed form);
non-finite flag -> planted inf/NaN and an fp32-overflowing unscale;
squared norm -> constant-gradient closed form and an exactly rounded sum;
moments and master -> first-step closed form, zero-gradient and lr = 0
invariants, and the N = 1, S = 1 special case against torch.optim.AdamW;
fp16 writeback -> IEEE binary16 bit patterns and torch's own rounding;
clip coefficient -> torch.nn.utils.clip_grad_norm_ in fp64, and the
constant-gradient closed form;
fp16 mean -> exact rational means rounded by hand-coded binary16 rounding on
exactly summable inputs, and identical replicas (the fp16 mean is then the
replica itself, and the split equals the fused step bit for bit).

Parity unpinned: the order of ``replica_sum`` where the sum is not exact.
Its value is pinned wherever every order gives the same bits, and bounded
elsewhere (within the recursive-summation error bound of the exact sum);
the fixed order 0..N-1 is a reading, since the ring's rotating order would
round differently and no source decides.  The squared norm is pinned as
arithmetic only; the pages define no norm.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Sequence

import numpy as np

F32 = np.float32


def widen(chunk: np.ndarray) -> np.ndarray:
    """fp16 -> fp32.  Every binary16 value is exact in binary32."""
    assert chunk.dtype == np.float16
    return chunk.astype(np.float32)


def replica_sum(chunks: Sequence[np.ndarray]) -> np.ndarray:
    """s = ((x_0 + x_1) + ...) + x_{N-1}, each addition rounded to fp32.

    The reduction a scatter-reduce leaves on the chunk's owner (ring example
    of the DDP section, DP/DDP/FSDP walkthrough), in fixed replica order.
    """
    s = widen(chunks[0])
    for x in chunks[1:]:
        s = s + widen(x)
    return s


def replica_mean(s: np.ndarray, n_replicas: int) -> np.ndarray:
    """The owner's averaged gradient, s / N (ZeRO notes, ZeRO-1, sync)."""
    return s / F32(n_replicas)


def unscale(mean: np.ndarray, loss_scale: float) -> np.ndarray:
    """Undo the loss scaling: g = mean / S (ZeRO notes, ZeRO-1, update)."""
    return mean / F32(loss_scale)


def unscaled_grad(chunks: Sequence[np.ndarray], loss_scale: float) -> np.ndarray:
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        return unscale(replica_mean(replica_sum(chunks), len(chunks)), loss_scale)


def nonfinite(g: np.ndarray) -> bool:
    """True if any element of g is +inf, -inf or NaN."""
    return bool(np.any(~np.isfinite(g)))


def grad_sqnorm(g: np.ndarray, start: float = 0.0) -> float:
    """sum_j g_j^2 with exact fp64 squares, accumulated in ascending j.

    ``start`` continues an earlier partial sum, so that a shard processed in
    slices gives the same value as one pass.
    """
    sq = np.square(g.astype(np.float64))
    acc = np.cumsum(np.concatenate([np.array([start], np.float64), sq]))
    return float(acc[-1])


@dataclasses.dataclass(frozen=True)
class AdamConstants:
    lr: np.float32
    beta1: np.float32
    beta2: np.float32
    c1: np.float32          # 1 - beta1
    c2: np.float32          # 1 - beta2
    bc1: np.float32         # 1 - beta1^t (1 without bias correction)
    bc2: np.float32         # 1 - beta2^t
    eps: np.float32
    wd: np.float32
    lrwd: np.float32        # lr * wd
    decoupled_wd: bool


def adam_constants(hyper) -> AdamConstants:
    """Per-step scalars, from fp32 hyperparameters and the 1-based step t."""
    b1, b2 = F32(hyper.beta1), F32(hyper.beta2)
    t = int(hyper.step)
    if hyper.bias_correction:
        bc1 = F32(1.0 - float(b1) ** t)
        bc2 = F32(1.0 - float(b2) ** t)
    else:
        bc1 = bc2 = F32(1.0)
    lr, wd = F32(hyper.lr), F32(hyper.weight_decay)
    return AdamConstants(lr=lr, beta1=b1, beta2=b2, c1=F32(1.0) - b1,
                         c2=F32(1.0) - b2, bc1=bc1, bc2=bc2, eps=F32(hyper.eps),
                         wd=wd, lrwd=lr * wd, decoupled_wd=bool(hyper.decoupled_wd))


def adamw_update(g, master, m, v, hyper):
    """One Adam/AdamW update of the shard from the fp32 gradient g.

    Order (ZeRO notes, ZeRO-1, update): moments first, then the fp32 master
    weights, then the fp16 params taken from the new master.
    Returns (master', m', v', p16').
    """
    k = adam_constants(hyper)
    with np.errstate(over="ignore", invalid="ignore", under="ignore",
                     divide="ignore"):
        if not k.decoupled_wd:
            g = g + k.wd * master
        m1 = k.beta1 * m + k.c1 * g
        v1 = k.beta2 * v + (k.c2 * g) * g
        m_hat = m1 / k.bc1
        v_hat = v1 / k.bc2
        u = m_hat / (np.sqrt(v_hat) + k.eps)
        p = master - k.lrwd * master if k.decoupled_wd else master
        master1 = p - k.lr * u
        p16 = master1.astype(np.float16)
    return master1, m1, v1, p16


@dataclasses.dataclass
class StepResult:
    overflow: bool
    sqnorm: float
    master: np.ndarray
    m: np.ndarray
    v: np.ndarray
    p16: np.ndarray


def step_from_grad(g, master, m, v, p16, hyper, sqnorm_start: float = 0.0) -> StepResult:
    """Flag, squared norm and (unless the flag is set) the AdamW update from
    the unscaled fp32 gradient g.  If any element of g is non-finite the step
    is skipped and the returned state equals the input state."""
    flag = nonfinite(g)
    sq = grad_sqnorm(g, sqnorm_start)
    if flag:
        return StepResult(True, sq, master.copy(), m.copy(), v.copy(), p16.copy())
    master1, m1, v1, p161 = adamw_update(g, master, m, v, hyper)
    return StepResult(False, sq, master1, m1, v1, p161)


def shard_step(chunks, master, m, v, p16, hyper, loss_scale,
               sqnorm_start: float = 0.0) -> StepResult:
    """The whole per-rank step on one shard (or one slice of it).

    The overflow decision here is local to the given slice: a caller that
    splits a shard combines the slices' flags before acting on them.
    """
    return step_from_grad(unscaled_grad(chunks, loss_scale), master, m, v, p16, hyper,
                          sqnorm_start)


# --------------------------------------------------------------------------
# Gradient-norm clipping (not on the pages; the usual global-norm rule).
# --------------------------------------------------------------------------

CLIP_EPS = 1e-6


def clip_coefficient(sqnorm: float, max_norm: float) -> np.float32:
    """The factor that scales g so that its 2-norm is at most max_norm:
    min(1, max_norm / (sqrt(sum g^2) + 1e-6)), evaluated in fp64 from the fp64
    squared norm and rounded once to fp32.  max_norm <= 0 means no clipping
    (factor 1).  The norm is that of the unscaled mean gradient of the whole
    shard, taken before clipping."""
    if not max_norm > 0.0:
        return F32(1.0)
    coef = float(max_norm) / (math.sqrt(float(sqnorm)) + CLIP_EPS)
    return F32(min(1.0, coef))


def shard_step_clipped(chunks, master, m, v, p16, hyper, loss_scale, max_norm) -> StepResult:
    """The two-pass step with clipping: the flag and squared norm of g first,
    then (unless the step is skipped) the update from fl32(g * coef)."""
    g = unscaled_grad(chunks, loss_scale)
    flag = nonfinite(g)
    sq = grad_sqnorm(g)
    if flag:
        return StepResult(True, sq, master.copy(), m.copy(), v.copy(), p16.copy())
    master1, m1, v1, p161 = adamw_update(g * clip_coefficient(sq, max_norm), master, m, v, hyper)
    return StepResult(False, sq, master1, m1, v1, p161)


# --------------------------------------------------------------------------
# The page-literal split: the owner first holds the mean in fp16, then updates.
# --------------------------------------------------------------------------

def replica_mean_fp16(chunks: Sequence[np.ndarray]) -> np.ndarray:
    """The owner's gradient mean as the ZeRO notes' ZeRO-1 sync step leaves
    it: in fp16.  Reading taken for how it is formed: the replica sum in fp32
    in fixed order, divided by N in fp32, then rounded to nearest-even
    binary16 once."""
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        return replica_mean(replica_sum(chunks), len(chunks)).astype(np.float16)


def accumulate_chunks(chunks: Sequence[np.ndarray]) -> np.ndarray:
    """The same fp16 mean, formed as chunks arrive one at a time: an fp32
    accumulator starts at the first chunk, each later chunk is added to it
    (one fp32 addition per element), and after the last one the accumulator
    is divided by N and rounded to binary16."""
    acc = widen(chunks[0])
    for x in chunks[1:]:
        acc = acc + widen(x)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        return (acc / F32(len(chunks))).astype(np.float16)


def shard_step_from_fp16_mean(mean16, master, m, v, p16, hyper, loss_scale,
                              sqnorm_start: float = 0.0) -> StepResult:
    """ZeRO notes, ZeRO-1 update step, from the stored fp16 mean: fp16 to fp32
    (not stored), scale (divide by S), fp32 moments, fp32 master weights,
    fp16 params."""
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        g = unscale(widen(mean16), loss_scale)
    return step_from_grad(g, master, m, v, p16, hyper, sqnorm_start)


def check_only(chunks, loss_scale, sqnorm_start: float = 0.0):
    """Overflow flag and squared norm without the update: (flag, sqnorm)."""
    g = unscaled_grad(chunks, loss_scale)
    return nonfinite(g), grad_sqnorm(g, sqnorm_start)
