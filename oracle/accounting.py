"""Memory and traffic accounting of the mixed-precision ZeRO step.

TEST INFRASTRUCTURE.  It pins the byte model used for the roofline.

ZeRO notes (rkmt.cn/news/44736), section "Deepspeed ZeRO" (memory): a DDP
replica holds per parameter an fp16 param (2 B), an fp16 gradient (2 B) and
12 B of optimizer state (4 B first moment, 4 B second moment, 4 B fp32
param), 16 B in all.  ZeRO-1 shards the optimizer state, ZeRO-2 also the
gradients, ZeRO-3 also the parameters.  Traffic: ring all-reduce sends N-1
messages of psi/N per phase (DDP section), ZeRO-1 and -2 keep DDP's volume,
ZeRO-3 adds a parameter broadcast in backward for 3 psi (summary).
"""
from __future__ import annotations

FP16_PARAM, FP16_GRAD = 2, 2
FP32_M, FP32_V, FP32_MASTER = 4, 4, 4


def ddp_bytes_per_param() -> int:
    return FP16_PARAM + FP16_GRAD + FP32_M + FP32_V + FP32_MASTER


def zero_bytes_per_param(stage: int, n_gpus: int) -> float:
    """Per-GPU bytes per model parameter under ZeRO stage 0..3."""
    opt = FP32_M + FP32_V + FP32_MASTER
    if stage == 0:
        return FP16_PARAM + FP16_GRAD + opt
    if stage == 1:
        return FP16_PARAM + FP16_GRAD + opt / n_gpus
    if stage == 2:
        return FP16_PARAM + (FP16_GRAD + opt) / n_gpus
    if stage == 3:
        return (FP16_PARAM + FP16_GRAD + opt) / n_gpus
    raise ValueError(stage)


def step_bytes_per_param(n_replicas: int) -> int:
    """HBM bytes the fused shard step moves per owned param: N fp16 replica
    gradients read, fp32 m, v, master read and written, fp16 param written."""
    return n_replicas * FP16_GRAD + 2 * (FP32_M + FP32_V + FP32_MASTER) + FP16_PARAM


def check_bytes_per_param(n_replicas: int) -> int:
    """The overflow check alone reads the N fp16 replica gradients."""
    return n_replicas * FP16_GRAD


def ring_allreduce_elements_sent_per_rank(psi: int, n_gpus: int) -> float:
    """2 (N - 1) psi / N: N - 1 messages of psi / N in each of two phases."""
    return 2 * (n_gpus - 1) * psi / n_gpus
