"""CPU oracle of gradient-bucket flattening.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; it shares no code with the HIP library.

Buckets: several parameters' gradients are grouped and reduced as one unit
(DP/DDP/FSDP walkthrough, pswp.cn/web/84187, section "DDP", the bucket
paragraph; ZeRO notes, rkmt.cn/news/44736, section "Deepspeed ZeRO-2", step
同步, where each finished bucket goes to the rank that owns it).  Reading
taken for the layout: tensors are laid end to end in the given order, each
start rounded up to a multiple of ``align`` elements, the total rounded up to
``pad_multiple`` (N * align, so the bucket splits into N equal shards), and
every gap and the tail hold zeros.

Pin: the layout's closed form (offsets are running sums of the rounded-up
sizes) on hand-worked cases stored under tests/golden.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def round_up(x: int, a: int) -> int:
    return -(-x // a) * a


def bucket_layout(numels: Sequence[int], align: int, pad_multiple: int) -> List[int]:
    """Element offset of each tensor, then the padded bucket length."""
    offsets = []
    end = 0
    for k in numels:
        start = round_up(end, align)
        offsets.append(start)
        end = start + int(k)
    offsets.append(round_up(end, pad_multiple) if pad_multiple > 0 else end)
    return offsets


def flatten(tensors: Sequence[np.ndarray], align: int, pad_multiple: int
            ) -> Tuple[np.ndarray, List[int]]:
    offsets = bucket_layout([t.size for t in tensors], align, pad_multiple)
    bucket = np.zeros(offsets[-1], dtype=np.float16)
    for t, o in zip(tensors, offsets):
        flat = t.reshape(-1)
        for j in range(0, flat.size, 1 << 22):
            piece = flat[j:j + (1 << 22)]
            bucket[o + j:o + j + piece.size] = piece
    return bucket, offsets
