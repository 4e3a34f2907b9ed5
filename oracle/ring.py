"""Brute-force simulation of ring all-reduce (scatter-reduce + all-gather).

TEST INFRASTRUCTURE.  It pins the oracle's replica sum to the pages' ring.

DDP section of the ZeRO notes (rkmt.cn/news/44736): ring all-reduce has two
phases, scatter-reduce (chunks are passed on and added) and all-gather
(complete chunks are passed on and overwrite).  DP/DDP/FSDP walkthrough
(pswp.cn/web/84187), section "DDP", works it through for 3 GPUs holding
a_i, b_i, c_i: in the first round GPU0 sends a0 to GPU1, GPU1 sends b1 to
GPU2, GPU2 sends c2 to GPU0; in the second round the partial sums move one
more hop, leaving GPU0 with b0+b1+b2, GPU1 with c0+c1+c2, GPU2 with a0+a1+a2;
the all-gather then spreads the complete chunks.

Generalised to N ranks: in scatter-reduce round k (k = 0..N-2) rank r sends
its chunk (r - k) mod N to rank r+1, which adds what it receives in front of
its own value; in all-gather round k rank r sends chunk (r + 1 - k) mod N,
which the receiver stores.  All sends of a round read the values held before
that round.  Rounds per phase: N - 1 (the 3-GPU example shows two).
"""
from __future__ import annotations

import operator
from typing import Any, Callable, List


def ring_allreduce(holdings: List[List[Any]], add: Callable[[Any, Any], Any] = operator.add,
                   size: Callable[[Any], int] = lambda x: 1):
    """holdings[r][c] is rank r's value of chunk c.  Returns the final
    holdings, the holdings after scatter-reduce, and the message log: one
    dict per message with phase, round, src, dst, chunk, elements, the value
    sent and the value the receiver holds afterwards."""
    n = len(holdings)
    h = [list(row) for row in holdings]
    log: List[dict] = []
    for k in range(n - 1):
        sends = [(r, (r + 1) % n, (r - k) % n) for r in range(n)]
        msgs = [(src, dst, c, h[src][c]) for src, dst, c in sends]
        for src, dst, c, val in msgs:
            h[dst][c] = add(val, h[dst][c])
            log.append(dict(phase="scatter_reduce", round=k, src=src, dst=dst,
                            chunk=c, elements=size(val), sent=val, holds=h[dst][c]))
    after_sr = [list(row) for row in h]
    for k in range(n - 1):
        sends = [(r, (r + 1) % n, (r + 1 - k) % n) for r in range(n)]
        msgs = [(src, dst, c, h[src][c]) for src, dst, c in sends]
        for src, dst, c, val in msgs:
            h[dst][c] = val
            log.append(dict(phase="all_gather", round=k, src=src, dst=dst,
                            chunk=c, elements=size(val), sent=val, holds=val))
    return h, after_sr, log


def owner_of_chunk_after_scatter_reduce(c: int, n: int) -> int:
    """The rank that holds chunk c complete after scatter-reduce: c - 1 mod N."""
    return (c - 1) % n
