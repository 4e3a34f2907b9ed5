"""Placement search for a shard's long-lived device arrays.

The fused step streams N + 7 arrays at once (N gradient chunks, three fp32
state arrays read and three written, the fp16 params).  On MI355X its
bandwidth depends on where those arrays sit in physical HBM, not only on
their virtual layout.  At the Llama-3-8B shard (n = 1,003,750,000, N = 8) the
same kernel over the same virtual layout took 6.8 to 7.8 ms from one fresh
allocation to the next, and each allocation kept its rate for as long as it
lived.  Arrays that are physically contiguous (hipExtMallocWithFlags with the
contiguous flag) took about 11 ms, whatever their relative offsets; arrays
assembled from small scattered holes ran faster than arrays from large ones.
The mapping of physical addresses to HBM3E channels, banks and rows is not
documented, so this module does not compute a placement: it measures one.

`place_shard` allocates complete new sets of the arrays, with spacer
allocations of random size between them so that each set lands somewhere
else in physical memory, copies the contents over, times the fused step on
each set, and keeps the fastest.  Re-allocating one array at a time was
tried first and mostly failed: a new array comes out of the free memory
that has not been used yet, which is the large contiguous kind, and few
single moves helped.  Contents are unchanged bit for bit; only where the
data sits changes.  It is a set-up step, for arrays that live as long as the
training run, and it runs before the first step.

The single-pass flow alternates the two state copies (a step reads copy cur
and writes the other), so the search times both directions, 0 -> 1 and
1 -> 0, and minimises their sum.  Those timing steps overwrite both copies, so
copy 0 is saved first and restored at the end; copy 1 is left holding the
last timing step's output, which the first real step overwrites.

Allocation goes through torch's caching allocator; the search empties its
cache after every trial, so that the next trial gets fresh memory and a
rejected set's memory goes back to the driver.

A whole new set needs room for two more sets beside the caller's.  Where
that does not fit (the 70B-class shard's two state copies alone take 124 GB),
`place_groups` re-places one group of arrays per trial instead (for example
the copy a step writes together with the gradient buffers, then the copy it
reads), keeping the others where they are.
"""
from __future__ import annotations

import dataclasses
import random
import statistics
import time
from typing import Callable, List, Optional, Sequence

import torch

from . import zero_shard_step_out, adamw_params, AdamWParams


@dataclasses.dataclass
class PlacementReport:
    """What a search did.  Times are one step in each direction, summed, in ms."""
    initial_ms: float
    final_ms: float
    trials: int
    kept: List[int]      # the trials whose set was kept (1-based)
    seconds: float

    @property
    def gain(self) -> float:
        return self.initial_ms / self.final_ms if self.final_ms > 0 else 1.0


def _time_both(chunks, copies, hp, loss_scale, flag, sq, stream, reps) -> float:
    """Median step time 0 -> 1 plus median 1 -> 0, HIP events on `stream`."""
    def launch(src, dst):
        zero_shard_step_out(chunks, loss_scale, src[0], src[1], src[2], dst[0], dst[1], dst[2],
                            dst[3], hp, flag, sq, stream=stream)

    launch(copies[0], copies[1])  # warm-up
    times = ([], [])
    for _ in range(reps):
        for d in (0, 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(copies[d], copies[1 - d])
            e1.record(stream)
            times[d].append((e0, e1))
    stream.synchronize()
    return sum(statistics.median(a.elapsed_time(b) for a, b in t) for t in times)


def _search(best_set: list, timed: Callable[[list], float],
            make_set: Callable[[list], Optional[list]], release: Callable[[], None], *,
            trials: int, budget_s: float, min_gain: float,
            clock: Callable[[], float] = time.perf_counter):
    """The search itself, apart from allocation and timing.  `timed(set)`
    gives a set's time; `make_set(set)` returns a new set with the same
    contents, or None when memory runs out; `release()` returns the memory of
    dropped sets.  Returns (best_set, initial_ms, best_ms, trials_done,
    kept), `kept` listing the 1-based trials whose set was kept."""
    t_start = clock()
    best = timed(best_set)
    initial = best
    done, kept = 0, []
    while done < trials and clock() - t_start < budget_s:
        new = make_set(best_set)
        if new is None:
            release()
            break
        t = timed(new)
        done += 1
        if t < best * (1.0 - min_gain):
            best, best_set = t, new
            kept.append(done)
        del new
        release()
    return best_set, initial, best, done, kept


def place_groups(arrays: Sequence[torch.Tensor], groups, timed: Callable[[list], float], *,
                 restore: Sequence[int] = (), trials: int = 12, budget_s: float = 30.0,
                 min_gain: float = 0.005, max_spacer: int = 4 << 30, seed: int = 0,
                 stream=None):
    """A leaner search: each trial re-places one group of the arrays, not the
    whole set, so it needs room for one group more rather than two sets more.

    arrays: a list of the long-lived device arrays, which the search takes
    over: it empties the list, so that the caller holds no reference that
    would keep a replaced array's memory alive; groups: a sequence of (indices,
    keep_contents), trial k re-placing group k mod len(groups) (each new
    array behind a spacer allocation of random size, its contents copied over
    when keep_contents is true); timed(arrays): the time to minimise, in ms,
    for the arrays as given.  The timing may overwrite arrays: those listed
    in `restore` are saved to host memory first and written back into the
    arrays kept at the end, so they come back bit for bit.  A trial is kept
    when it beats the best time by more than `min_gain` (relative).  Returns
    (arrays, report); the caller must use the returned arrays and drop its
    references to the ones it passed in."""
    if stream is None:
        stream = torch.cuda.current_stream()
    rng = random.Random(seed)
    # the search's list is reachable only through `holder` until _search takes
    # it: a kept trial then drops the last reference to the group it replaced
    holder = [list(arrays)]
    arrays.clear()
    dev = holder[0][0].device
    t_start = time.perf_counter()
    turn = [0]

    def make_set(cur):
        idx, keep = groups[turn[0] % len(groups)]
        turn[0] += 1
        new = list(cur)
        spacers = []
        try:
            for i in idx:
                spacers.append(torch.empty(1 + rng.randrange(max_spacer), dtype=torch.uint8,
                                           device=dev))
                new[i] = torch.empty_like(cur[i])
        except torch.OutOfMemoryError:
            return None
        del spacers
        if keep:
            for i in idx:
                new[i].copy_(cur[i])
        return new

    with torch.cuda.stream(stream):
        saved = {i: holder[0][i].cpu() for i in restore}
        best_set, initial, best, done, kept = _search(
            holder.pop(), timed, make_set, torch.cuda.empty_cache, trials=trials,
            budget_s=budget_s, min_gain=min_gain)
        for i, host in saved.items():
            best_set[i].copy_(host)
        del saved
        stream.synchronize()
        torch.cuda.empty_cache()
    report = PlacementReport(initial_ms=initial, final_ms=best, trials=done, kept=kept,
                             seconds=time.perf_counter() - t_start)
    return best_set, report


def place_shard(chunks: Sequence[torch.Tensor], copies, hp, loss_scale: float, *,
                trials: int = 12, budget_s: float = 30.0, min_gain: float = 0.005,
                max_spacer: int = 4 << 30, reps: int = 2, seed: int = 0, stream=None):
    """Search for a faster physical placement of a shard's arrays.

    chunks: the N fp16 gradient-chunk buffers; copies: two (master, exp_avg,
    exp_avg_sq, param_fp16) tuples, copy 0 holding the state.  Each trial
    allocates a complete new set of the N + 8 arrays, with spacer
    allocations of random size (up to `max_spacer` bytes) before each array
    so that the set lands somewhere new, copies the contents over, and times
    the step in both directions.  The set with the lowest time is kept (a
    new set must beat the kept one by more than `min_gain`, relative).  The
    search stops after `trials` trials, after `budget_s` seconds, or at the
    first allocation that fails.  While it runs it needs room for three
    sets (the caller's, the kept one and the trial), the spacers and a
    saved copy of copy 0.

    Returns (chunks, copies, report) with the same contents in possibly new
    tensors.  The caller must use the returned tensors and drop its
    references to the ones it passed in: the timing steps overwrite those
    state copies, and their memory stays held while referenced.  The chunks
    are only read."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if not isinstance(hp, AdamWParams):
        hp = adamw_params(hp)
    rng = random.Random(seed)
    n_chunks = len(chunks)
    first_set = list(chunks) + list(copies[0]) + list(copies[1])
    dev = first_set[0].device
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    sq = torch.zeros(1, dtype=torch.float64, device=dev)
    t_start = time.perf_counter()

    def split(arrs):
        return arrs[:n_chunks], (arrs[n_chunks:n_chunks + 4], arrs[n_chunks + 4:])

    def timed(arrs):
        c, cp = split(arrs)
        return _time_both(c, cp, hp, loss_scale, flag, sq, stream, reps)

    def make_set(cur):
        spacers, new = [], []
        try:
            for t in cur:
                spacers.append(torch.empty(1 + rng.randrange(max_spacer), dtype=torch.uint8,
                                           device=dev))
                new.append(torch.empty_like(t))
        except torch.OutOfMemoryError:
            return None
        del spacers
        for dst, src in zip(new, cur):
            dst.copy_(src)
        return new

    with torch.cuda.stream(stream):
        saved = [t.clone() for t in first_set[n_chunks:n_chunks + 4]]
        best_set, initial, best, done, kept = _search(
            first_set, timed, make_set, torch.cuda.empty_cache, trials=trials,
            budget_s=budget_s, min_gain=min_gain)
        del first_set
        for dst, src in zip(best_set[n_chunks:n_chunks + 4], saved):
            dst.copy_(src)
        del saved
        stream.synchronize()
        torch.cuda.empty_cache()
    c, cp = split(best_set)
    report = PlacementReport(initial_ms=initial, final_ms=best, trials=done, kept=kept,
                             seconds=time.perf_counter() - t_start)
    return list(c), (tuple(cp[0]), tuple(cp[1])), report
