"""The C client's input and output files (the format zero_client.c states)."""
from __future__ import annotations

import dataclasses
import struct
from typing import List

import numpy as np

MAGIC = 0x5A43


@dataclasses.dataclass
class ClientInput:
    replicas: List[List[np.ndarray]]   # N lists of T fp16 tensors
    rank: int
    align: int
    hyper: object                      # lr, beta1, beta2, eps, weight_decay, step, ...
    loss_scale: float
    growth_factor: float
    backoff_factor: float
    min_scale: float
    max_scale: float
    growth_interval: int
    good_steps: int
    skipped_steps: int
    master: np.ndarray                 # the rank's shard of the state
    m: np.ndarray
    v: np.ndarray
    p16: np.ndarray

    def to_bytes(self) -> bytes:
        h = self.hyper
        numels = [t.size for t in self.replicas[0]]
        head = struct.pack("<11q", MAGIC, len(self.replicas), len(numels), self.rank, self.align,
                           h.step, int(h.decoupled_wd), int(h.bias_correction),
                           self.growth_interval, self.good_steps, self.skipped_steps)
        head += struct.pack(f"<{len(numels)}q", *numels)
        head += struct.pack("<10d", self.loss_scale, h.lr, h.beta1, h.beta2, h.eps,
                            h.weight_decay, self.growth_factor, self.backoff_factor,
                            self.min_scale, self.max_scale)
        body = [np.ascontiguousarray(t, np.float16).tobytes()
                for rep in self.replicas for t in rep]
        body.append(struct.pack("<q", self.master.size))
        body += [np.ascontiguousarray(a, d).tobytes() for a, d in
                 ((self.master, np.float32), (self.m, np.float32), (self.v, np.float32),
                  (self.p16, np.float16))]
        return head + b"".join(body)


@dataclasses.dataclass
class ClientOutput:
    L: int
    s: int
    overflow: int
    skip: int
    good_steps: int
    skipped_steps: int
    sqnorm: float
    scale: float
    offsets: List[int]
    master: np.ndarray
    m: np.ndarray
    v: np.ndarray
    p16: np.ndarray


def read_output(data: bytes, n_tensors: int) -> ClientOutput:
    L, s, overflow, skip, good, skipped = struct.unpack_from("<6q", data, 0)
    sqnorm, scale = struct.unpack_from("<2d", data, 48)
    pos = 64
    offsets = list(struct.unpack_from(f"<{n_tensors + 1}q", data, pos))
    pos += 8 * (n_tensors + 1)
    arrays = []
    for dtype, width in ((np.float32, 4), (np.float32, 4), (np.float32, 4), (np.float16, 2)):
        arrays.append(np.frombuffer(data, dtype, s, pos).copy())
        pos += width * s
    if pos != len(data):
        raise ValueError(f"output holds {len(data)} bytes, expected {pos}")
    return ClientOutput(L, s, overflow, skip, good, skipped, sqnorm, scale, offsets, *arrays)
