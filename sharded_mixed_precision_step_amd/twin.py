"""Python binding of libzerotwin.so: the benchmark's measurement aids
(zero_twin.h).  Not part of the step library; only bench.py and its tests
load it.  Argument marshalling only, as in the package's main binding."""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

from . import _build
from . import ZeroStepError, _dev, _ptr_array, _stream

LIB_PATH = _build.TWIN_LIB
EXPORTED = ("zero_traffic_twin", "zero_stream_read", "zero_twin_last_error_string")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.zero_traffic_twin.argtypes = [pp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.zero_traffic_twin.restype = ctypes.c_int
    lib.zero_stream_read.argtypes = [vp, i64, vp, vp]
    lib.zero_stream_read.restype = ctypes.c_int
    lib.zero_twin_last_error_string.argtypes = []
    lib.zero_twin_last_error_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(rc: int) -> None:
    if rc != 0:
        raise ZeroStepError(rc, lib.zero_twin_last_error_string().decode())


def zero_traffic_twin(grad_chunks: Sequence[torch.Tensor], master_in: torch.Tensor,
                      exp_avg_in: torch.Tensor, exp_avg_sq_in: torch.Tensor,
                      master_out: torch.Tensor, exp_avg_out: torch.Tensor,
                      exp_avg_sq_out: torch.Tensor, param_fp16_out: torch.Tensor,
                      stream=None) -> None:
    """The fused step's memory accesses with XORs for arithmetic: a bandwidth
    reference for the step's access pattern (see zero_twin.h)."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = master_in.numel()
    for name, t in (("exp_avg_in", exp_avg_in), ("exp_avg_sq_in", exp_avg_sq_in),
                    ("master_out", master_out), ("exp_avg_out", exp_avg_out),
                    ("exp_avg_sq_out", exp_avg_sq_out), ("param_fp16_out", param_fp16_out),
                    *((f"grad_chunks[{i}]", c) for i, c in enumerate(grad_chunks))):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    _check(lib.zero_traffic_twin(
        _ptr_array(ptrs), len(ptrs), n, _dev(master_in, torch.float32, "master_in"),
        _dev(exp_avg_in, torch.float32, "exp_avg_in"),
        _dev(exp_avg_sq_in, torch.float32, "exp_avg_sq_in"),
        _dev(master_out, torch.float32, "master_out"),
        _dev(exp_avg_out, torch.float32, "exp_avg_out"),
        _dev(exp_avg_sq_out, torch.float32, "exp_avg_sq_out"),
        _dev(param_fp16_out, torch.float16, "param_fp16_out"), _stream(stream)))


def zero_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of ``src`` (contiguous, a multiple of 16 bytes) once and
    XOR its 32-bit words into ``sink`` (int32[1]): a read-only stream."""
    if not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous device tensor")
    _check(lib.zero_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                _dev(sink, torch.int32, "sink"), _stream(stream)))
