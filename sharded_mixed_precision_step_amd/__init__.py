"""Python binding of libzerostep.so, the MI355X (gfx950) ZeRO-1/2 shard step.

Argument marshalling only: tensors become raw device pointers, the current
torch stream becomes a hipStream_t, and every call goes straight to the C ABI
declared in include/zero_step.h.  All arithmetic of the step runs in the HIP
kernels; nothing here computes on data.  If the library is missing the import
fails loudly: there is no fallback path.

torch is imported before the library is loaded so that the process holds a
single HIP runtime (torch's libamdhip64.so.7 satisfies the library's
dependency of the same soname) and torch's stream handles are valid for it.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch  # noqa: F401  (loads the HIP runtime first; see module docstring)

from . import _build

LIB_PATH = _build.LIB

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EALIGN = -2
ZERO_ERANGE = -3
ZERO_EHIP = -4
ZERO_MAX_CHUNKS = 64

EXPORTED = ("zero_overflow_check", "zero_shard_step", "zero_shard_step_out",
            "zero_shard_step_buckets", "zero_reduce_mean_fp16", "zero_accumulate_chunk",
            "zero_accumulate_chunks", "zero_accumulate_chunk_noalloc", "zero_bucket_flatten",
            "zero_bucket_flatten_batch",
            "zero_update_loss_scale",
            "zero_control_init",
            "zero_control_begin", "zero_overflow_check_ctl", "zero_control_decide",
            "zero_shard_step_ctl", "zero_shard_step_out_ctl", "zero_shard_step_buckets_ctl",
            "zero_last_error_string")
ZERO_CTL_STEPS = 64
ZERO_NORM_SLOTS = 16
ZERO_NORM_STRIDE = 8
ZERO_CHECK_PARTS = 1536
ZERO_FOLD_SCRATCH_ELEMS = 8388608


class ZeroStepError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class AdamWParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64),
                ("decoupled_wd", ctypes.c_int32), ("bias_correction", ctypes.c_int32)]


class LossScaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("growth_factor", ctypes.c_float),
                ("backoff_factor", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("max_scale", ctypes.c_float), ("growth_interval", ctypes.c_int32),
                ("good_steps", ctypes.c_int32), ("skipped_steps", ctypes.c_int64)]

    @classmethod
    def create(cls, scale=65536.0, growth_factor=2.0, backoff_factor=0.5,
               min_scale=1.0, max_scale=float(2 ** 24), growth_interval=1000):
        return cls(scale, growth_factor, backoff_factor, min_scale, max_scale,
                   growth_interval, 0, 0)


class StepControl(ctypes.Structure):
    """zero_step_control: the device-resident loss scale, t and step decision."""
    _fields_ = [("scale", ctypes.c_float), ("growth_factor", ctypes.c_float),
                ("backoff_factor", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("max_scale", ctypes.c_float), ("growth_interval", ctypes.c_int32),
                ("good_steps", ctypes.c_int32), ("cur", ctypes.c_int32),
                ("skipped_steps", ctypes.c_int64), ("step", ctypes.c_int64),
                ("step_used", ctypes.c_int64), ("sqnorm", ctypes.c_double),
                ("scale_used", ctypes.c_float), ("clip_coef", ctypes.c_float),
                ("overflow", ctypes.c_int32), ("skip", ctypes.c_int32),
                ("error", ctypes.c_int32), ("check_ran", ctypes.c_int32),
                ("bc1_used", ctypes.c_float), ("bc2_used", ctypes.c_float),
                ("table_miss", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("sqnorm_part", ctypes.c_double * (ZERO_NORM_SLOTS * ZERO_NORM_STRIDE)),
                ("check_part", ctypes.c_double * ZERO_CHECK_PARTS)]


class FlattenBucketC(ctypes.Structure):
    _fields_ = [("tensors", ctypes.POINTER(ctypes.c_void_p)),
                ("numels", ctypes.POINTER(ctypes.c_int64)),
                ("offsets_out", ctypes.POINTER(ctypes.c_int64)), ("bucket", ctypes.c_void_p),
                ("bucket_capacity", ctypes.c_int64), ("n_tensors", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


class BucketSliceC(ctypes.Structure):
    _fields_ = [("grad_chunks", ctypes.POINTER(ctypes.c_void_p)), ("n", ctypes.c_int64),
                ("offset", ctypes.c_int64)]


def adamw_params(hyper) -> AdamWParams:
    """AdamWParams from any object with lr, beta1, beta2, eps, weight_decay,
    step, decoupled_wd and bias_correction attributes."""
    return AdamWParams(hyper.lr, hyper.beta1, hyper.beta2, hyper.eps,
                       hyper.weight_decay, int(hyper.step), int(bool(hyper.decoupled_wd)),
                       int(bool(getattr(hyper, "bias_correction", True))))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.zero_overflow_check.argtypes = [pp, i32, i64, ctypes.c_float, vp, vp, vp]
    lib.zero_shard_step.argtypes = [pp, i32, i64, ctypes.c_float, vp, vp, vp, vp,
                                    ctypes.POINTER(AdamWParams), vp, vp, vp]
    lib.zero_shard_step_out.argtypes = [pp, i32, i64, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.POINTER(AdamWParams), vp, vp, vp]
    lib.zero_shard_step_buckets.argtypes = [ctypes.POINTER(BucketSliceC), i32, i32,
                                             ctypes.c_float, i64, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.POINTER(AdamWParams), vp, vp, vp]
    lib.zero_reduce_mean_fp16.argtypes = [pp, i32, i64, ctypes.c_float, vp, vp, vp, vp]
    lib.zero_accumulate_chunk.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.zero_accumulate_chunk_noalloc.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.zero_accumulate_chunks.argtypes = [pp, i32, i64, i32, i32, vp, vp, vp]
    lib.zero_bucket_flatten.argtypes = [pp, ctypes.POINTER(ctypes.c_int64), i32, i64, i64,
                                        vp, i64, ctypes.POINTER(ctypes.c_int64), vp]
    lib.zero_bucket_flatten_batch.argtypes = [ctypes.POINTER(FlattenBucketC), i32, i64, i64, vp]
    lib.zero_update_loss_scale.argtypes = [ctypes.POINTER(LossScaler), i32,
                                           ctypes.POINTER(ctypes.c_int32)]
    lib.zero_control_init.argtypes = [ctypes.POINTER(StepControl), ctypes.POINTER(LossScaler),
                                      i64]
    lib.zero_control_begin.argtypes = [vp, ctypes.POINTER(AdamWParams), vp]
    lib.zero_overflow_check_ctl.argtypes = [pp, i32, i64, vp, vp]
    lib.zero_control_decide.argtypes = [vp, ctypes.c_float, i32, vp]
    lib.zero_shard_step_ctl.argtypes = [pp, i32, i64, vp, vp, vp, vp, ctypes.POINTER(AdamWParams),
                                        vp, vp]
    lib.zero_shard_step_out_ctl.argtypes = [pp, i32, i64, pp, pp, pp, pp,
                                            ctypes.POINTER(AdamWParams), vp, vp]
    lib.zero_shard_step_buckets_ctl.argtypes = [ctypes.POINTER(BucketSliceC), i32, i32, i64, pp,
                                                pp, pp, pp, ctypes.POINTER(AdamWParams), vp, vp]
    lib.zero_last_error_string.argtypes = []
    lib.zero_last_error_string.restype = ctypes.c_char_p
    for name in EXPORTED[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _check(rc: int) -> None:
    if rc != ZERO_OK:
        raise ZeroStepError(rc, lib.zero_last_error_string().decode())


def _ptr_array(ptrs: Sequence[int]):
    arr = (ctypes.c_void_p * max(len(ptrs), 1))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor], dtype: torch.dtype, name: str) -> Optional[int]:
    return None if t is None else _dev(t, dtype, name)


def zero_overflow_check(grad_chunks: Sequence[torch.Tensor], loss_scale: float,
                        d_overflow: torch.Tensor, d_sqnorm: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """OR the non-finite flag of g = (sum chunks / N) / loss_scale into
    d_overflow (int32[1]) and add sum g^2 to d_sqnorm (float64[1])."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = grad_chunks[0].numel() if grad_chunks else 0
    for i, c in enumerate(grad_chunks):
        if c.numel() != n:
            raise ValueError(f"grad_chunks[{i}] has {c.numel()} elements, expected {n}")
    _check(lib.zero_overflow_check(_ptr_array(ptrs), len(ptrs), n, float(loss_scale),
                                   _dev(d_overflow, torch.int32, "d_overflow"),
                                   _opt(d_sqnorm, torch.float64, "d_sqnorm"), _stream(stream)))


def zero_shard_step(grad_chunks: Sequence[torch.Tensor], loss_scale: float,
                    master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                    param_fp16: torch.Tensor, hp: AdamWParams,
                    d_overflow: Optional[torch.Tensor] = None,
                    d_sqnorm: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fused Adam/AdamW update of one shard in place (see zero_step.h)."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = master.numel()
    for name, t in (("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq),
                    ("param_fp16", param_fp16), *[(f"grad_chunks[{i}]", c)
                                                  for i, c in enumerate(grad_chunks)]):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    if not isinstance(hp, AdamWParams):
        hp = adamw_params(hp)
    _check(lib.zero_shard_step(
        _ptr_array(ptrs), len(ptrs), n, float(loss_scale),
        _dev(master, torch.float32, "master"), _dev(exp_avg, torch.float32, "exp_avg"),
        _dev(exp_avg_sq, torch.float32, "exp_avg_sq"),
        _dev(param_fp16, torch.float16, "param_fp16"), ctypes.byref(hp),
        _opt(d_overflow, torch.int32, "d_overflow"), _opt(d_sqnorm, torch.float64, "d_sqnorm"),
        _stream(stream)))


def zero_shard_step_out(grad_chunks: Sequence[torch.Tensor], loss_scale: float,
                        master_in: torch.Tensor, exp_avg_in: torch.Tensor,
                        exp_avg_sq_in: torch.Tensor, master_out: torch.Tensor,
                        exp_avg_out: torch.Tensor, exp_avg_sq_out: torch.Tensor,
                        param_fp16_out: torch.Tensor, hp: AdamWParams,
                        d_overflow: Optional[torch.Tensor] = None,
                        d_sqnorm: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fused update from the *_in state into the *_out state (see zero_step.h)."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = master_in.numel()
    named = [("exp_avg_in", exp_avg_in), ("exp_avg_sq_in", exp_avg_sq_in),
             ("master_out", master_out), ("exp_avg_out", exp_avg_out),
             ("exp_avg_sq_out", exp_avg_sq_out), ("param_fp16_out", param_fp16_out)]
    named += [(f"grad_chunks[{i}]", c) for i, c in enumerate(grad_chunks)]
    for name, t in named:
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    if not isinstance(hp, AdamWParams):
        hp = adamw_params(hp)
    _check(lib.zero_shard_step_out(
        _ptr_array(ptrs), len(ptrs), n, float(loss_scale),
        _dev(master_in, torch.float32, "master_in"), _dev(exp_avg_in, torch.float32, "exp_avg_in"),
        _dev(exp_avg_sq_in, torch.float32, "exp_avg_sq_in"),
        _dev(master_out, torch.float32, "master_out"),
        _dev(exp_avg_out, torch.float32, "exp_avg_out"),
        _dev(exp_avg_sq_out, torch.float32, "exp_avg_sq_out"),
        _dev(param_fp16_out, torch.float16, "param_fp16_out"), ctypes.byref(hp),
        _opt(d_overflow, torch.int32, "d_overflow"), _opt(d_sqnorm, torch.float64, "d_sqnorm"),
        _stream(stream)))


class BucketSlices:
    """A table of bucket slices for zero_shard_step_buckets, marshalled once.

    ``slices`` is a sequence of (chunks, offset): the N replica gradient
    chunks of one bucket's slice (fp16 device tensors of equal length) and the
    slice's first element in the shard's state arrays.  The tensors are
    referenced, so their memory stays valid while the table exists; their
    contents may change between steps (bucket buffers are reused)."""

    def __init__(self, slices):
        self.tensors = []
        self.ptr_arrays = []
        self.n_chunks = None
        self.table = (BucketSliceC * max(len(slices), 1))()
        for k, (chunks, offset) in enumerate(slices):
            if self.n_chunks is None:
                self.n_chunks = len(chunks)
            elif len(chunks) != self.n_chunks:
                raise ValueError(f"slice {k} has {len(chunks)} chunks, expected {self.n_chunks}")
            n = chunks[0].numel()
            ptrs = []
            for i, c in enumerate(chunks):
                if c.numel() != n:
                    raise ValueError(f"slice {k} chunk {i} has {c.numel()} elements, expected {n}")
                ptrs.append(_dev(c, torch.float16, f"slice {k} chunk {i}"))
            arr = _ptr_array(ptrs)
            self.ptr_arrays.append(arr)
            self.tensors.append(list(chunks))
            self.table[k].grad_chunks = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
            self.table[k].n = n
            self.table[k].offset = int(offset)
        self.count = len(slices)
        if self.n_chunks is None:
            self.n_chunks = 1


def zero_shard_step_buckets(slices: BucketSlices, loss_scale: float, master_in: torch.Tensor,
                            exp_avg_in: torch.Tensor, exp_avg_sq_in: torch.Tensor,
                            master_out: torch.Tensor, exp_avg_out: torch.Tensor,
                            exp_avg_sq_out: torch.Tensor, param_fp16_out: torch.Tensor,
                            hp: AdamWParams, d_overflow: Optional[torch.Tensor] = None,
                            d_sqnorm: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fused update over every bucket slice of ``slices`` (see zero_step.h)."""
    n = master_in.numel()
    for name, t in (("exp_avg_in", exp_avg_in), ("exp_avg_sq_in", exp_avg_sq_in),
                    ("master_out", master_out), ("exp_avg_out", exp_avg_out),
                    ("exp_avg_sq_out", exp_avg_sq_out), ("param_fp16_out", param_fp16_out)):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    if not isinstance(hp, AdamWParams):
        hp = adamw_params(hp)
    _check(lib.zero_shard_step_buckets(
        slices.table, slices.count, slices.n_chunks, float(loss_scale), n,
        _dev(master_in, torch.float32, "master_in"), _dev(exp_avg_in, torch.float32, "exp_avg_in"),
        _dev(exp_avg_sq_in, torch.float32, "exp_avg_sq_in"),
        _dev(master_out, torch.float32, "master_out"),
        _dev(exp_avg_out, torch.float32, "exp_avg_out"),
        _dev(exp_avg_sq_out, torch.float32, "exp_avg_sq_out"),
        _dev(param_fp16_out, torch.float16, "param_fp16_out"), ctypes.byref(hp),
        _opt(d_overflow, torch.int32, "d_overflow"), _opt(d_sqnorm, torch.float64, "d_sqnorm"),
        _stream(stream)))


def zero_reduce_mean_fp16(grad_chunks: Sequence[torch.Tensor], mean_fp16: torch.Tensor,
                          loss_scale: float = 1.0, d_overflow: Optional[torch.Tensor] = None,
                          d_sqnorm: Optional[torch.Tensor] = None, stream=None) -> None:
    """mean_fp16 = fp16(sum of the chunks / N); optional flag and squared norm
    of fp32(mean_fp16) / loss_scale (see zero_step.h)."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = mean_fp16.numel()
    for i, c in enumerate(grad_chunks):
        if c.numel() != n:
            raise ValueError(f"grad_chunks[{i}] has {c.numel()} elements, expected {n}")
    _check(lib.zero_reduce_mean_fp16(_ptr_array(ptrs), len(ptrs), n, float(loss_scale),
                                     _dev(mean_fp16, torch.float16, "mean_fp16"),
                                     _opt(d_overflow, torch.int32, "d_overflow"),
                                     _opt(d_sqnorm, torch.float64, "d_sqnorm"), _stream(stream)))


def zero_accumulate_chunk(chunk: torch.Tensor, index: int, n_chunks: int,
                          acc: Optional[torch.Tensor], mean_fp16: Optional[torch.Tensor],
                          stream=None) -> None:
    """Fold replica `index`'s chunk into the fp32 accumulator; the last of
    n_chunks writes the fp16 mean (see zero_step.h)."""
    n = chunk.numel()
    for name, t in (("acc", acc), ("mean_fp16", mean_fp16)):
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    _check(lib.zero_accumulate_chunk(_dev(chunk, torch.float16, "chunk"), n, int(index),
                                     int(n_chunks), _opt(acc, torch.float32, "acc"),
                                     _opt(mean_fp16, torch.float16, "mean_fp16"),
                                     _stream(stream)))


def zero_accumulate_chunks(chunks: Sequence[torch.Tensor], first: int, n_chunks: int,
                           acc: Optional[torch.Tensor], mean_fp16: Optional[torch.Tensor],
                           stream=None) -> None:
    """Fold replicas first .. first + len(chunks) - 1 of n_chunks into the
    fp32 accumulator in one pass; the group holding the last replica writes
    the fp16 mean (see zero_step.h)."""
    n = chunks[0].numel() if chunks else 0
    ptrs = []
    for i, c in enumerate(chunks):
        if c.numel() != n:
            raise ValueError(f"chunks[{i}] has {c.numel()} elements, expected {n}")
        ptrs.append(_dev(c, torch.float16, f"chunks[{i}]"))
    for name, t in (("acc", acc), ("mean_fp16", mean_fp16)):
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    _check(lib.zero_accumulate_chunks(_ptr_array(ptrs), len(ptrs), n, int(first), int(n_chunks),
                                      _opt(acc, torch.float32, "acc"),
                                      _opt(mean_fp16, torch.float16, "mean_fp16"),
                                      _stream(stream)))


def zero_accumulate_chunk_noalloc(chunk: torch.Tensor, index: int, n_chunks: int,
                                  mean_fp16: Optional[torch.Tensor], stream=None) -> None:
    """zero_accumulate_chunk with the library's own accumulator (no device
    memory allocated; see zero_step.h for the sharing rules)."""
    n = chunk.numel()
    if mean_fp16 is not None and mean_fp16.numel() != n:
        raise ValueError(f"mean_fp16 has {mean_fp16.numel()} elements, expected {n}")
    _check(lib.zero_accumulate_chunk_noalloc(_dev(chunk, torch.float16, "chunk"), n, int(index),
                                             int(n_chunks),
                                             _opt(mean_fp16, torch.float16, "mean_fp16"),
                                             _stream(stream)))


def zero_bucket_flatten(tensors: Sequence[torch.Tensor], bucket: torch.Tensor,
                        align: int = 256, pad_multiple: int = 0, stream=None) -> list:
    """Pack fp16 tensors into ``bucket``; returns the offsets and padded length."""
    ptrs, numels = [], []
    for i, t in enumerate(tensors):
        ptrs.append(_dev(t, torch.float16, f"tensors[{i}]") if t.numel() else 0)
        numels.append(t.numel())
    nt = len(ptrs)
    numel_arr = (ctypes.c_int64 * max(nt, 1))(*numels)
    offs = (ctypes.c_int64 * (nt + 1))()
    _check(lib.zero_bucket_flatten(_ptr_array(ptrs), numel_arr, nt, int(align), int(pad_multiple),
                                   _dev(bucket, torch.float16, "bucket"), bucket.numel(), offs,
                                   _stream(stream)))
    return list(offs)


class FlattenBatch:
    """Arguments of zero_bucket_flatten_batch marshalled once: ``buckets`` is a
    sequence of (tensors, bucket), fp16 device tensors.  The tensors are
    referenced, so their memory stays valid while the object exists; their
    contents may change between calls.  ``offsets`` holds each bucket's slot
    offsets and padded length after a call."""

    def __init__(self, buckets, align: int = 256, pad_multiple: int = 0):
        self.align, self.pad_multiple = int(align), int(pad_multiple)
        self.count = len(buckets)
        self.table = (FlattenBucketC * max(self.count, 1))()
        self._keep = []
        self._offs = []
        for k, (tensors, bucket) in enumerate(buckets):
            ptrs = [_dev(t, torch.float16, f"bucket {k} tensor {i}") if t.numel() else 0
                    for i, t in enumerate(tensors)]
            nt = len(ptrs)
            parr = _ptr_array(ptrs)
            narr = (ctypes.c_int64 * max(nt, 1))(*[t.numel() for t in tensors])
            oarr = (ctypes.c_int64 * (nt + 1))()
            self._keep.append((list(tensors), bucket, parr, narr))
            self._offs.append(oarr)
            self.table[k].tensors = ctypes.cast(parr, ctypes.POINTER(ctypes.c_void_p))
            self.table[k].numels = ctypes.cast(narr, ctypes.POINTER(ctypes.c_int64))
            self.table[k].offsets_out = ctypes.cast(oarr, ctypes.POINTER(ctypes.c_int64))
            self.table[k].bucket = _dev(bucket, torch.float16, f"bucket {k}")
            self.table[k].bucket_capacity = bucket.numel()
            self.table[k].n_tensors = nt

    @property
    def offsets(self) -> list:
        return [list(o) for o in self._offs]

    def __call__(self, stream=None) -> list:
        _check(lib.zero_bucket_flatten_batch(self.table, self.count, self.align,
                                             self.pad_multiple, _stream(stream)))
        return self.offsets


def zero_bucket_flatten_batch(buckets, align: int = 256, pad_multiple: int = 0,
                              stream=None) -> list:
    """Pack each bucket's fp16 tensors into it, all buckets in few launches;
    ``buckets``: a sequence of (tensors, bucket).  Returns every bucket's
    offsets and padded length."""
    return FlattenBatch(buckets, align, pad_multiple)(stream)


def zero_update_loss_scale(scaler: LossScaler, overflow: int) -> bool:
    """Advance the dynamic loss scale after a step; True means skip the step."""
    skip = ctypes.c_int32(0)
    _check(lib.zero_update_loss_scale(ctypes.byref(scaler), int(overflow), ctypes.byref(skip)))
    return bool(skip.value)


@dataclasses.dataclass
class ShardStepResult:
    overflow: bool
    skipped: bool
    sqnorm: float


def checked_step(grad_chunks, master, exp_avg, exp_avg_sq, param_fp16, hp: AdamWParams,
                 scaler: LossScaler, d_overflow: torch.Tensor, d_sqnorm: torch.Tensor,
                 stream=None) -> ShardStepResult:
    """One clean-or-skipped step as a rank runs it: check, read the flag back,
    update the loss scale, then update the shard only if the step is clean.
    d_overflow and d_sqnorm are caller-owned device scalars (zeroed here);
    hp.step is advanced on a clean step."""
    d_overflow.zero_()
    d_sqnorm.zero_()
    scale = scaler.scale
    zero_overflow_check(grad_chunks, scale, d_overflow, d_sqnorm, stream=stream)
    flag = int(d_overflow.item())          # device -> host: the skip decision
    skip = zero_update_loss_scale(scaler, flag)
    if not skip:
        zero_shard_step(grad_chunks, scale, master, exp_avg, exp_avg_sq, param_fp16, hp,
                        stream=stream)
        hp.step += 1
    return ShardStepResult(bool(flag), skip, float(d_sqnorm.item()))


class DoubleBufferedShard:
    """Two copies of a shard's state (fp32 master, m, v and fp16 params) for
    the single-pass step: a step reads copy ``cur`` and writes the other, and
    is committed by making the other copy current.  Memory is owned by the
    caller's tensors; this object only tracks which copy is current."""

    def __init__(self, master, exp_avg, exp_avg_sq, param_fp16, spare=None):
        if spare is None:
            spare = tuple(torch.empty_like(t) for t in (master, exp_avg, exp_avg_sq, param_fp16))
        self.copies = [(master, exp_avg, exp_avg_sq, param_fp16), tuple(spare)]
        self.cur = 0

    @property
    def current(self):
        return self.copies[self.cur]

    @property
    def other(self):
        return self.copies[1 - self.cur]


def committed_step(grad_chunks, shard: DoubleBufferedShard, hp: AdamWParams,
                   scaler: LossScaler, d_overflow: torch.Tensor, d_sqnorm: torch.Tensor,
                   stream=None) -> ShardStepResult:
    """One clean-or-skipped step in a single pass over the gradients: the
    fused out-of-place update (with the flag and squared norm), the flag read
    back, the loss-scale update, and the commit (the written copy becomes
    current) only if the step is clean.  hp.step is advanced on a clean step."""
    d_overflow.zero_()
    d_sqnorm.zero_()
    scale = scaler.scale
    m_in, a_in, v_in, _ = shard.current
    m_out, a_out, v_out, p_out = shard.other
    zero_shard_step_out(grad_chunks, scale, m_in, a_in, v_in, m_out, a_out, v_out, p_out, hp,
                        d_overflow, d_sqnorm, stream=stream)
    flag = int(d_overflow.item())          # device -> host: the skip decision
    skip = zero_update_loss_scale(scaler, flag)
    if not skip:
        shard.cur = 1 - shard.cur
        hp.step += 1
    return ShardStepResult(bool(flag), skip, float(d_sqnorm.item()))


# ---------------------------------------------------------------------------
# Device-resident step control: the whole step enqueued with no read-back.
# ---------------------------------------------------------------------------

def control_new(scaler: LossScaler, step: int, device) -> torch.Tensor:
    """A zero_step_control block in device memory (a uint8 tensor), filled
    from the scaler and the first update's t."""
    host = StepControl()
    _check(lib.zero_control_init(ctypes.byref(host), ctypes.byref(scaler), int(step)))
    raw = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8)
    return raw.to(device)


def control_read(ctl: torch.Tensor) -> StepControl:
    """A host copy of the block (synchronises with the device)."""
    return StepControl.from_buffer_copy(ctl.cpu().numpy().tobytes())


def _ctl(ctl: torch.Tensor) -> int:
    if ctl.dtype != torch.uint8 or ctl.numel() != ctypes.sizeof(StepControl):
        raise TypeError("ctl must be the uint8 tensor control_new returns")
    return _dev(ctl, torch.uint8, "ctl")


def zero_control_begin(ctl: torch.Tensor, hp: AdamWParams, stream=None) -> None:
    """Start a step; hp gives the table of bias corrections (base t0 =
    hp.step) from which the step's are looked up."""
    if not isinstance(hp, AdamWParams):
        hp = adamw_params(hp)
    _check(lib.zero_control_begin(_ctl(ctl), ctypes.byref(hp), _stream(stream)))


def zero_overflow_check_ctl(grad_chunks: Sequence[torch.Tensor], ctl: torch.Tensor,
                            stream=None) -> None:
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = grad_chunks[0].numel() if grad_chunks else 0
    for i, c in enumerate(grad_chunks):
        if c.numel() != n:
            raise ValueError(f"grad_chunks[{i}] has {c.numel()} elements, expected {n}")
    _check(lib.zero_overflow_check_ctl(_ptr_array(ptrs), len(ptrs), n, _ctl(ctl),
                                       _stream(stream)))


def zero_control_decide(ctl: torch.Tensor, max_grad_norm: float = 0.0, flip_copy: bool = False,
                        stream=None) -> None:
    _check(lib.zero_control_decide(_ctl(ctl), float(max_grad_norm), int(bool(flip_copy)),
                                   _stream(stream)))


def zero_shard_step_ctl(grad_chunks: Sequence[torch.Tensor], master: torch.Tensor,
                        exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                        param_fp16: torch.Tensor, hp: AdamWParams, ctl: torch.Tensor,
                        stream=None) -> None:
    """The two-pass update under the control block (hp.step: the base t of
    the bias-correction table)."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = master.numel()
    for name, t in (("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq), ("param_fp16", param_fp16),
                    *[(f"grad_chunks[{i}]", c) for i, c in enumerate(grad_chunks)]):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    _check(lib.zero_shard_step_ctl(
        _ptr_array(ptrs), len(ptrs), n, _dev(master, torch.float32, "master"),
        _dev(exp_avg, torch.float32, "exp_avg"), _dev(exp_avg_sq, torch.float32, "exp_avg_sq"),
        _dev(param_fp16, torch.float16, "param_fp16"), ctypes.byref(hp), _ctl(ctl),
        _stream(stream)))


def zero_shard_step_out_ctl(grad_chunks: Sequence[torch.Tensor], copies, hp: AdamWParams,
                            ctl: torch.Tensor, stream=None) -> None:
    """The single-pass update under the control block: from copy ctl.cur into
    the other.  copies: two (master, exp_avg, exp_avg_sq, param_fp16) tuples."""
    ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
    n = copies[0][0].numel()
    for k, cp in enumerate(copies):
        for j, t in enumerate(cp):
            if t.numel() != n:
                raise ValueError(f"copy {k} array {j} has {t.numel()} elements, expected {n}")
    for i, c in enumerate(grad_chunks):
        if c.numel() != n:
            raise ValueError(f"grad_chunks[{i}] has {c.numel()} elements, expected {n}")
    dts = (torch.float32, torch.float32, torch.float32, torch.float16)
    tables = [_ptr_array([_dev(copies[k][j], dts[j], f"copy {k} array {j}") for k in range(2)])
              for j in range(4)]
    _check(lib.zero_shard_step_out_ctl(_ptr_array(ptrs), len(ptrs), n, *tables, ctypes.byref(hp),
                                       _ctl(ctl), _stream(stream)))


def zero_shard_step_buckets_ctl(slices: BucketSlices, copies, hp: AdamWParams,
                                ctl: torch.Tensor, stream=None) -> None:
    """The single-pass update over a bucket table under the control block:
    every slice from copy ctl.cur into the other.  The slices must tile the
    state arrays exactly."""
    n = copies[0][0].numel()
    for k, cp in enumerate(copies):
        for j, t in enumerate(cp):
            if t.numel() != n:
                raise ValueError(f"copy {k} array {j} has {t.numel()} elements, expected {n}")
    dts = (torch.float32, torch.float32, torch.float32, torch.float16)
    tables = [_ptr_array([_dev(copies[k][j], dts[j], f"copy {k} array {j}") for k in range(2)])
              for j in range(4)]
    _check(lib.zero_shard_step_buckets_ctl(slices.table, slices.count, slices.n_chunks, n,
                                           *tables, ctypes.byref(hp), _ctl(ctl),
                                           _stream(stream)))


_ON_STREAM = object()   # a streamed bucket whose chunks arrive on the step's stream


class _Tiling:
    """Bucket ranges [offset, offset + length) of an n-element state, added
    one at a time: each must lie inside the state and overlap none before
    it, and `complete()` tells whether they now cover it exactly."""

    def __init__(self, n: int):
        self.n = n
        self.starts: list = []
        self.ends: list = []
        self.covered = 0

    def add(self, offset: int, length: int) -> None:
        import bisect
        if offset < 0 or length < 0 or offset + length > self.n:
            raise ValueError(f"bucket [{offset}, {offset + length}) lies outside the "
                             f"{self.n}-element state")
        if length == 0:
            return
        k = bisect.bisect_right(self.starts, offset)
        if k > 0 and self.ends[k - 1] > offset:
            raise ValueError(f"bucket [{offset}, {offset + length}) overlaps "
                             f"[{self.starts[k - 1]}, {self.ends[k - 1]})")
        if k < len(self.starts) and self.starts[k] < offset + length:
            raise ValueError(f"bucket [{offset}, {offset + length}) overlaps "
                             f"[{self.starts[k]}, {self.ends[k]})")
        self.starts.insert(k, offset)
        self.ends.insert(k, offset + length)
        self.covered += length

    def complete(self) -> bool:
        return self.covered == self.n


class DeviceStepper:
    """Enqueues whole steps under a control block with no read-back.  Each
    step's bias corrections are looked up at its begin in a table based at
    t0 = hp.step and covering ZERO_CTL_STEPS values of t; since t grows by at
    most one per step, the stepper reads the block back (once per
    ZERO_CTL_STEPS steps) only to move the base to the current t."""

    def __init__(self, ctl: torch.Tensor, hp: AdamWParams):
        self.ctl = ctl
        self.hp = AdamWParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step,
                              hp.decoupled_wd, hp.bias_correction)
        self.since_base = 0
        self.bucket_done = None       # see single_pass_streamed

    def _rebase(self):
        if self.since_base >= ZERO_CTL_STEPS:
            # the steps may have run on any stream: wait for the whole device
            # before reading t back, so the new base is never stale
            torch.cuda.synchronize(self.ctl.device)
            self.hp.step = control_read(self.ctl).step
            self.since_base = 0

    def two_pass(self, grad_chunks, master, exp_avg, exp_avg_sq, param_fp16,
                 max_grad_norm: float = 0.0, stream=None) -> None:
        """Check, decide (skip, loss scale, clip factor, t), update in place."""
        self._rebase()
        zero_control_begin(self.ctl, self.hp, stream=stream)
        zero_overflow_check_ctl(grad_chunks, self.ctl, stream=stream)
        zero_control_decide(self.ctl, max_grad_norm, False, stream=stream)
        zero_shard_step_ctl(grad_chunks, master, exp_avg, exp_avg_sq, param_fp16, self.hp,
                            self.ctl, stream=stream)
        self.since_base += 1

    def two_pass_buckets(self, buckets, master, exp_avg, exp_avg_sq, param_fp16,
                         max_grad_norm: float = 0.0, stream=None) -> None:
        """two_pass over a ZeRO-2 shard held as bucket slices: `buckets` is a
        sequence of (grad_chunks, offset) that covers the state exactly once.
        One check per bucket (their partial sums accumulate in a fixed order),
        one decision for the whole shard (skip, loss scale, clip factor from
        the whole shard's norm, t), then one in-place update per bucket."""
        n = master.numel()
        tiling = _Tiling(n)
        # Everything the per-bucket updates would refuse is refused here, before
        # the decision: once decide has run, t and the scale have moved and the
        # first buckets' updates would be in place.
        state = [(master, torch.float32, 4), (exp_avg, torch.float32, 4),
                 (exp_avg_sq, torch.float32, 4), (param_fp16, torch.float16, 2)]
        spans = []
        for j, (t, dt, es) in enumerate(state):
            if t.numel() != n:
                raise ValueError(f"state array {j} has {t.numel()} elements, expected {n}")
            base = _dev(t, dt, f"state array {j}")
            if base % 16:
                raise ValueError(f"state array {j} is not 16-byte aligned")
            spans.append((base, n * es))
        for k, (chunks, off) in enumerate(buckets):
            off = int(off)
            nb = chunks[0].numel()
            if off % 8:
                raise ValueError(f"bucket {k} offset {off} is not a multiple of 8")
            tiling.add(off, nb)
            for i, c in enumerate(chunks):
                if c.numel() != nb:
                    raise ValueError(f"bucket {k} chunk {i} has {c.numel()} elements, "
                                     f"expected {nb}")
                p = _dev(c, torch.float16, f"bucket {k} chunk {i}")
                if nb and p % 16:
                    raise ValueError(f"bucket {k} chunk {i} is not 16-byte aligned")
                for j, (lo, size) in enumerate(spans):
                    if nb and p < lo + size and lo < p + 2 * nb:
                        raise ValueError(f"bucket {k} chunk {i} overlaps state array {j}")
        if not tiling.complete():
            raise ValueError(f"the buckets cover {tiling.covered} elements of a "
                             f"{n}-element state")
        self._rebase()
        zero_control_begin(self.ctl, self.hp, stream=stream)
        for chunks, _ in buckets:
            zero_overflow_check_ctl(chunks, self.ctl, stream=stream)
        zero_control_decide(self.ctl, max_grad_norm, False, stream=stream)
        for chunks, off in buckets:
            nb = chunks[0].numel()
            zero_shard_step_ctl(chunks, *(t[off:off + nb] for t in
                                          (master, exp_avg, exp_avg_sq, param_fp16)),
                                self.hp, self.ctl, stream=stream)
        self.since_base += 1

    def single_pass(self, grad_chunks, copies, stream=None) -> None:
        """Fused update from copy cur into the other, then decide and commit."""
        self._rebase()
        zero_control_begin(self.ctl, self.hp, stream=stream)
        zero_shard_step_out_ctl(grad_chunks, copies, self.hp, self.ctl, stream=stream)
        zero_control_decide(self.ctl, 0.0, True, stream=stream)
        self.since_base += 1

    def single_pass_buckets(self, slices: BucketSlices, copies, stream=None) -> None:
        """single_pass over the bucket slices of a ZeRO-2 shard."""
        self._rebase()
        zero_control_begin(self.ctl, self.hp, stream=stream)
        zero_shard_step_buckets_ctl(slices, copies, self.hp, self.ctl, stream=stream)
        zero_control_decide(self.ctl, 0.0, True, stream=stream)
        self.since_base += 1

    def single_pass_page_literal(self, grad_chunks, mean_fp16: torch.Tensor, copies,
                                 stream=None) -> None:
        """The page-literal split under the control block: the owner's
        gradient mean stored as fp16 in mean_fp16 (it does not depend on the
        loss scale), then the single-pass update from it as a one-chunk step,
        which unscales by the block's S and fuses the flag and squared norm
        of g = fp32(mean16) / S; then decide and commit."""
        self._rebase()
        zero_control_begin(self.ctl, self.hp, stream=stream)
        zero_reduce_mean_fp16(grad_chunks, mean_fp16, stream=stream)
        zero_shard_step_out_ctl([mean_fp16], copies, self.hp, self.ctl, stream=stream)
        zero_control_decide(self.ctl, 0.0, True, stream=stream)
        self.since_base += 1

    def prepare_single_pass(self, grad_chunks, copies, stream=None) -> "PreparedSinglePass":
        """single_pass with its arguments marshalled once: for short steps,
        where the per-call argument checks and pointer tables cost host time
        comparable to the kernels.  See PreparedSinglePass."""
        return PreparedSinglePass(self, grad_chunks, copies, stream)

    def single_pass_streamed(self, arrivals, copies, stream=None, side_streams=(),
                             track_done: bool = True) -> None:
        """single_pass over a shard whose gradients arrive bucket by bucket.
        `arrivals` yields (grad_chunks, offset) in arrival order; each bucket
        is updated as it is yielded, from copy cur into the other at state
        elements [offset, offset + len(chunk)), and the decision and commit
        follow the last.  The buckets must cover the state arrays exactly
        once: a bucket outside the state or overlapping an earlier one is
        refused before its update is enqueued, and a shortfall after the
        last; either way ValueError is raised before the decision, so nothing
        is committed.

        Work runs on `stream` (the current stream if None).  With
        `side_streams`, bucket k's update runs on side_streams[k % len], so
        consecutive updates overlap each other's start and finish; the
        decision waits for all of them.  A bucket yielded as (grad_chunks,
        offset) waits, on its side stream, for everything enqueued on
        `stream` so far (its arrival); one yielded as (grad_chunks, offset,
        ready) waits for the event `ready` instead (recorded where its chunks
        were produced), or for nothing if ready is None (chunks already in
        place).  With side streams and track_done, after each bucket's update
        is enqueued `bucket_done` holds an event recorded after it on the
        stream that runs it, before the generator is asked for the next
        bucket; a generator that refills a chunk buffer must first make
        `stream` wait on the bucket_done event of the update that last read
        that buffer.  Without side streams stream order already implies that
        wait, and bucket_done stays None.  Side streams pay off when the updates are
        short (tens of microseconds, as for ZeRO-2 buckets of a few million
        params), where one update's ramp-up and drain can hide under its
        neighbour's; for updates of milliseconds they cost a little."""
        self._rebase()
        main = torch.cuda.current_stream() if stream is None else stream
        n = copies[0][0].numel()
        tiling = _Tiling(n)
        # the copies are checked once; a bucket's state pointers are then the
        # base pointers plus its offset (fp32 master, m, v; fp16 params)
        dts = (torch.float32, torch.float32, torch.float32, torch.float16)
        bases = []
        for j in range(4):
            pair = []
            for k in range(2):
                t = copies[k][j]
                if t.numel() != n:
                    raise ValueError(f"copy {k} array {j} has {t.numel()} elements, expected {n}")
                pair.append(_dev(t, dts[j], f"copy {k} array {j}"))
            bases.append((pair, t.element_size()))
        ctl_ptr = _ctl(self.ctl)
        zero_control_begin(self.ctl, self.hp, stream=main)
        used = set()
        self.bucket_done = None
        # one "arrived" event per side stream, re-recorded for each bucket: a
        # wait binds to the record that precedes it, so reuse is safe
        arrived = [torch.cuda.Event() for _ in side_streams]
        try:
            for k, item in enumerate(arrivals):
                chunks, off = item[0], int(item[1])
                ready = item[2] if len(item) > 2 else _ON_STREAM
                nb = chunks[0].numel()
                tiling.add(off, nb)           # refused before its update is enqueued
                ptrs = []
                for i, c in enumerate(chunks):
                    if c.numel() != nb:
                        raise ValueError(f"grad_chunks[{i}] has {c.numel()} elements, "
                                         f"expected {nb}")
                    ptrs.append(_dev(c, torch.float16, f"grad_chunks[{i}]"))
                tables = [_ptr_array([p + off * es for p in pair]) for pair, es in bases]
                run_on = main
                if side_streams:
                    i = k % len(side_streams)
                    run_on = side_streams[i]
                    if i not in used:                # first use this step: after begin
                        arrived[i].record(main)
                        run_on.wait_event(arrived[i])
                    if ready is _ON_STREAM:
                        arrived[i].record(main)
                        run_on.wait_event(arrived[i])
                    elif ready is not None:
                        run_on.wait_event(ready)
                    used.add(i)
                _check(lib.zero_shard_step_out_ctl(_ptr_array(ptrs), len(ptrs), nb, *tables,
                                                   ctypes.byref(self.hp), ctl_ptr,
                                                   _stream(run_on)))
                if side_streams and track_done:
                    self.bucket_done = torch.cuda.Event()
                    self.bucket_done.record(run_on)
        finally:
            # later work on `stream` (a decision, the next step's begin) comes
            # after every update, also when a bucket was refused
            for i in sorted(used):
                joined = torch.cuda.Event()
                joined.record(side_streams[i])
                main.wait_event(joined)
        if not tiling.complete():
            raise ValueError(f"the buckets cover {tiling.covered} elements of a "
                             f"{n}-element state")
        zero_control_decide(self.ctl, 0.0, True, stream=main)
        self.since_base += 1


class PreparedSinglePass:
    """One device-controlled single-pass step (begin, fused update from copy
    cur into the other, decide and commit) over fixed tensors, with the
    dtype, device, layout and length checks done and the pointer tables built
    once.  Each call then makes the three library calls, which still
    validate their arguments.  The tensors are kept referenced; their storage
    must not be resized or replaced while the object is in use."""

    def __init__(self, stepper: DeviceStepper, grad_chunks, copies, stream=None):
        n = copies[0][0].numel()
        for k, cp in enumerate(copies):
            for j, t in enumerate(cp):
                if t.numel() != n:
                    raise ValueError(f"copy {k} array {j} has {t.numel()} elements, expected {n}")
        for i, c in enumerate(grad_chunks):
            if c.numel() != n:
                raise ValueError(f"grad_chunks[{i}] has {c.numel()} elements, expected {n}")
        ptrs = [_dev(c, torch.float16, f"grad_chunks[{i}]") for i, c in enumerate(grad_chunks)]
        dts = (torch.float32, torch.float32, torch.float32, torch.float16)
        tables = [_ptr_array([_dev(copies[k][j], dts[j], f"copy {k} array {j}")
                              for k in range(2)]) for j in range(4)]
        self.stepper = stepper
        self._keep = (list(grad_chunks), [tuple(cp) for cp in copies])
        self._ctl = _ctl(stepper.ctl)
        self._stream = _stream(stream)
        self._args = (_ptr_array(ptrs), len(ptrs), n, *tables, ctypes.byref(stepper.hp),
                      self._ctl, self._stream)

    def __call__(self) -> None:
        st = self.stepper
        st._rebase()
        _check(lib.zero_control_begin(self._ctl, ctypes.byref(st.hp), self._stream))
        _check(lib.zero_shard_step_out_ctl(*self._args))
        _check(lib.zero_control_decide(self._ctl, 0.0, 1, self._stream))
        st.since_base += 1


# ---------------------------------------------------------------------------
# Checkpoint and resume: the shard's state is its four arrays plus the step
# control block (loss scale, t, current copy); nothing else carries over.
# ---------------------------------------------------------------------------

def save_shard_state(path: str, master: torch.Tensor, exp_avg: torch.Tensor,
                     exp_avg_sq: torch.Tensor, param_fp16: torch.Tensor,
                     ctl: Optional[torch.Tensor] = None) -> None:
    """Write the shard's state (and control block, if any) as raw tensors to
    a safetensors file."""
    from safetensors.torch import save_file
    tensors = {"master": master, "exp_avg": exp_avg, "exp_avg_sq": exp_avg_sq,
               "param_fp16": param_fp16}
    if ctl is not None:
        tensors["control"] = ctl
    save_file({k: v.detach().contiguous().cpu() for k, v in tensors.items()}, path)


def load_shard_state(path: str, device) -> dict:
    """The tensors save_shard_state wrote, on `device`, bit for bit."""
    from safetensors.torch import load_file
    return {k: v.to(device) for k, v in load_file(path).items()}
