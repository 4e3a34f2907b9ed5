"""The C ABI on the host: the library loads, exports what the header
declares, rejects bad arguments before any launch, and its host-only loss
scaler walks the same states as the oracle's.  No device work runs here:
every call below either fails validation or is host-only."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle.loss_scale as ols
import sharded_mixed_precision_step_amd as zs

pytestmark = pytest.mark.cpu

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "zero_step.h")
TWIN_HEADER = os.path.join(INCLUDE, "zero_twin.h")

A = 0x7f0000001000          # a 16-byte aligned fake device address (never dereferenced)


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(zs.EXPORTED)
    lib = ctypes.CDLL(zs.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm


def test_measurement_aids_live_in_their_own_library():
    """The step library exports the step calls only; the benchmark's twin and
    read stream are in libzerotwin.so, which exports what zero_twin.h
    declares."""
    from sharded_mixed_precision_step_amd import twin as zt
    names = declared_functions(TWIN_HEADER)
    assert set(names) == set(zt.EXPORTED)
    lib = ctypes.CDLL(zt.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm
    step_lib = ctypes.CDLL(zs.LIB_PATH)
    for nm in ("zero_traffic_twin", "zero_stream_read"):
        assert not hasattr(step_lib, nm), nm


def test_single_hip_runtime_in_process():
    maps = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln]
    assert len(set(maps)) == 1, set(maps)


def _ptrs(*p):
    return zs._ptr_array(list(p))


def _check(*args):
    return zs.lib.zero_overflow_check(*args)


def _step(chunks, n_chunks, n, scale, master, m, v, p16, hp, flag=None, sq=None):
    return zs.lib.zero_shard_step(chunks, n_chunks, n, scale, master, m, v, p16,
                                  ctypes.byref(hp) if hp is not None else None, flag, sq, None)


def _hp(**kw):
    d = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1,
             decoupled_wd=1, bias_correction=1)
    d.update(kw)
    return zs.AdamWParams(**d)


def _last():
    return zs.lib.zero_last_error_string().decode()


@pytest.mark.parametrize("args,code", [
    ((None, 3, 10, 1024.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 0, 10, 1024.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(*[A] * 65), 65, 10, 1024.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 3, -1, 1024.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 3, 10, 0.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 3, 10, float("inf"), A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 3, 10, float("nan"), A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 3, 10, -2.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, 0, A), 3, 10, 1024.0, A, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A + 2, A), 3, 10, 1024.0, A, None, None), zs.ZERO_EALIGN),
    ((_ptrs(A, A, A), 3, 10, 1024.0, None, None, None), zs.ZERO_EINVAL),
    ((_ptrs(A, A, A), 3, 10, 1024.0, A + 2, None, None), zs.ZERO_EALIGN),
    ((_ptrs(A, A, A), 3, 10, 1024.0, A, A + 4, None), zs.ZERO_EALIGN),
])
def test_overflow_check_rejects(args, code):
    assert _check(*args) == code
    assert _last()


def test_zero_length_is_a_noop():
    assert _check(_ptrs(A, A, A), 3, 0, 1024.0, A, None, None) == zs.ZERO_OK
    assert _last() == ""
    assert _step(_ptrs(A, A), 2, 0, 1.0, A, A + 4096, A + 8192, A + 12288, _hp()) == zs.ZERO_OK
    # with n == 0 no array is read, so empty (NULL) arrays are accepted ...
    assert _check(_ptrs(0, 0), 2, 0, 4.0, A, None, None) == zs.ZERO_OK
    assert _step(_ptrs(0), 1, 0, 1.0, None, None, None, None, _hp()) == zs.ZERO_OK
    # ... but scalars are still checked
    assert _step(_ptrs(0), 1, 0, 1.0, None, None, None, None, _hp(step=0)) == zs.ZERO_EINVAL
    assert _check(_ptrs(0, 0), 2, 0, -4.0, A, None, None) == zs.ZERO_EINVAL


@pytest.mark.parametrize("kw", [
    dict(lr=-1e-3), dict(beta1=1.0), dict(beta1=-0.1), dict(beta2=1.0), dict(eps=-1.0),
    dict(weight_decay=-0.01), dict(step=0), dict(lr=float("nan")), dict(eps=float("inf")),
])
def test_shard_step_rejects_hyperparameters(kw):
    B = A + (1 << 20)
    rc = _step(_ptrs(A, A), 2, 16, 1024.0, B, B + 4096, B + 8192, B + 12288, _hp(**kw))
    assert rc == zs.ZERO_EINVAL, (kw, _last())


def test_shard_step_rejects_bad_state():
    B = A + (1 << 20)
    n = 1000
    good = (B, B + 4 * n, B + 8 * n, B + 12 * n)
    assert _step(_ptrs(A), 1, n, 1.0, *good[:3], None, _hp()) == zs.ZERO_EINVAL
    assert _step(_ptrs(A), 1, n, 1.0, good[0] + 8, *good[1:], _hp()) == zs.ZERO_EALIGN
    assert _step(_ptrs(A), 1, n, 1.0, good[0], good[0] + 16, *good[2:], _hp()) == zs.ZERO_EINVAL
    assert "overlaps" in _last()
    # a chunk overlapping the master weights
    assert _step(_ptrs(B + 16), 1, n, 1.0, *good, _hp()) == zs.ZERO_EINVAL
    assert _step(_ptrs(A), 1, n, 1.0, *good, None) == zs.ZERO_EINVAL
    assert _step(_ptrs(A), 1, n, 1.0, *good, _hp(), A + 2) == zs.ZERO_EALIGN


def _step_out(chunks, n_chunks, n, ins, outs, hp, flag=None, sq=None):
    return zs.lib.zero_shard_step_out(chunks, n_chunks, n, 1.0, *ins, *outs,
                                      ctypes.byref(hp) if hp is not None else None, flag, sq,
                                      None)


def test_shard_step_out_rejects_bad_state():
    """Out-of-place step: every output must be 16-byte aligned and may equal
    its own input exactly, but may share no byte with any other input, any
    other output or a gradient chunk."""
    B = A + (1 << 20)
    n = 1000
    ins = (B, B + 4 * n, B + 8 * n)
    C = B + (1 << 20)
    outs = (C, C + 4 * n, C + 8 * n, C + 12 * n)
    ch = _ptrs(A)
    # missing or misaligned arrays
    assert _step_out(ch, 1, n, (None,) + ins[1:], outs, _hp()) == zs.ZERO_EINVAL
    assert _step_out(ch, 1, n, ins, outs[:3] + (None,), _hp()) == zs.ZERO_EINVAL
    assert _step_out(ch, 1, n, (ins[0] + 4,) + ins[1:], outs, _hp()) == zs.ZERO_EALIGN
    assert _step_out(ch, 1, n, ins, (outs[0] + 8,) + outs[1:], _hp()) == zs.ZERO_EALIGN
    # an output inside another input, shifted inside its own input, or on a chunk
    assert _step_out(ch, 1, n, ins, (ins[1],) + outs[1:], _hp()) == zs.ZERO_EINVAL
    assert "overlaps" in _last()
    assert _step_out(ch, 1, n, ins, (ins[0] + 16,) + outs[1:], _hp()) == zs.ZERO_EINVAL
    assert _step_out(ch, 1, n, ins, outs[:3] + (ins[2] + 32,), _hp()) == zs.ZERO_EINVAL
    assert _step_out(_ptrs(C + 4 * n + 64), 1, n, ins, outs, _hp()) == zs.ZERO_EINVAL
    # two outputs on each other
    assert _step_out(ch, 1, n, ins, (outs[0], outs[0] + 16) + outs[2:], _hp()) == zs.ZERO_EINVAL
    # bad hyperparameters and flag alignment
    assert _step_out(ch, 1, n, ins, outs, _hp(step=0)) == zs.ZERO_EINVAL
    assert _step_out(ch, 1, n, ins, outs, None) == zs.ZERO_EINVAL
    assert _step_out(ch, 1, n, ins, outs, _hp(), A + 2) == zs.ZERO_EALIGN
    # n == 0 is a no-op whatever the pointers
    assert _step_out(_ptrs(0), 1, 0, (None, None, None), (None,) * 4, _hp()) == zs.ZERO_OK


def test_traffic_twin_rejects_what_the_step_rejects():
    """The traffic twin takes the out-of-place step's arrays under its rules."""
    B = A + (1 << 20)
    n = 1000
    ins = (B, B + 4 * n, B + 8 * n)
    C = B + (1 << 20)
    outs = (C, C + 4 * n, C + 8 * n, C + 12 * n)
    from sharded_mixed_precision_step_amd import twin as zt
    twin = lambda ch, nc, nn, i, o: zt.lib.zero_traffic_twin(ch, nc, nn, *i, *o, None)
    assert twin(_ptrs(A), 0, n, ins, outs) == zs.ZERO_EINVAL
    assert twin(_ptrs(A + 2), 1, n, ins, outs) == zs.ZERO_EALIGN
    assert twin(_ptrs(A), 1, -1, ins, outs) == zs.ZERO_EINVAL
    assert twin(_ptrs(A), 1, n, (None,) + ins[1:], outs) == zs.ZERO_EINVAL
    assert twin(_ptrs(A), 1, n, ins, (outs[0] + 8,) + outs[1:]) == zs.ZERO_EALIGN
    assert twin(_ptrs(A), 1, n, ins, (ins[1],) + outs[1:]) == zs.ZERO_EINVAL
    assert twin(_ptrs(C + 64), 1, n, ins, outs) == zs.ZERO_EINVAL          # chunk on an output
    assert "grad_chunks[0]" in zt.lib.zero_twin_last_error_string().decode()
    assert twin(_ptrs(0), 1, 0, (None,) * 3, (None,) * 4) == zs.ZERO_OK    # n == 0: no-op
    read = lambda src, nbytes, sink: zt.lib.zero_stream_read(src, nbytes, sink, None)
    assert read(A, 24, A) == zs.ZERO_EINVAL                                 # not 16-byte units
    assert read(A + 8, 32, A) == zs.ZERO_EALIGN
    assert read(A, 32, A + 2) == zs.ZERO_EALIGN
    assert read(None, 32, A) == zs.ZERO_EINVAL
    assert read(None, 0, None) == zs.ZERO_OK                                # nothing to read


def _buckets(specs, n_chunks, n_state, ins, outs, hp, flag=None):
    """specs: (chunk pointers, n, offset) per slice."""
    keep = []
    table = (zs.BucketSliceC * max(len(specs), 1))()
    for k, (ptrs, n, off) in enumerate(specs):
        arr = _ptrs(*ptrs) if ptrs is not None else None
        keep.append(arr)
        table[k].grad_chunks = (ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
                                if arr is not None else None)
        table[k].n = n
        table[k].offset = off
    return zs.lib.zero_shard_step_buckets(table, len(specs), n_chunks, 1024.0, n_state, *ins,
                                          *outs, ctypes.byref(hp) if hp is not None else None,
                                          flag, None, None)


def test_shard_step_buckets_rejects_bad_slices():
    n_state = 4096
    B = A + (1 << 24)
    ins = (B, B + 4 * n_state, B + 8 * n_state)
    C = B + (1 << 20)
    outs = (C, C + 4 * n_state, C + 8 * n_state, C + 12 * n_state)
    ch = [A, A + 65536]
    ok = [(ch, 1000, 0), (ch, 1000, 1024)]
    # a well-formed table fails only at launch, which never happens here: use
    # one bad field at a time
    assert _buckets([(ch, 1000, 4)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EALIGN
    assert _buckets([(ch, 1000, 3200)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert "past n_state" in _last()
    assert _buckets([(ch, -1, 0)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets([(ch, 8, -8)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets([(None, 8, 0)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets([([A, 0], 8, 0)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets([([A, A + 2], 8, 0)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EALIGN
    # two slices sharing state elements, in either order
    assert _buckets([(ch, 1000, 0), (ch, 1000, 992)], 2, n_state, ins, outs, _hp()) \
        == zs.ZERO_EINVAL
    assert "overlap" in _last()
    assert _buckets([(ch, 1000, 992), (ch, 1000, 0)], 2, n_state, ins, outs, _hp()) \
        == zs.ZERO_EINVAL
    # an output over a chunk, an output over another input
    assert _buckets([([C + 64, A], 8, 0)], 2, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets(ok, 2, n_state, ins, (ins[1],) + outs[1:], _hp()) == zs.ZERO_EINVAL
    # scalars
    assert _buckets(ok, 0, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets(ok, 65, n_state, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets(ok, 2, n_state, ins, outs, _hp(step=0)) == zs.ZERO_EINVAL
    assert _buckets(ok, 2, n_state, ins, outs, None) == zs.ZERO_EINVAL
    assert _buckets(ok, 2, -1, ins, outs, _hp()) == zs.ZERO_EINVAL
    assert _buckets(ok, 2, n_state, ins, outs, _hp(), A + 2) == zs.ZERO_EALIGN
    # only empty slices, or none: a no-op whatever the state pointers
    assert _buckets([(None, 0, 0)], 2, n_state, (None,) * 3, (None,) * 4, _hp()) == zs.ZERO_OK
    assert _buckets([], 2, 0, (None,) * 3, (None,) * 4, _hp()) == zs.ZERO_OK


def test_reduce_mean_and_accumulate_reject_bad_arguments():
    B = A + (1 << 20)
    n = 1000
    rm = lambda chunks, nc, nn, mean, S=1.0, flag=None: zs.lib.zero_reduce_mean_fp16(
        chunks, nc, nn, S, mean, flag, None, None)
    assert rm(_ptrs(A, A + 4096), 2, n, None) == zs.ZERO_EINVAL
    assert rm(_ptrs(A, A + 4096), 2, n, B + 2) == zs.ZERO_EALIGN
    assert rm(_ptrs(A, A + 4096), 2, n, A + 1024) == zs.ZERO_EINVAL      # over a chunk
    assert rm(_ptrs(A, A + 4096), 2, n, B, S=0.0) == zs.ZERO_EINVAL
    assert rm(_ptrs(A, A + 4096), 2, n, B, flag=A + 2) == zs.ZERO_EALIGN
    assert rm(_ptrs(A, A + 4), 2, n, B) == zs.ZERO_EALIGN
    assert rm(_ptrs(0, 0), 2, 0, None) == zs.ZERO_OK                    # n == 0: no-op
    acc = lambda ch, nn, idx, nc, a, mean: zs.lib.zero_accumulate_chunk(ch, nn, idx, nc, a,
                                                                        mean, None)
    assert acc(A, n, 3, 3, B, B + 8192) == zs.ZERO_EINVAL               # index past N - 1
    assert acc(A, n, -1, 3, B, B + 8192) == zs.ZERO_EINVAL
    assert acc(A, n, 0, 0, B, B + 8192) == zs.ZERO_EINVAL
    assert acc(A, n, 0, 3, None, None) == zs.ZERO_EINVAL                # first needs acc
    assert acc(A, n, 1, 3, B + 4, None) == zs.ZERO_EALIGN
    assert acc(A, n, 2, 3, B, None) == zs.ZERO_EINVAL                   # last needs the mean
    assert acc(A, n, 2, 3, B, B + 1024) == zs.ZERO_EINVAL               # mean over acc
    assert acc(A, n, 0, 3, A + 512, None) == zs.ZERO_EINVAL             # acc over the chunk
    assert acc(A + 8, n, 0, 1, None, B) == zs.ZERO_EALIGN
    assert acc(None, n, 0, 1, None, B) == zs.ZERO_EINVAL
    assert acc(None, 0, 0, 1, None, None) == zs.ZERO_OK                 # n == 0: no-op


def test_allocation_free_fold_refuses_what_it_cannot_hold():
    """n above the library accumulator's ZERO_FOLD_SCRATCH_ELEMS is refused
    with ZERO_ERANGE before anything reaches the device; bad arguments are
    refused as zero_accumulate_chunk refuses them."""
    B = A + (1 << 24)
    fold = lambda ch, nn, idx, nc, mean: zs.lib.zero_accumulate_chunk_noalloc(ch, nn, idx, nc,
                                                                               mean, None)
    assert fold(A, zs.ZERO_FOLD_SCRATCH_ELEMS + 1, 0, 8, B) == zs.ZERO_ERANGE
    assert "allocation-free" in _last()
    assert fold(A, 100, 8, 8, B) == zs.ZERO_EINVAL
    assert fold(A, 100, 0, 65, B) == zs.ZERO_EINVAL
    assert fold(A, -1, 0, 8, B) == zs.ZERO_EINVAL
    assert fold(A + 8, 100, 0, 8, B) == zs.ZERO_EALIGN
    assert fold(A, 100, 7, 8, None) == zs.ZERO_EINVAL                  # the last needs the mean
    assert fold(A, 100, 7, 8, B + 8) == zs.ZERO_EALIGN
    assert fold(None, 0, 0, 8, None) == zs.ZERO_OK                       # n == 0: no-op


def test_control_init_and_ctl_calls_reject_bad_arguments():
    ctl = zs.StepControl()
    good = zs.LossScaler.create(scale=65536.0, growth_interval=3)
    assert zs.lib.zero_control_init(ctypes.byref(ctl), ctypes.byref(good), 7) == zs.ZERO_OK
    assert (ctl.scale, ctl.step, ctl.step_used, ctl.growth_interval, ctl.cur) == \
        (65536.0, 7, 7, 3, 0)
    assert ctl.clip_coef == 1.0 and ctl.overflow == 0 and ctl.error == 0
    assert zs.lib.zero_control_init(ctypes.byref(ctl), ctypes.byref(good), 0) == zs.ZERO_EINVAL
    bad = zs.LossScaler.create(scale=float("inf"))
    assert zs.lib.zero_control_init(ctypes.byref(ctl), ctypes.byref(bad), 1) == zs.ZERO_EINVAL
    assert zs.lib.zero_control_init(None, ctypes.byref(good), 1) == zs.ZERO_EINVAL
    # device-side calls: bad pointers are refused before any launch
    hp = _hp()
    assert zs.lib.zero_control_begin(None, ctypes.byref(hp), None) == zs.ZERO_EINVAL
    assert zs.lib.zero_control_begin(A + 4, ctypes.byref(hp), None) == zs.ZERO_EALIGN
    assert zs.lib.zero_control_begin(A, None, None) == zs.ZERO_EINVAL       # no table
    bad_hp = _hp(step=0)
    assert zs.lib.zero_control_begin(A, ctypes.byref(bad_hp), None) == zs.ZERO_EINVAL
    bad_hp = _hp(beta2=1.0)
    assert zs.lib.zero_control_begin(A, ctypes.byref(bad_hp), None) == zs.ZERO_EINVAL
    assert zs.lib.zero_control_decide(A, float("nan"), 0, None) == zs.ZERO_EINVAL
    assert zs.lib.zero_control_decide(None, 1.0, 0, None) == zs.ZERO_EINVAL
    assert zs.lib.zero_overflow_check_ctl(_ptrs(A), 1, 10, None, None) == zs.ZERO_EINVAL
    assert zs.lib.zero_overflow_check_ctl(_ptrs(A + 2), 1, 10, A, None) == zs.ZERO_EALIGN
    B = A + (1 << 20)
    n = 1000
    st = (B, B + 4 * n, B + 8 * n, B + 12 * n)
    step_ctl = lambda ch, s4, hp, c: zs.lib.zero_shard_step_ctl(
        ch, 1, n, *s4, ctypes.byref(hp) if hp is not None else None, c, None)
    assert step_ctl(_ptrs(A), st, _hp(), None) == zs.ZERO_EINVAL
    assert step_ctl(_ptrs(A), st, _hp(step=0), A) == zs.ZERO_EINVAL
    assert step_ctl(_ptrs(A), (st[0], st[0] + 16) + st[2:], _hp(), A) == zs.ZERO_EINVAL
    assert step_ctl(_ptrs(B + 64), st, _hp(), A) == zs.ZERO_EINVAL          # chunk on the state
    C = B + (1 << 20)
    other = (C, C + 4 * n, C + 8 * n, C + 12 * n)
    out_ctl = lambda c0, c1: zs.lib.zero_shard_step_out_ctl(
        _ptrs(A), 1, n, *[_ptrs(c0[j], c1[j]) for j in range(4)], ctypes.byref(_hp()), A, None)
    assert out_ctl(st, st) == zs.ZERO_EINVAL                                # the same copy twice
    assert out_ctl(st, (st[1],) + other[1:]) == zs.ZERO_EINVAL               # copies overlap
    assert out_ctl(st, (other[0] + 4,) + other[1:]) == zs.ZERO_EALIGN
    assert out_ctl(st, other[:3] + (A,)) == zs.ZERO_EINVAL                   # over the chunk
    # the bucket table under the block must tile the state exactly
    table = (zs.BucketSliceC * 2)()
    keep = [_ptrs(A), _ptrs(A + 65536)]
    for k, (nn, off) in enumerate(((504, 0), (496, 504))):
        table[k].grad_chunks = ctypes.cast(keep[k], ctypes.POINTER(ctypes.c_void_p))
        table[k].n, table[k].offset = nn, off
    bctl = lambda count, n_state: zs.lib.zero_shard_step_buckets_ctl(
        table, count, 1, n_state, *[_ptrs(st[j], other[j]) for j in range(4)],
        ctypes.byref(_hp()), A, None)
    assert bctl(1, n) == zs.ZERO_EINVAL                                     # a gap at the end
    assert "cover" in _last()
    table[1].offset = 512
    assert bctl(2, 1008) == zs.ZERO_EINVAL                                   # a gap between


def _flatten(ptrs, numels, align, pad, bucket, cap):
    nt = len(numels)
    offs = (ctypes.c_int64 * (nt + 1))()
    rc = zs.lib.zero_bucket_flatten(_ptrs(*ptrs) if ptrs else None,
                                    (ctypes.c_int64 * max(nt, 1))(*numels), nt, align, pad,
                                    bucket, cap, offs, None)
    return rc, list(offs)


def test_flatten_validation_and_layout():
    B = A + (1 << 24)
    assert _flatten([], [], 256, 512, B, 0) == (zs.ZERO_OK, [0])
    assert _flatten([A, A + 4096], [0, 0], 256, 512, B, 0) == (zs.ZERO_OK, [0, 0, 0])
    rc, offs = _flatten([A, A + 4096, A + 8192], [5, 300, 1], 256, 512, B, 1000)
    assert rc == zs.ZERO_ERANGE and offs == [0, 256, 768, 1024]
    assert _flatten([A], [5], 256, 512, B + 8, 4096)[0] == zs.ZERO_EALIGN
    assert _flatten([A + 1], [5], 256, 512, B, 4096)[0] == zs.ZERO_EALIGN
    assert _flatten([A], [-5], 256, 512, B, 4096)[0] == zs.ZERO_EINVAL
    assert _flatten([0], [5], 256, 512, B, 4096)[0] == zs.ZERO_EINVAL
    assert _flatten([A], [5], 0, 512, B, 4096)[0] == zs.ZERO_EINVAL
    assert _flatten([B + 64], [5], 256, 512, B, 4096)[0] == zs.ZERO_EINVAL   # source inside bucket


def _flatten_batch(specs, align, pad):
    """specs: (tensor pointers, numels, bucket, capacity) per bucket."""
    table = (zs.FlattenBucketC * max(len(specs), 1))()
    keep, offs = [], []
    for k, (ptrs, numels, bucket, cap) in enumerate(specs):
        nt = len(numels)
        parr = _ptrs(*ptrs) if ptrs else _ptrs(0)
        narr = (ctypes.c_int64 * max(nt, 1))(*numels)
        oarr = (ctypes.c_int64 * (nt + 1))()
        keep.append((parr, narr))
        offs.append(oarr)
        table[k].tensors = ctypes.cast(parr, ctypes.POINTER(ctypes.c_void_p))
        table[k].numels = ctypes.cast(narr, ctypes.POINTER(ctypes.c_int64))
        table[k].offsets_out = ctypes.cast(oarr, ctypes.POINTER(ctypes.c_int64))
        table[k].bucket, table[k].bucket_capacity, table[k].n_tensors = bucket, cap, nt
    rc = zs.lib.zero_bucket_flatten_batch(table, len(specs), align, pad, None)
    return rc, [list(o) for o in offs]


def test_flatten_batch_validates_every_bucket_first():
    """The batch refuses a bad bucket anywhere in it, names it, and fills the
    offsets of the buckets before it; empty batches and empty buckets are
    no-ops."""
    B = A + (1 << 24)
    C = B + (1 << 24)
    assert _flatten_batch([], 256, 512) == (zs.ZERO_OK, [])
    assert _flatten_batch([([], [], B, 0), ([A], [0], C, 0)], 256, 512) == \
        (zs.ZERO_OK, [[0], [0, 0]])
    rc, offs = _flatten_batch([([A], [5], B, 4096), ([A + 4096, A + 8192], [300, 1], C, 700)],
                              256, 512)
    assert rc == zs.ZERO_ERANGE and offs == [[0, 512], [0, 512, 1024]]
    assert "bucket 1" in _last()
    assert _flatten_batch([([A], [5], B, 4096), ([A], [5], B + 512, 4096)],
                          256, 512)[0] == zs.ZERO_EINVAL                    # buckets overlap
    assert _flatten_batch([([A], [5], B, 4096), ([B + 64], [5], C, 4096)],
                          256, 512)[0] == zs.ZERO_EINVAL                    # source on bucket 0
    assert _flatten_batch([([A], [5], B, 4096), ([A + 1], [5], C, 4096)],
                          256, 512)[0] == zs.ZERO_EALIGN
    assert zs.lib.zero_bucket_flatten_batch(None, 1, 256, 512, None) == zs.ZERO_EINVAL
    assert zs.lib.zero_bucket_flatten_batch(None, -1, 256, 512, None) == zs.ZERO_EINVAL


def test_scaler_matches_oracle_on_forced_sequences():
    rng = np.random.default_rng(11)
    for interval in (1, 3, 1000):
        for trial in range(20):
            flags = rng.random(60) < rng.choice([0.05, 0.3, 0.8])
            c = zs.LossScaler.create(scale=65536.0, growth_interval=interval,
                                     min_scale=4.0, max_scale=2.0 ** 18)
            o = ols.ScalerState(scale=65536.0, growth_interval=interval, min_scale=4.0,
                                max_scale=2.0 ** 18)
            for f in flags:
                assert zs.zero_update_loss_scale(c, int(f)) == ols.update_loss_scale(o, bool(f))
                assert (c.scale, c.good_steps, c.skipped_steps) == (o.scale, o.good_steps,
                                                                    o.skipped_steps)


@pytest.mark.parametrize("field,value", [
    ("scale", 0.0), ("scale", float("inf")), ("growth_factor", 0.5), ("backoff_factor", 0.0),
    ("backoff_factor", 1.5), ("min_scale", 0.0), ("max_scale", 0.5), ("growth_interval", 0),
])
def test_scaler_rejects(field, value):
    s = zs.LossScaler.create()
    setattr(s, field, value)
    before = bytes(s)
    with pytest.raises(zs.ZeroStepError) as e:
        zs.zero_update_loss_scale(s, 1)
    assert e.value.code == zs.ZERO_EINVAL and bytes(s) == before


def test_ctypes_structs_and_constants_match_the_header(tmp_path):
    """The binding's ctypes structures have the C header's sizes and field
    offsets, and its constants the header's values, as a C compiler sees
    them."""
    import subprocess
    structs = {"zero_adamw_params": zs.AdamWParams, "zero_loss_scaler": zs.LossScaler,
               "zero_bucket_slice": zs.BucketSliceC, "zero_step_control": zs.StepControl}
    consts = ("ZERO_OK", "ZERO_EINVAL", "ZERO_EALIGN", "ZERO_ERANGE", "ZERO_EHIP",
              "ZERO_MAX_CHUNKS", "ZERO_CTL_STEPS", "ZERO_NORM_SLOTS", "ZERO_NORM_STRIDE",
              "ZERO_CHECK_PARTS")
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "zero_step.h"',
             "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    for c in consts:
        lines.append(f'printf("const {c} %d\\n", (int)({c}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    seen = 0
    for line in out.splitlines():
        a, b, v = line.split()
        if a == "const":
            assert getattr(zs, b) == int(v), b
        elif b == "sizeof":
            assert ctypes.sizeof(structs[a]) == int(v), a
        else:
            assert getattr(structs[a], b).offset == int(v), (a, b)
        seen += 1
    assert seen == len(consts) + sum(1 + len(py._fields_) for py in structs.values())


def test_kernel_digest_follows_code_not_comments():
    """The digest that ties the committed counter summary to the kernel
    sources ignores comments and layout, and sees any change of code."""
    from sharded_mixed_precision_step_amd import _build
    base = 'int f(int a) {\n  return a + 1;  // one more\n}\nconst char* s = "/* kept */";\n'
    same = '/* a header */\nint f(int a)\n{\n    return a + 1;\n}\nconst char* s = "/* kept */"; // x\n'
    other = 'int f(int a) {\n  return a + 2;\n}\nconst char* s = "/* kept */";\n'
    assert _build.code_text(base) == _build.code_text(same)
    assert _build.code_text(base) != _build.code_text(other)
    assert "/* kept */" in _build.code_text(base)
    assert re.fullmatch(r"[0-9a-f]{64}", _build.kernel_digest())


def test_bucket_tiling_refuses_overlaps_gaps_and_strays():
    """The binding's check that streamed or two-pass buckets cover the state
    exactly once: a stray or overlapping bucket is refused when it is added,
    a gap shows as an incomplete cover, in any arrival order."""
    t = zs._Tiling(100)
    for off, nb in ((40, 20), (0, 8), (60, 40), (8, 32)):
        t.add(off, nb)
    assert t.complete()
    t = zs._Tiling(100)
    t.add(0, 50)
    with pytest.raises(ValueError, match="overlaps"):
        t.add(40, 20)                  # the left neighbour's tail
    with pytest.raises(ValueError, match="overlaps"):
        t.add(49, 1)
    t.add(50, 25)
    with pytest.raises(ValueError, match="overlaps"):
        t.add(70, 10)                  # the right neighbour's head
    with pytest.raises(ValueError, match="overlaps"):
        t.add(0, 100)                  # covering several
    with pytest.raises(ValueError, match="outside"):
        t.add(90, 20)
    with pytest.raises(ValueError, match="outside"):
        t.add(-8, 8)
    t.add(80, 0)                       # empty buckets are no-ops
    assert not t.complete() and t.covered == 75      # [75, 100) is a gap
    t.add(75, 25)
    assert t.complete()
