"""The device-resident step control against the CPU oracle.

Whole steps are enqueued with no read-back: two-pass (with and without
gradient-norm clipping) and single pass (commit on the device). They walk
the same states as the oracle's step, loss scaler and t over clean and
overflowing steps. This holds over the whole shard, a bucket table, buckets
streamed as they arrive, and the two-pass flow over buckets, at N = 1..64.
Also: the two-pass norm and clip factor repeat bit for bit; a step whose t
lies outside its bias-correction table changes nothing in any flow; a
misaligned bucket is refused before the decision; the prepared step equals
the unprepared one; and a HIP graph of one step replays like the eager
calls."""
import struct

import numpy as np
import pytest
import torch

import oracle.loss_scale as ols
import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import assert_matches_oracle, device

pytestmark = pytest.mark.gpu

N, n = 8, 40_009
PLAN = [False, True, False, False, True, False, False]      # overflow injected or not


def _workload():
    base = wl.LLAMA3_8B_SHARD
    return wl.ShardWorkload(name="ctl", wid=base.wid, n=n, n_replicas=N, grad_sigma=1e-4,
                            loss_scale=65536.0, hyper=base.hyper.replace(step=3),
                            m_sigma=1e-4, v_sigma=1e-8)


def _grads(w, k, S, plant):
    g = [wl.host_fp16_grad(wl.seed_of(w.wid, 900 + k, wl.ARRAY_GRAD, i), n, w.grad_sigma, S)
         for i in range(N)]
    if plant:
        g[k % N][(97 * k) % n] = np.float16(np.inf if k % 2 else np.nan)
    return g


def _scaler():
    return (zs.LossScaler.create(scale=65536.0, growth_interval=2),
            ols.ScalerState(scale=65536.0, growth_interval=2))


def _check_control(c, os_, t, skip, want):
    assert c.scale == np.float32(os_.scale) and c.good_steps == os_.good_steps
    assert c.skipped_steps == os_.skipped_steps and c.step == t
    assert c.skip == int(skip) and c.overflow == int(want.overflow) and c.error == 0
    if not want.overflow:
        assert abs(c.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm


@pytest.mark.parametrize("clip", [0.0, 2e-3, 1e9])
def test_two_pass_sequence_matches_oracle(clip):
    """Check, decide, update in place, all on the device.  clip 0: none;
    2e-3: the update's gradient is clipped (its norm is about 7e-3, the mean
    of 8 replicas of N(0, 1e-4) over 40,009 params); 1e9: factor 1."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=901)
    d = {k: torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16")}
    scaler, os_ = _scaler()
    ctl = zs.control_new(scaler, w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    state, t = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step
    chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    for k, plant in enumerate(PLAN):
        S = os_.scale
        g = _grads(w, k, S, plant)
        for c, src in zip(chunks, g):
            c.copy_(torch.from_numpy(src))
        stepper.two_pass(chunks, d["master"], d["m"], d["v"], d["p16"], max_grad_norm=clip)
        want = ozs.shard_step_clipped(g, *state, w.hyper.replace(step=t), S, clip)
        skip = ols.update_loss_scale(os_, want.overflow)
        t += 0 if skip else 1
        c = zs.control_read(ctl)
        print(f"case: ctl two-pass clip={clip} step {k} plant={plant} S={S}", flush=True)
        _check_control(c, os_, t, skip, want)
        if not skip:
            coef = ozs.clip_coefficient(want.sqnorm, clip)
            assert abs(c.clip_coef - coef) <= 1e-6 * coef
        if clip == 2e-3 and not skip:
            assert c.clip_coef < 0.5
        if clip == 2e-3:
            # The clip factor comes from the squared norm, summed in fp64 in a
            # fixed tree order on the device and in index order by the oracle; the
            # factor can then differ by an fp32 ulp, and where the moment
            # update cancels to near zero a tiny absolute difference is many
            # ulps.  The bar here is the stated one: 1e-6 relative or 1e-9
            # absolute, fp16 params within 1 ulp.
            assert_matches_oracle(d, want, label=f"step {k} ", max_ulp=None)
        else:
            for name, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
                assert np.array_equal(d[name].cpu().numpy().view(np.uint32),
                                      ref.view(np.uint32)), (k, name)
            assert np.array_equal(d["p16"].cpu().numpy().view(np.uint16),
                                  want.p16.view(np.uint16))
        state = (want.master, want.m, want.v, want.p16)


def test_single_pass_sequence_matches_oracle():
    """Fused update into the other copy, then decide and commit on the device."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=902)
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    b = tuple(torch.full_like(x, float("nan")) for x in a)
    copies = (a, b)
    scaler, os_ = _scaler()
    ctl = zs.control_new(scaler, w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    state, t, cur = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step, 0
    chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    for k, plant in enumerate(PLAN):
        S = os_.scale
        g = _grads(w, k, S, plant)
        for c, src in zip(chunks, g):
            c.copy_(torch.from_numpy(src))
        before = [x.clone() for x in copies[cur]]
        stepper.single_pass(chunks, copies)
        want = ozs.shard_step(g, *state, w.hyper.replace(step=t), S)
        skip = ols.update_loss_scale(os_, want.overflow)
        t += 0 if skip else 1
        c = zs.control_read(ctl)
        print(f"case: ctl single-pass step {k} plant={plant} S={S}", flush=True)
        _check_control(c, os_, t, skip, want)
        if skip:
            assert c.cur == cur
            for x, y in zip(before, copies[cur]):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
            continue
        cur = 1 - cur
        assert c.cur == cur
        got = dict(zip(("master", "m", "v", "p16"), copies[cur]))
        for name, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
            assert np.array_equal(got[name].cpu().numpy().view(np.uint32),
                                  ref.view(np.uint32)), (k, name)
        assert np.array_equal(got["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))
        state = (want.master, want.m, want.v, want.p16)


def test_two_pass_without_clip_equals_host_driven_step():
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=903)
    a = {k: torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16")}
    b = {k: x.clone() for k, x in a.items()}
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    scaler, _ = _scaler()
    ctl = zs.control_new(scaler, w.hyper.step, dev)
    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).two_pass(chunks, a["master"], a["m"],
                                                             a["v"], a["p16"])
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    sq = torch.zeros(1, dtype=torch.float64, device=dev)
    r = zs.checked_step(chunks, b["master"], b["m"], b["v"], b["p16"], zs.adamw_params(w.hyper),
                        zs.LossScaler.create(scale=65536.0, growth_interval=2), fl, sq)
    torch.cuda.synchronize()
    assert not r.skipped
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


_KEPT = ("scale", "growth_factor", "backoff_factor", "min_scale", "max_scale",
         "growth_interval", "good_steps", "cur", "skipped_steps", "step")


def _bits(tensors):
    return [x.clone().view(torch.uint8) for x in tensors]


@pytest.mark.parametrize("flow", ["single_pass", "bucket_table", "streamed", "two_pass",
                                  "two_pass_buckets"])
@pytest.mark.parametrize("t_block,t0", [(100, 1), (65, 1), (5, 6)])
def test_bias_table_miss_changes_nothing(flow, t_block, t0):
    """A step whose t lies outside the table zero_control_begin was given
    (t = 100 or 65 against t0 = 1, which covers 1..64; t = 5 below t0 = 6)
    is void in every flow: error bit 0, table_miss and skip are set, and t,
    the loss scale, good_steps, skipped_steps and the current copy stay as
    they were, as do both copies of the state, bit for bit.  The two-pass
    flows decide before they update, so the miss has to be known from begin
    on; the single-pass flows must not commit the copy no kernel wrote.  With
    the table moved to cover t, the next step runs and matches the oracle."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=904)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    b = tuple(torch.full_like(x, float("nan")) for x in a)
    copies = (a, b)
    scaler = zs.LossScaler.create(scale=65536.0, growth_interval=2)
    scaler.good_steps = 1                       # a clean step would grow the scale
    ctl = zs.control_new(scaler, t_block, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper.replace(step=t0)))
    before = zs.control_read(ctl)
    snap = _bits(a) + _bits(b)
    sizes = [8 * 1000, 8 * 1001, n - 8 * 2001]
    offs = [0, 8 * 1000, 8 * 2001]
    buckets = [([c[o:o + s] for c in chunks], o) for o, s in zip(offs, sizes)]

    def run():
        if flow == "single_pass":
            stepper.single_pass(chunks, copies)
        elif flow == "bucket_table":
            stepper.single_pass_buckets(zs.BucketSlices(buckets), copies)
        elif flow == "streamed":
            stepper.single_pass_streamed(iter(buckets), copies)
        elif flow == "two_pass":
            stepper.two_pass(chunks, *a, max_grad_norm=1.0)
        else:
            stepper.two_pass_buckets(buckets, *a, max_grad_norm=1.0)

    print(f"case: bias-table miss flow={flow} t={t_block} t0={t0}", flush=True)
    run()
    c = zs.control_read(ctl)
    assert c.error & 1 and c.table_miss == 1 and c.skip == 1, (c.error, c.table_miss, c.skip)
    for name in _KEPT:
        assert getattr(c, name) == getattr(before, name), name
    for x, y in zip(snap, _bits(a) + _bits(b)):
        assert torch.equal(x, y)
    # the caller clears the error and moves the table base to t: the step runs
    host = zs.control_read(ctl)
    host.error = 0
    ctl.copy_(torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8))
    stepper.hp.step = t_block
    run()
    c = zs.control_read(ctl)
    want = ozs.shard_step_clipped(h["chunks"], h["master"], h["m"], h["v"], h["p16"],
                                  w.hyper.replace(step=t_block), 65536.0,
                                  1.0 if flow.startswith("two_pass") else 0.0)
    assert c.error == 0 and c.table_miss == 0 and c.skip == 0 and c.step == t_block + 1
    assert c.scale == 131072.0 and c.good_steps == 0       # grew on this clean step
    got = a if flow.startswith("two_pass") else copies[c.cur]
    assert_matches_oracle(dict(zip(("master", "m", "v", "p16"), got)), want, max_ulp=None)


def test_last_entry_of_the_bias_table_is_used():
    """t = t0 + ZERO_CTL_STEPS - 1, the table's last entry, is a hit: the
    single pass runs and matches the oracle at that t."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=916)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    copies = _state(h, dev)
    t = 1 + zs.ZERO_CTL_STEPS - 1
    ctl = zs.control_new(zs.LossScaler.create(scale=65536.0), t, dev)
    print(f"case: bias table last entry t={t} t0=1", flush=True)
    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper.replace(step=1))).single_pass(chunks, copies)
    c = zs.control_read(ctl)
    assert c.error == 0 and c.table_miss == 0 and c.skip == 0 and c.step == t + 1
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"],
                          w.hyper.replace(step=t), 65536.0)
    _assert_state(copies[1], want, "last table entry")


def test_two_pass_buckets_refuse_a_misaligned_bucket_before_deciding():
    """A bucket whose offset is not a multiple of 8, or whose chunks are not
    16-byte aligned, would be refused by its in-place update only after the
    decision had moved t and the scale and earlier buckets had been updated.
    two_pass_buckets refuses it first: the block and the state are left
    bit-identical."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=914)
    state = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    before = zs.control_read(ctl)
    snap = _bits(state)
    cut = 8 * 1000 + 4                               # offset of the second bucket: 4 mod 8
    bad_offset = [([c[:cut] for c in chunks], 0), ([c[cut:] for c in chunks], cut)]
    with pytest.raises(ValueError, match="multiple of 8"):
        stepper.two_pass_buckets(bad_offset, *state)
    spare = [torch.empty(n + 8, dtype=torch.float16, device=dev) for _ in range(N)]
    for sp, c in zip(spare, chunks):
        sp[1:n + 1].copy_(c)
    bad_chunk = [([c[:8 * 1000] for c in chunks], 0),
                 ([sp[1 + 8 * 1000:n + 1] for sp in spare], 8 * 1000)]   # 2 bytes off
    with pytest.raises(ValueError, match="16-byte aligned"):
        stepper.two_pass_buckets(bad_chunk, *state)
    print("case: two-pass buckets refuse a misaligned bucket", flush=True)
    c = zs.control_read(ctl)
    for name in _KEPT + ("error", "step_used"):
        assert getattr(c, name) == getattr(before, name), name
    for x, y in zip(snap, _bits(state)):
        assert torch.equal(x, y)


def test_stepping_on_a_side_stream_past_the_table_rebases_correctly():
    """Steps enqueued on a stream that is not torch's current one, past
    ZERO_CTL_STEPS of them with no synchronisation from the caller: the
    stepper's rebase waits for the device before reading t back, so no step
    misses the table and t counts every clean step."""
    dev = device()
    w = _workload()
    nn = 4_099
    h = wl.host_shard(w, n=nn, offset_seed=915)
    chunks = [torch.from_numpy(c[:nn]).to(dev) for c in h["chunks"]]
    a = tuple(torch.from_numpy(h[k][:nn]).to(dev) for k in ("master", "m", "v", "p16"))
    copies = (a, tuple(torch.empty_like(x) for x in a))
    ctl = zs.control_new(zs.LossScaler.create(scale=65536.0), w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    side = torch.cuda.Stream()
    steps = 2 * zs.ZERO_CTL_STEPS + 5
    print(f"case: {steps} single-pass steps on a side stream", flush=True)
    torch.cuda.synchronize()
    for _ in range(steps):
        stepper.single_pass(chunks, copies, stream=side)
    side.synchronize()
    c = zs.control_read(ctl)
    assert c.error == 0 and c.table_miss == 0 and c.step == w.hyper.step + steps


def test_graph_of_one_step_replays_like_eager_calls():
    """One single-pass step (begin, fused update, decide and commit) captured
    in a HIP graph and replayed five times, with eager work and device
    synchronisations between replays: after every replay the state copies
    and the control block equal those of the same steps run eagerly."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=905)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]

    def fresh():
        a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        b = tuple(torch.zeros_like(x) for x in a)
        scaler, _ = _scaler()
        ctl = zs.control_new(scaler, w.hyper.step, dev)
        return (a, b), ctl, zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))

    g_copies, g_ctl, g_stepper = fresh()
    e_copies, e_ctl, e_stepper = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_stepper.single_pass(chunks, g_copies)
    torch.cuda.synchronize()
    # capture does not run the step: the block is untouched
    assert zs.control_read(g_ctl).step == w.hyper.step
    for r in range(5):
        graph.replay()
        torch.cuda.synchronize()
        e_stepper.single_pass(chunks, e_copies)
        junk = torch.randn(1 << 20, device=dev).sum()      # unrelated eager work
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        gc, ec = zs.control_read(g_ctl), zs.control_read(e_ctl)
        print(f"case: graph replay {r}: t={gc.step} cur={gc.cur}", flush=True)
        # every field equal, except the squared norm and its slots: each slot
        # takes one fp64 atomic add per block, in whatever order the blocks
        # finish
        for name, _ in zs.StepControl._fields_:
            if name == "sqnorm":
                assert abs(gc.sqnorm - ec.sqnorm) <= 1e-12 * ec.sqnorm
            elif name in ("sqnorm_part", "check_part"):
                for a, b in zip(getattr(gc, name), getattr(ec, name)):
                    assert abs(a - b) <= 1e-12 * abs(b)
            else:
                assert getattr(gc, name) == getattr(ec, name), name
        assert gc.step == w.hyper.step + r + 1
        for cp_g, cp_e in zip(g_copies, e_copies):
            for x, y in zip(cp_g, cp_e):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_graph_of_clipped_two_pass_steps_replays_like_eager_calls():
    """The two-pass flow with clipping (begin, check, decide with the clip
    factor, update in place) captured once in a HIP graph and replayed four
    times, with eager work and synchronisations between replays: after every
    replay the state and the whole control block equal those of the same
    steps run eagerly, bit for bit (this flow's norm is reduced in a fixed
    order)."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=917)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]

    def fresh():
        a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
        return a, ctl, zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))

    g_state, g_ctl, g_st = fresh()
    e_state, e_ctl, e_st = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_st.two_pass(chunks, *g_state, max_grad_norm=2e-3)
    torch.cuda.synchronize()
    assert zs.control_read(g_ctl).step == w.hyper.step       # capture runs nothing
    for r in range(4):
        graph.replay()
        torch.cuda.synchronize()
        e_st.two_pass(chunks, *e_state, max_grad_norm=2e-3)
        junk = torch.randn(1 << 20, device=dev).sum()      # unrelated eager work
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        gc, ec = zs.control_read(g_ctl), zs.control_read(e_ctl)
        print(f"case: two-pass graph replay {r}: t={gc.step} clip={gc.clip_coef}", flush=True)
        assert bytes(gc) == bytes(ec)
        assert gc.step == w.hyper.step + r + 1 and gc.clip_coef < 1.0
        for x, y in zip(g_state, e_state):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("flow", ["bucket_table", "two_pass_buckets"])
def test_graph_of_a_bucketed_step_replays_like_eager_calls(flow):
    """A ZeRO-2 step over ragged bucket slices, captured once in a HIP graph
    and replayed four times with eager work in between: the single pass over
    a bucket table (its update launches between begin and decide), or the
    two-pass flow over the buckets (a check per bucket, the decision with a
    clip factor, an in-place update per bucket).  After every replay the
    state equals that of the eager steps bit for bit, and so does the control
    block (the squared norm to 1e-12 where per-block atomics sum it)."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=918)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    sizes = [8 * 1000, 8 * 1001, n - 8 * 2001]
    offs = [0, 8 * 1000, 8 * 2001]
    buckets = [([c[o:o + sz] for c in chunks], o) for o, sz in zip(offs, sizes)]
    table = zs.BucketSlices(buckets)

    def fresh():
        a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        copies = (a, tuple(torch.full_like(x, float("nan")) for x in a))
        ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
        return copies, ctl, zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))

    def step(st, copies):
        if flow == "bucket_table":
            st.single_pass_buckets(table, copies)
        else:
            st.two_pass_buckets(buckets, *copies[0], max_grad_norm=2e-3)

    g_copies, g_ctl, g_st = fresh()
    e_copies, e_ctl, e_st = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_st, g_copies)
    torch.cuda.synchronize()
    assert zs.control_read(g_ctl).step == w.hyper.step       # capture runs nothing
    for r in range(4):
        graph.replay()
        torch.cuda.synchronize()
        step(e_st, e_copies)
        junk = torch.randn(1 << 20, device=dev).sum()      # unrelated eager work
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        gc, ec = zs.control_read(g_ctl), zs.control_read(e_ctl)
        print(f"case: {flow} graph replay {r}: t={gc.step} cur={gc.cur}", flush=True)
        for name in _KEPT + ("skip", "overflow", "error", "clip_coef", "step_used"):
            assert getattr(gc, name) == getattr(ec, name), (r, name)
        assert abs(gc.sqnorm - ec.sqnorm) <= 1e-12 * ec.sqnorm
        assert gc.step == w.hyper.step + r + 1
        for cp_g, cp_e in zip(g_copies, e_copies):
            for x, y in zip(cp_g, cp_e):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_bucket_table_single_pass_matches_oracle():
    """ZeRO-2 slices (ragged, tiling the shard) stepped by one call per step
    under the control block: the skip decision covers every slice, and the
    committed copy is the oracle's step of the whole shard."""
    dev = device()
    w = _workload()
    sizes = [8 * s for s in (1, 511, 512, 513, 2048, 1, 7, 1000)]
    sizes.append(n // 8 * 8 - sum(sizes))
    assert sizes[-1] > 0
    nn = sum(sizes)
    h = wl.host_shard(w, n=nn, offset_seed=906)
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    b = tuple(torch.full_like(x, float("nan")) for x in a)
    copies = (a, b)
    scaler, os_ = _scaler()
    ctl = zs.control_new(scaler, w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    full = [torch.empty(nn, dtype=torch.float16, device=dev) for _ in range(N)]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int)
    table = zs.BucketSlices([([f[o:o + s] for f in full], int(o)) for o, s in zip(offs, sizes)])
    state, t, cur = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step, 0
    for k, plant in enumerate(PLAN):
        S = os_.scale
        g = [wl.host_fp16_grad(wl.seed_of(w.wid, 950 + k, i), nn, w.grad_sigma, S)
             for i in range(N)]
        if plant:
            g[k % N][int(offs[-1]) + 5] = np.float16(np.nan)    # in the last slice only
        for f, src in zip(full, g):
            f.copy_(torch.from_numpy(src))
        stepper.single_pass_buckets(table, copies)
        want = ozs.shard_step(g, *state, w.hyper.replace(step=t), S)
        skip = ols.update_loss_scale(os_, want.overflow)
        t += 0 if skip else 1
        c = zs.control_read(ctl)
        print(f"case: ctl bucket table step {k} plant={plant} S={S}", flush=True)
        _check_control(c, os_, t, skip, want)
        if skip:
            assert c.cur == cur
            continue
        cur = 1 - cur
        assert c.cur == cur
        got = dict(zip(("master", "m", "v", "p16"), copies[cur]))
        for name, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
            assert np.array_equal(got[name].cpu().numpy().view(np.uint32),
                                  ref.view(np.uint32)), (k, name)
        assert np.array_equal(got["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))
        state = (want.master, want.m, want.v, want.p16)


@pytest.mark.parametrize("n_side,ready", [(0, "stream"), (2, "stream"), (2, "event")])
def test_streamed_buckets_single_pass_matches_oracle(n_side, ready):
    """Buckets arriving one at a time through two reused chunk buffers (the
    last one ragged), each updated as it arrives, one decision per step: the
    same states as the oracle's step of the whole shard, with an overflow in
    any one bucket skipping the whole step.  With side streams the updates
    alternate between two streams, and a buffer is refilled only after the
    update that read it (its bucket_done event); each bucket's arrival is
    either the work on the step's stream or an event the generator records
    after refilling."""
    dev = device()
    w = _workload()
    sizes = [8 * s for s in (1, 511, 512, 513, 2048, 7)]
    sizes.append(n - sum(sizes))
    assert sizes[-1] % 8 != 0
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int)
    h = wl.host_shard(w, n=n, offset_seed=907)
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    b = tuple(torch.full_like(x, float("nan")) for x in a)
    copies = (a, b)
    scaler, os_ = _scaler()
    ctl = zs.control_new(scaler, w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    bufs = [[torch.empty(max(sizes), dtype=torch.float16, device=dev) for _ in range(N)]
            for _ in range(2)]
    sides = [torch.cuda.Stream() for _ in range(n_side)]
    state, t, cur = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step, 0
    for k, plant in enumerate(PLAN):
        S = os_.scale
        g = [wl.host_fp16_grad(wl.seed_of(w.wid, 960 + k, i), n, w.grad_sigma, S)
             for i in range(N)]
        if plant:
            g[k % N][int(offs[3]) + 17] = np.float16(-np.inf)    # in bucket 3 only

        def arrivals():
            done = {}
            for j, (o, s) in enumerate(zip(offs, sizes)):
                if j >= 2 and done[j - 2] is not None:   # buffer j % 2: read by bucket j - 2
                    torch.cuda.current_stream().wait_event(done[j - 2])
                chunks = [buf[:s] for buf in bufs[j % 2]]
                for c, src in zip(chunks, g):
                    c.copy_(torch.from_numpy(src[o:o + s]))
                if ready == "event":
                    landed = torch.cuda.Event()
                    landed.record(torch.cuda.current_stream())
                    yield chunks, int(o), landed
                else:
                    yield chunks, int(o)
                done[j] = stepper.bucket_done

        stepper.single_pass_streamed(arrivals(), copies, side_streams=sides)
        want = ozs.shard_step(g, *state, w.hyper.replace(step=t), S)
        skip = ols.update_loss_scale(os_, want.overflow)
        t += 0 if skip else 1
        c = zs.control_read(ctl)
        print(f"case: ctl streamed buckets (side streams {n_side}, ready {ready}) step {k} "
              f"plant={plant} S={S}", flush=True)
        _check_control(c, os_, t, skip, want)
        if skip:
            assert c.cur == cur
            continue
        cur = 1 - cur
        assert c.cur == cur
        got = dict(zip(("master", "m", "v", "p16"), copies[cur]))
        for name, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
            assert np.array_equal(got[name].cpu().numpy().view(np.uint32),
                                  ref.view(np.uint32)), (k, name)
        assert np.array_equal(got["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))
        state = (want.master, want.m, want.v, want.p16)


def test_streamed_buckets_that_miss_the_state_commit_nothing():
    """Buckets that do not cover the state exactly once (a shortfall, a
    stray, an overlap) raise before the decision: the control block's t and
    current copy, and the current state, stay where they were."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=908)
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    b = tuple(torch.empty_like(x) for x in a)
    ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    half = [c[:8 * 2500] for c in chunks]
    with pytest.raises(ValueError, match="cover"):
        stepper.single_pass_streamed(iter([(half, 0)]), (a, b))
    with pytest.raises(ValueError, match="outside"):
        stepper.single_pass_streamed(iter([(chunks, 8)]), (a, b))
    # two overlapping buckets whose lengths sum to n: refused at the second
    third = [c[:8 * 1700] for c in chunks]
    rest = [c[8 * 1700 - 8:] for c in chunks]
    assert third[0].numel() + rest[0].numel() - 8 == n
    with pytest.raises(ValueError, match="overlaps"):
        stepper.single_pass_streamed(iter([(third, 0), (rest, 8 * 1700 - 8),
                                           ([c[:8] for c in chunks], 0)]), (a, b))
    with pytest.raises(ValueError, match="overlaps"):
        stepper.two_pass_buckets([(third, 0), (rest, 8 * 1700 - 8)], *a)
    c = zs.control_read(ctl)
    assert c.cur == 0 and c.step == w.hyper.step and c.error == 0
    for x, k in zip(a, ("master", "m", "v", "p16")):
        bits = np.uint16 if h[k].dtype == np.float16 else np.uint32
        assert np.array_equal(x.cpu().numpy().view(bits), h[k].view(bits))


def test_prepared_single_pass_equals_single_pass():
    """The prepared step (arguments marshalled once) walks the same states as
    DeviceStepper.single_pass over clean and overflowing steps, and past a
    rebase of the bias-correction table."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=909)

    def setup():
        a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        copies = (a, tuple(torch.empty_like(x) for x in a))
        ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
        return copies, ctl, zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))

    pc, p_ctl, p_st = setup()
    ec, e_ctl, e_st = setup()
    chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
    step = p_st.prepare_single_pass(chunks, pc)
    plan = PLAN + [False] * (zs.ZERO_CTL_STEPS + 3)        # runs past one rebase
    for k, plant in enumerate(plan):
        S = zs.control_read(e_ctl).scale
        for c, src in zip(chunks, _grads(w, k % 50, S, plant)):
            c.copy_(torch.from_numpy(src))
        step()
        e_st.single_pass(chunks, ec)
        if k < len(PLAN) or k % 16 == 0 or k == len(plan) - 1:
            a, b = zs.control_read(p_ctl), zs.control_read(e_ctl)
            print(f"case: prepared single pass step {k} plant={plant}", flush=True)
            for name in ("scale", "good_steps", "skipped_steps", "step", "cur", "skip",
                         "overflow", "error"):
                assert getattr(a, name) == getattr(b, name), (k, name)
            if np.isfinite(b.sqnorm):
                assert abs(a.sqnorm - b.sqnorm) <= 1e-12 * abs(b.sqnorm)
            else:                   # an overflow step: inf or NaN on both sides
                assert np.isnan(a.sqnorm) == np.isnan(b.sqnorm) and not np.isfinite(a.sqnorm)
            for x, y in zip(pc[a.cur], ec[b.cur]):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), k
    assert zs.control_read(p_ctl).step > w.hyper.step + zs.ZERO_CTL_STEPS


def _state(h, dev):
    a = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
    return a, tuple(torch.full_like(x, float("nan")) for x in a)


def _assert_state(got, want, label):
    for name, g, ref in zip(("master", "m", "v", "p16"), got,
                            (want.master, want.m, want.v, want.p16)):
        bits = np.uint16 if ref.dtype == np.float16 else np.uint32
        assert np.array_equal(g.cpu().numpy().view(bits), ref.view(bits)), (label, name)


@pytest.mark.parametrize("NN", [1, 2, 3, 16, 17, 64])
def test_control_flows_at_any_replica_count(NN):
    """Both device-controlled flows at N = 1 .. 64 (the unrolled and the
    runtime-loop kernels), on a ragged shard, against the oracle: the single
    pass, and the two-pass check, decision and in-place update."""
    dev = device()
    nn = 9_011
    base = wl.LLAMA3_8B_SHARD
    w = wl.ShardWorkload(name="ctl_n", wid=base.wid, n=nn, n_replicas=NN, grad_sigma=1e-4,
                         loss_scale=1024.0, hyper=base.hyper.replace(step=5),
                         m_sigma=1e-4, v_sigma=1e-8)
    h = wl.host_shard(w, n=nn, offset_seed=910 + NN)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper,
                          w.loss_scale)
    print(f"case: control flows N={NN} n={nn}", flush=True)
    # single pass
    copies = _state(h, dev)
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).single_pass(chunks, copies)
    c = zs.control_read(ctl)
    assert c.cur == 1 and c.skip == 0 and c.overflow == 0 and c.error == 0
    assert abs(c.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
    _assert_state(copies[1], want, f"single pass N={NN}")
    # two-pass, in place
    state, _ = _state(h, dev)
    ctl2 = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    zs.DeviceStepper(ctl2, zs.adamw_params(w.hyper)).two_pass(chunks, *state)
    c2 = zs.control_read(ctl2)
    assert c2.skip == 0 and c2.overflow == 0 and c2.error == 0 and c2.step == w.hyper.step + 1
    assert abs(c2.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
    _assert_state(state, want, f"two-pass N={NN}")


@pytest.mark.parametrize("NN", [1, 17, 64])
def test_bucket_table_under_control_at_any_replica_count(NN):
    """The bucket table under the control block at N = 1, 17 and 64: at
    N = 64 the 9 slices take 3 launches (4 slices of 64 chunk pointers per
    launch), all sharing one decision."""
    dev = device()
    sizes = [8 * s for s in (1, 511, 512, 513, 7, 64, 100, 3)]
    sizes.append(4001)
    nn = sum(sizes)
    base = wl.LLAMA3_8B_SHARD
    w = wl.ShardWorkload(name="ctl_b", wid=base.wid, n=nn, n_replicas=NN, grad_sigma=1e-4,
                         loss_scale=65536.0, hyper=base.hyper.replace(step=9),
                         m_sigma=1e-4, v_sigma=1e-8)
    h = wl.host_shard(w, n=nn, offset_seed=930 + NN)
    full = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int)
    table = zs.BucketSlices([([f[o:o + s] for f in full], int(o)) for o, s in zip(offs, sizes)])
    copies = _state(h, dev)
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    print(f"case: control bucket table N={NN} slices={len(sizes)}", flush=True)
    zs.DeviceStepper(ctl, zs.adamw_params(w.hyper)).single_pass_buckets(table, copies)
    want = ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper,
                          w.loss_scale)
    c = zs.control_read(ctl)
    assert c.cur == 1 and c.skip == 0 and c.overflow == 0 and c.error == 0
    assert abs(c.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
    _assert_state(copies[1], want, f"bucket table N={NN}")


def test_two_pass_norm_and_clip_repeat_bit_for_bit():
    """The two-pass flow's squared norm comes from the check's fixed-grid
    partials folded in a fixed order, so two runs from the same state give
    the same norm, clip factor and clipped state, bit for bit."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=911)

    def run():
        state = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
        stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
        chunks = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
        seen = []
        for k in range(4):
            for c, src in zip(chunks, _grads(w, 20 + k, zs.control_read(ctl).scale, False)):
                c.copy_(torch.from_numpy(src))
            stepper.two_pass(chunks, *state, max_grad_norm=2e-3)
            c = zs.control_read(ctl)
            seen.append((c.sqnorm, c.clip_coef, c.skip, c.step))
        return seen, [x.clone() for x in state]

    print("case: two-pass clipped norm repeats", flush=True)
    a, sa = run()
    b, sb = run()
    assert a == b                       # fp64 norm and fp32 clip factor, bit for bit
    assert any(coef < 1.0 for _, coef, _, _ in a)
    for x, y in zip(sa, sb):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_check_partials_accumulate_over_buckets():
    """Two zero_overflow_check_ctl calls on the two halves of a shard (one per
    bucket) fold to the squared norm of the whole shard, the same bits on
    every run, and within 1e-12 of the oracle's ascending-order sum."""
    dev = device()
    w = _workload()
    h = wl.host_shard(w, n=n, offset_seed=912)
    chunks = [torch.from_numpy(c).to(dev) for c in h["chunks"]]
    half = (n // 2) // 8 * 8
    want_flag, want_sq = ozs.check_only(h["chunks"], w.loss_scale)
    got = []
    for rep in range(2):
        ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
        zs.zero_control_begin(ctl, zs.adamw_params(w.hyper))
        zs.zero_overflow_check_ctl([c[:half] for c in chunks], ctl)
        zs.zero_overflow_check_ctl([c[half:] for c in chunks], ctl)
        zs.zero_control_decide(ctl, 0.0, False)
        c = zs.control_read(ctl)
        print(f"case: check partials over two buckets, run {rep}", flush=True)
        assert c.overflow == int(want_flag) == 0
        got.append(c.sqnorm)
    assert got[0] == got[1]
    assert abs(got[0] - want_sq) <= 1e-12 * want_sq


@pytest.mark.parametrize("clip", [0.0, 2e-3])
def test_two_pass_over_buckets_matches_oracle(clip):
    """A ZeRO-2 shard held as ragged bucket slices, stepped by the two-pass
    flow: one check per bucket, one decision (and clip factor) for the whole
    shard, one in-place update per bucket.  Against the oracle's step of the
    whole shard over clean and overflowing steps; bit for bit without
    clipping, to the tolerance with it (the norm's summation order differs
    from the oracle's); and the same bits on a second run."""
    dev = device()
    w = _workload()
    sizes = [8 * s for s in (1, 511, 513, 2048, 7)]
    sizes.append(n - sum(sizes))
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int)
    h = wl.host_shard(w, n=n, offset_seed=913)

    def run():
        state = tuple(torch.from_numpy(h[k]).to(dev) for k in ("master", "m", "v", "p16"))
        ctl = zs.control_new(_scaler()[0], w.hyper.step, dev)
        stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
        full = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(N)]
        buckets = [([f[o:o + s] for f in full], int(o)) for o, s in zip(offs, sizes)]
        log = []
        for k, plant in enumerate(PLAN[:5]):
            S = zs.control_read(ctl).scale
            g = _grads(w, 30 + k, S, plant)
            for f, src in zip(full, g):
                f.copy_(torch.from_numpy(src))
            stepper.two_pass_buckets(buckets, *state, max_grad_norm=clip)
            log.append((g, S, zs.control_read(ctl), [x.clone() for x in state]))
        return log

    first, second = run(), run()
    os_ = ols.ScalerState(scale=65536.0, growth_interval=2)
    st, t = (h["master"], h["m"], h["v"], h["p16"]), w.hyper.step
    for k, ((g, S, c, got), (_, _, c2, got2)) in enumerate(zip(first, second)):
        print(f"case: two-pass over buckets clip={clip} step {k}", flush=True)
        assert S == np.float32(os_.scale)
        want = ozs.shard_step_clipped(g, *st, w.hyper.replace(step=t), S, clip)
        skip = ols.update_loss_scale(os_, want.overflow)
        t += 0 if skip else 1
        _check_control(c, os_, t, skip, want)
        # the same bits on both runs (NaN on an overflow step included)
        assert struct.pack("<d", c.sqnorm) == struct.pack("<d", c2.sqnorm)
        assert struct.pack("<f", c.clip_coef) == struct.pack("<f", c2.clip_coef)
        for x, y in zip(got, got2):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
        if skip:
            # untouched: the device's own state before this step, bit for bit
            prev = first[k - 1][3] if k else [torch.from_numpy(h[key]) for key in
                                              ("master", "m", "v", "p16")]
            for x, y in zip(got, prev):
                assert torch.equal(x.cpu().view(torch.uint8), y.cpu().view(torch.uint8))
            continue
        if clip == 0.0:
            _assert_state(got, want, f"two-pass buckets step {k}")
        else:
            assert_matches_oracle(dict(zip(("master", "m", "v", "p16"), got)), want, max_ulp=None)
        st = (want.master, want.m, want.v, want.p16)
