"""Benchmark of the per-rank ZeRO-1/2 mixed-precision shard step on one MI355X.

Workload: the Llama-3-8B shard (psi = 8.03e9 params over N = 8 ranks, so this
rank owns 1,003,750,000 params), 8 fp16 replica gradient chunks in HBM,
loss scale 65536, AdamW at t = 1000 with non-zero fp32 m and v.  Inputs are
seeded synthetic draws made on the device before timing starts.

One timed step is the whole per-rank path in its single-pass form, with the
decision on the device: start the step in the control block; run the fused
update (replica sum, mean, unscale, inf/NaN flag, squared norm, moments,
fp32 master, fp16 params) from the current copy of the state into the other
copy; then decide on the device (skip, loss-scale move, t, and commit of the
written copy if the step is clean).  Nothing is read back between steps.

Timed afterwards on the same state and reported under "extra": the
host-decided single pass (flag read-back, host loss scale, swap); the
two-pass form (overflow check, then the in-place update), host- and
device-decided; the page-literal split (the gradient mean stored as fp16,
then the update from it) and the arrival folds; the step's traffic twin (the
same loads and stores with XORs for arithmetic); plain read, write, copy
and 2:1 and 3:1 streams on the same device; one bucket flatten; and the tiny
workload's launch-bound step, eager and in HIP graphs.

Before timing, the shard's 16 arrays go through the placement search of
sharded_mixed_precision_step_amd.placement (whole new sets of the arrays,
each behind random spacer allocations, timed in turn; the fastest set is
kept, contents unchanged), as a training run would do once at start-up.
`extra.placement` gives the two-direction step time before and after, and
the fused step is also timed where torch first put the arrays;
`--no-placement` skips the search.

Prints one JSON line.  `value` is params/s of the whole step.  `roofline`
rates the fused update kernel, the dominant one, by its algorithmic bytes
(2N + 24 + 2 per param) over its average duration measured with HIP events
on the launch stream, against the 8 TB/s HBM peak.  `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILE_DIR, "shard_step_kernel_llama3_8b_shard_pmc.txt")
METRIC = "optimizer-shard params/s and achieved HBM GB/s (% of peak), 1 MI355X"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_shard",
                    choices=("tiny", "llama3_8b_shard", "overflow", "llama70b_shard",
                             "zero2_bucketed", "replica_sweep"),
                    help="llama3_8b_shard (default), or zero2_bucketed (160 bucket slices "
                         "in one table), llama70b_shard (23 buckets streamed), tiny, overflow, "
                         "replica_sweep (the fused step and its twin at N = 1..32)")
    ap.add_argument("--cpu-sample-slices", type=int, default=0,
                    help="CPU baseline sample: this many slices of 2^22 params "
                         "(0: the whole shard)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB fp32 copy kernel (counter calibration)")
    ap.add_argument("--no-flatten", action="store_true")
    ap.add_argument("--no-placement", action="store_true",
                    help="time the arrays where torch allocated them, without the "
                         "placement search")
    ap.add_argument("--placement-trials", type=int, default=12,
                    help="trial sets of the placement search (default 12)")
    ap.add_argument("--two-pass-steps", type=int, default=10,
                    help="steps of the two-pass path (check, then in-place step), "
                         "timed after the main loop for comparison")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(digest: str, n: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m = re.search(r"^kernel_digest_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m or m.group(1) != digest:
        return None
    vals = {}
    for key in ("fetch_bytes_per_param", "write_bytes_per_param"):
        mm = re.search(rf"^{key}:\s*([0-9.eE+-]+)", text, re.M)
        if not mm:
            return None
        vals[key] = float(mm.group(1))
    return (vals["fetch_bytes_per_param"] + vals["write_bytes_per_param"]) * n


# One GPU's share of a GPU host's cores: the oracle's thread pool never takes
# more, however many cores the process can see (the host is shared by the
# jobs of its other GPUs).
ORACLE_MAX_THREADS = 16


def oracle_threads() -> int:
    return max(1, min(ORACLE_MAX_THREADS, len(os.sched_getaffinity(0))))


def host_cpus() -> dict:
    """The host's cores as this process sees them, beside the pool's size."""
    return {"host_cpus_visible": len(os.sched_getaffinity(0)),
            "host_cpu_count": os.cpu_count(),
            "cores_rule": f"thread pool of min({ORACLE_MAX_THREADS}, visible cores): one "
                          f"GPU's share of the host"}


ORACLE_PIECE = 1 << 22


def cpu_baseline(dev_shard, w, slices: int, keep: list | None = None):
    """The CPU oracle as it stands, on the first `slices` x 2^22 params of the
    shard (host copies of the device inputs), over a thread pool.  With
    `keep`, the oracle's result for each 2^22-param slice is appended to it."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle.zero_step as ozs

    piece = ORACLE_PIECE
    total = min(slices * piece, w.n) if slices > 0 else w.n
    host = dict(chunks=[c[:total].cpu().numpy() for c in dev_shard["chunks"]],
                master=dev_shard["master"][:total].cpu().numpy(),
                m=dev_shard["m"][:total].cpu().numpy(), v=dev_shard["v"][:total].cpu().numpy(),
                p16=dev_shard["p16"][:total].cpu().numpy())
    threads = oracle_threads()

    def run(k):
        sl = slice(k * piece, min((k + 1) * piece, total))
        return ozs.shard_step([c[sl] for c in host["chunks"]], host["master"][sl],
                              host["m"][sl], host["v"][sl], host["p16"][sl], w.hyper,
                              w.loss_scale)

    count = (total + piece - 1) // piece
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        results = list(ex.map(run, range(count)))
    dt = time.perf_counter() - t0
    assert not any(r.overflow for r in results)
    # the same oracle on one core, over the first few slices only
    single = min(8, count)
    t0 = time.perf_counter()
    for k in range(single):
        run(k)
    dt1 = time.perf_counter() - t0
    n1 = min(single * piece, total)
    if keep is not None:
        keep.extend(results)
    # a pool of `threads` on `count` slices keeps at most `count` of them busy
    return {"value": total / dt, "unit": "params/s", "cores": min(threads, count),
            "kind": "oracle", **host_cpus(), "pool_threads": threads, "seconds": dt,
            "single_core_value": n1 / dt1,
            "single_core_sample": f"the first {n1} params ({single} slices of 2^22), one thread",
            "sample": (f"{'whole' if total == w.n else 'first ' + str(total) + ' params of the'} "
                       f"{w.name} shard ({total} params, {count} slices of 2^22, "
                       f"N={w.n_replicas} replicas): overflow check and AdamW update")}


def ulp_line(x, sbits):
    """IEEE floats (sign and magnitude) mapped to integers in value order, one
    step per representable value: the distance of two maps is the ulp
    distance of the floats (+0 and -0 map to 0)."""
    import numpy as np
    i = x.view(sbits).astype(np.int64)
    mag = i & ((1 << (8 * x.itemsize - 1)) - 1)
    return np.where(i < 0, -mag, mag)


def parity_of_step(zs, d, spare, w, results, stream) -> dict:
    """One fused step on the device (zero_shard_step_out) from the shard's
    inputs into the spare copy, against the oracle's results for the same
    inputs (kept from the CPU baseline, 2^22-param slices from the start of
    the shard): bit equality per array, and the largest distance in fp32 ulps
    (master, m, v) and fp16 ulps (params) where the bits differ."""
    import numpy as np
    import torch

    hp = zs.adamw_params(w.hyper)
    flag = torch.zeros(1, dtype=torch.int32, device=spare[0].device)
    zs.zero_shard_step_out(d["chunks"], w.loss_scale, d["master"], d["m"], d["v"], *spare, hp,
                           flag, None, stream=stream)
    torch.cuda.synchronize()

    worst = {"master": 0, "m": 0, "v": 0, "p16": 0}
    elements = 0
    for k, r in enumerate(results):
        a = k * ORACLE_PIECE
        b = a + r.master.size
        for name, t, ref in zip(("master", "m", "v", "p16"), spare,
                                (r.master, r.m, r.v, r.p16)):
            got = t[a:b].cpu().numpy()
            bits = np.uint16 if ref.dtype == np.float16 else np.uint32
            if not np.array_equal(got.view(bits), ref.view(bits)):
                sbits = np.int16 if ref.dtype == np.float16 else np.int32
                d_ulp = np.abs(ulp_line(got, sbits) - ulp_line(ref, sbits))
                worst[name] = max(worst[name], int(d_ulp.max()))
        elements = b
    return {"elements": elements, "overflow": int(flag.item()),
            "bit_exact": all(v == 0 for v in worst.values()),
            "max_ulp_master": worst["master"], "max_ulp_m": worst["m"],
            "max_ulp_v": worst["v"], "max_ulp_p16_fp16": worst["p16"],
            "against": "the oracle's step of the same inputs (the CPU baseline's results)"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the shard step has no cross-GPU traffic here, "
              f"so --gpus {args.gpus} is not supported (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sharded_mixed_precision_step_amd as zs
    import workloads as wl
    from sharded_mixed_precision_step_amd import _build

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.workload == "zero2_bucketed":
        return bench_zero2(args, dev)
    if args.workload == "llama70b_shard":
        return bench_streamed(args, dev)
    if args.workload == "overflow":
        return bench_overflow(args, dev)
    if args.workload == "replica_sweep":
        return bench_replica_sweep(args, dev)
    w = wl.WORKLOADS[args.workload]
    n, N = w.n, w.n_replicas
    log(f"bench: workload={w.name} n={n} N={N} steps={args.steps} warmup={args.warmup}")
    t0 = time.perf_counter()
    d = wl.device_shard(w, dev)
    torch.cuda.synchronize()
    log(f"bench: inputs drawn on device in {time.perf_counter() - t0:.1f} s")

    cpu = None
    stream = torch.cuda.current_stream()
    spare = tuple(torch.empty_like(d[k]) for k in ("master", "m", "v", "p16"))
    parity = None
    if not args.no_cpu_baseline:
        oracle_results = []
        cpu = cpu_baseline(d, w, args.cpu_sample_slices, keep=oracle_results)
        log(f"bench: cpu oracle {cpu['value']:.3e} params/s on {cpu['cores']} threads "
            f"({cpu['seconds']:.1f} s)")
        parity = parity_of_step(zs, d, spare, w, oracle_results, stream)
        del oracle_results
        log(f"bench: one device step against the oracle over {parity['elements']} params: "
            f"bit-exact {parity['bit_exact']}")
    unplaced = fused_step_median(zs, d["chunks"], (d["master"], d["m"], d["v"], d["p16"]),
                                 spare, w, stream)
    log(f"bench: fused step where torch allocated the arrays: median {unplaced:.3f} ms")
    placed = None
    if not args.no_placement:
        from sharded_mixed_precision_step_amd import placement
        chunks, copies, rep = placement.place_shard(
            d["chunks"], ((d["master"], d["m"], d["v"], d["p16"]), spare), w.hyper,
            w.loss_scale, trials=args.placement_trials,
            budget_s=max(30.0, 2.5 * args.placement_trials), stream=stream)
        d["chunks"] = chunks
        d["master"], d["m"], d["v"], d["p16"] = copies[0]
        spare = copies[1]
        del chunks, copies
        placed = {"initial_ms_two_steps": rep.initial_ms, "final_ms_two_steps": rep.final_ms,
                  "gain": rep.gain, "trials": rep.trials, "kept_trials": rep.kept,
                  "seconds": rep.seconds}
        log(f"bench: placement search {rep.seconds:.1f} s, {rep.trials} trials, kept "
            f"{rep.kept}: two steps {rep.initial_ms:.3f} -> {rep.final_ms:.3f} ms")
    shard = zs.DoubleBufferedShard(d["master"], d["m"], d["v"], d["p16"], spare=spare)
    del spare
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    fused_events = []

    def step(record: bool):
        """One step under the device control block: begin, the fused
        out-of-place update (flag and squared norm into the block), then the
        decision, loss-scale move and commit on the device.  Nothing is read
        back, so the host enqueues the next step at once."""
        stepper._rebase()
        zs.zero_control_begin(ctl, stepper.hp, stream=stream)
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
        zs.zero_shard_step_out_ctl(d["chunks"], shard.copies, stepper.hp, ctl, stream=stream)
        if record:
            e[1].record(stream)
            fused_events.append(e)
        zs.zero_control_decide(ctl, 0.0, True, stream=stream)
        stepper.since_base += 1

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    k1_times = sorted(a.elapsed_time(b) for a, b in fused_events)
    k1_ms = sum(k1_times) / max(len(k1_times), 1)
    k1_median_ms = k1_times[len(k1_times) // 2] if k1_times else float("nan")
    c = zs.control_read(ctl)
    if c.error:
        raise RuntimeError(f"step control reported error {c.error}")
    skipped = c.skipped_steps
    log(f"bench: device single pass {ms_per_step:.3f} ms/step, fused step {k1_ms:.3f} ms, "
        f"skipped {skipped}, t = {c.step}")
    # the other forms continue from the current copy at the block's t and scale
    shard.cur = c.cur & 1
    scaler = zs.LossScaler.create(scale=c.scale)
    hp = zs.adamw_params(w.hyper.replace(step=int(c.step)))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    sq = torch.zeros(1, dtype=torch.float64, device=dev)
    twin = traffic_twin(zs, d, shard, w, stream)
    log(f"bench: traffic twin {twin['twin_ms']:.3f} ms ({twin['twin_gbps']:.0f} GB/s)")
    host = host_single_pass(zs, d, shard, scaler, hp, flag, sq, stream, args.two_pass_steps, n)
    log(f"bench: host-synced single pass {host['host_single_pass_ms_per_step']:.3f} ms/step")
    two = two_pass(zs, d, shard, w, scaler, hp, flag, sq, stream, args.two_pass_steps)
    log(f"bench: two-pass {two['two_pass_ms_per_step']:.3f} ms/step, check "
        f"{two['check_ms']:.3f} ms, in-place step {two['inplace_step_ms']:.3f} ms")
    dtp = device_two_pass(zs, d, shard, w, scaler, hp, stream, args.two_pass_steps)
    log(f"bench: device two-pass {dtp['device_two_pass_ms_per_step']:.3f} ms/step, clipped "
        f"{dtp['device_two_pass_clipped_ms_per_step']:.3f} ms/step")
    lit = page_literal(zs, d, shard, w, scaler, hp, flag, sq, stream, args.two_pass_steps)
    log(f"bench: page-literal split {lit['split_ms_per_step']:.3f} ms/step, fp16 mean "
        f"{lit['mean_fp16_ms']:.3f} ms, one-chunk step {lit['split_step_ms']:.3f} ms")

    k1_bytes = w.bytes_per_param_step() * n
    k1_gbps = k1_bytes / (k1_ms * 1e-3) / 1e9
    traffic = read_traffic(_build.kernel_digest(), n)
    extra = {
        "path": "single pass under the device control block: zero_control_begin, "
                "zero_shard_step_out_ctl (flag and squared norm), zero_control_decide "
                "(skip, loss scale, t, commit); no read-back inside the loop",
        "fused_step_ms": k1_ms, "fused_step_params_per_s": n / (k1_ms * 1e-3),
        "fused_step_median_ms": k1_median_ms,
        "fused_step_gbps": k1_gbps, "fused_step_pct_peak": 100 * k1_gbps / HBM_PEAK_GBPS,
        "step_gbps": k1_bytes / (ms_per_step * 1e-3) / 1e9,
        "skipped_steps": skipped,
        "placement": placed if placed is not None else "allocation as made (--no-placement)",
        "fused_step_counter_gbps": (traffic / (k1_ms * 1e-3) / 1e9) if traffic else None,
        "unplaced_fused_step_median_ms": unplaced,
        "unplaced_fused_step_pct_peak":
            100 * w.bytes_per_param_step() * n / (unplaced * 1e-3) / 1e9 / HBM_PEAK_GBPS,
    }
    extra.update(twin)
    extra["fused_step_pct_twin"] = 100 * k1_gbps / twin["twin_gbps"]
    extra.update(host)
    extra.update(two)
    extra.update(dtp)
    extra.update(lit)

    if not args.no_flatten:
        extra.update(bench_flatten(zs, wl, dev, stream))
    extra.update(copy_ceiling(dev, stream))
    extra["fused_step_pct_copy_ceiling"] = 100 * k1_gbps / extra["copy_ceiling_gbps"]
    extra["fused_step_pct_add_ceiling"] = 100 * k1_gbps / extra["add_ceiling_gbps"]
    extra.update(tiny_graph(dev))
    if args.calibrate_copy:
        calibration_copy(dev)

    out = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded device draws; fp16 grads, fp32 state)",
        "config": {"workload": w.name, "shard_params": n, "replicas": N,
                   "loss_scale": w.loss_scale, "adam_step": w.hyper.step,
                   "bytes_per_param_fused_step": w.bytes_per_param_step()},
        "roofline": {"bound": "hbm", "achieved": k1_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": k1_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "parity": parity,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def calibration_copy(dev):
    """Three plain 1 GiB fp32 copies (torch's elementwise dst = -src), whose
    known bytes calibrate the rocprofv3 FETCH_SIZE and WRITE_SIZE counters."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _timed(fn, steps: int, warmup: int = 2):
    """Average wall time (ms) of fn() over `steps` calls, each ending in a
    device synchronisation, after `warmup` untimed calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def bench_zero2(args, dev):
    """ZeRO-2 bucketed workload: 160 buckets of 32 decoder layers, N = 8; this
    rank owns slice 3 of every bucket (973,111,296 params).  Times, per step:
    the whole step under the device control block (begin, the update of all
    160 slices in one zero_shard_step_buckets_ctl call, decide and commit),
    and the same step streamed (one zero_shard_step_out_ctl per bucket, as
    buckets arrive), on one stream and alternating over two side streams
    (chunks already resident, so no per-bucket arrival waits);
    the update alone as one zero_shard_step_buckets call, as 160
    zero_shard_step_out calls, and as one call over the contiguous shard
    (same bytes, the launch-free ideal); and the rank flattening its own 160
    gradient buckets, in one zero_bucket_flatten_batch call and in one
    zero_bucket_flatten call per bucket.  Prints one JSON line."""
    import torch

    import sharded_mixed_precision_step_amd as zs
    import workloads as wl

    w = wl.ZERO2
    N, r, S = w.n_replicas, wl.ZERO2_RANK, w.loss_scale
    align, pad = wl.ZERO2_ALIGN, wl.ZERO2_ALIGN * N
    stream = torch.cuda.current_stream()
    plan = wl.zero2_bucket_plan()
    log(f"bench: workload={w.name} buckets={len(plan)} n={w.n} N={N}")
    # this rank's own gradients, flattened bucket by bucket (the layout gives
    # each bucket's length and so each slice)
    grads = [[wl.zero2_device_tensor(r, k, dev) for k in idx] for idx in plan]
    lmax = 0
    lengths = []
    scratch = torch.empty(60_000_000, dtype=torch.float16, device=dev)
    for ts in grads:
        offs = zs.zero_bucket_flatten(ts, scratch, align, pad, stream=stream)
        lengths.append(offs[-1])
        lmax = max(lmax, offs[-1])
    buckets = [torch.empty(L, dtype=torch.float16, device=dev) for L in lengths]

    def flatten_each():
        for ts, bk in zip(grads, buckets):
            zs.zero_bucket_flatten(ts, bk, align, pad, stream=stream)

    batch = zs.FlattenBatch(list(zip(grads, buckets)), align, pad)

    def flatten_all():
        batch(stream=stream)

    flat_each_ms = _timed(flatten_each, args.steps)
    flat_ms = _timed(flatten_all, args.steps)
    flat_bytes = sum(2 * sum(t.numel() for t in ts) + 2 * L for ts, L in zip(grads, lengths))
    del grads, buckets, scratch
    torch.cuda.empty_cache()
    # the slices this rank owns, as the per-bucket reduce-scatter delivers them
    offsets, off = [], 0
    for L in lengths:
        offsets.append((off, L // N))
        off += L // N
    assert off == w.n
    owned = wl.device_chunks(w, dev)
    st = wl.device_state(w, dev)
    cur = (st["master"], st["m"], st["v"], st["p16"])
    del st
    out = tuple(torch.empty_like(t) for t in cur)
    placed = "allocation as made (--no-placement)"
    if not args.no_placement:
        # the slices are views into the N replica buffers and the two state
        # copies, so the whole-shard search places them all at once
        from sharded_mixed_precision_step_amd import placement
        owned, (cur, out), rep = placement.place_shard(
            owned, (cur, out), w.hyper, S, trials=args.placement_trials,
            budget_s=max(30.0, 2.5 * args.placement_trials), stream=stream)
        placed = {"initial_ms_two_steps": rep.initial_ms, "final_ms_two_steps": rep.final_ms,
                  "gain": rep.gain, "trials": rep.trials, "kept_trials": rep.kept,
                  "seconds": rep.seconds}
        log(f"bench: placement search {rep.seconds:.1f} s, {rep.trials} trials, kept "
            f"{rep.kept}: two steps {rep.initial_ms:.3f} -> {rep.final_ms:.3f} ms")
    table = zs.BucketSlices([([o[a:a + n] for o in owned], a) for a, n in offsets])
    views = [([o[a:a + n] for o in owned], tuple(t[a:a + n] for t in cur[:3]),
              tuple(t[a:a + n] for t in out)) for a, n in offsets]
    hp = zs.adamw_params(w.hyper)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    sq = torch.zeros(1, dtype=torch.float64, device=dev)

    def multi():
        zs.zero_shard_step_buckets(table, S, *cur[:3], *out, hp, flag, sq, stream=stream)

    def per_bucket():
        for ch, si, so in views:
            zs.zero_shard_step_out(ch, S, *si, *so, hp, flag, sq, stream=stream)

    def whole():
        zs.zero_shard_step_out(owned, S, *cur[:3], *out, hp, flag, sq, stream=stream)

    ctl = zs.control_new(zs.LossScaler.create(scale=S), w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    copies = (cur, out)

    def device_step():
        stepper.single_pass_buckets(table, copies, stream=stream)

    ctl_s = zs.control_new(zs.LossScaler.create(scale=S), w.hyper.step, dev)
    stepper_s = zs.DeviceStepper(ctl_s, zs.adamw_params(w.hyper))
    arrivals = [([o[a:a + n] for o in owned], a) for a, n in offsets]

    def device_streamed():
        stepper_s.single_pass_streamed(iter(arrivals), copies, stream=stream)

    ctl_2s = zs.control_new(zs.LossScaler.create(scale=S), w.hyper.step, dev)
    stepper_2s = zs.DeviceStepper(ctl_2s, zs.adamw_params(w.hyper))
    sides = [torch.cuda.Stream() for _ in range(2)]
    resident = [(ch, a, None) for ch, a in arrivals]      # chunks already in place

    def device_streamed_2s():
        stepper_2s.single_pass_streamed(iter(resident), copies, stream=stream,
                                        side_streams=sides, track_done=False)

    ms = {name: _timed(fn, args.steps) for name, fn in
          (("device_step", device_step), ("device_streamed", device_streamed),
           ("device_streamed_2s", device_streamed_2s),
           ("multi_bucket", multi), ("per_bucket", per_bucket), ("whole_shard", whole))}
    # the table update of the whole step alone (its launches between begin
    # and decide), timed with HIP events on the launch stream
    events = []
    for k in range(args.steps + 2):
        stepper._rebase()
        zs.zero_control_begin(ctl, stepper.hp, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        zs.zero_shard_step_buckets_ctl(table, copies, stepper.hp, ctl, stream=stream)
        e[1].record(stream)
        zs.zero_control_decide(ctl, 0.0, True, stream=stream)
        stepper.since_base += 1
        if k >= 2:
            events.append(e)
    torch.cuda.synchronize()
    update_ms = sum(a.elapsed_time(b) for a, b in events) / len(events)
    for c in (ctl, ctl_s, ctl_2s):
        assert zs.control_read(c).error == 0
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_buckets(w, arrivals, cur, (0, 40, 80, 120, 159), piece=1 << 20)
        log(f"bench: cpu oracle {cpu['value']:.3e} params/s on {cpu['cores']} threads "
            f"({cpu['seconds']:.1f} s for {cpu['params']} params)")
    step_bytes = w.bytes_per_param_step() * w.n
    update_gbps = step_bytes / (update_ms * 1e-3) / 1e9
    log("bench: " + ", ".join(f"{k} {v:.3f} ms" for k, v in ms.items()) +
        f", table update {update_ms:.3f} ms (events), flatten {flat_ms:.3f} ms (one batch "
        f"call), {flat_each_ms:.3f} ms (a call per bucket)")
    out_line = {
        "metric": METRIC,
        "value": w.n / (ms["device_step"] * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 2,
        "ms_per_step": ms["device_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded device draws; fp16 grads, fp32 state)",
        "config": {"workload": w.name, "buckets": len(plan), "shard_params": w.n,
                   "replicas": N, "rank": r, "bytes_per_param_fused_step":
                   w.bytes_per_param_step()},
        "roofline": {"bound": "hbm", "achieved": update_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": update_gbps / HBM_PEAK_GBPS, "traffic": None},
        "cpu_baseline": cpu,
        "extra": {
            "path": "single pass under the device control block over the bucket table: "
                    "zero_control_begin, zero_shard_step_buckets_ctl (5 launches), "
                    "zero_control_decide",
            "table_update_ms": update_ms,
            "table_update_gbps": update_gbps,
            **{f"{k}_ms": v for k, v in ms.items()},
            **{f"{k}_gbps": step_bytes / (v * 1e-3) / 1e9 for k, v in ms.items()},
            "flatten_own_buckets_ms": flat_ms,
            "flatten_own_buckets_gbps": flat_bytes / (flat_ms * 1e-3) / 1e9,
            "flatten_own_buckets_per_call_ms": flat_each_ms,
            "flatten_own_buckets_per_call_gbps": flat_bytes / (flat_each_ms * 1e-3) / 1e9,
            "placement": placed,
        },
    }
    print(json.dumps(out_line), flush=True)


def bench_streamed(args, dev):
    """70B-class shard (7.06e10 params over N = 16 ranks: 4,412,500,000 on
    this rank), its gradients arriving in 23 buckets (22 x 2e8 + 1.25e7)
    through two chunk buffers of 16 x 2e8 fp16, the state (two copies,
    124 GB) resident.  One timed step is the device-controlled single pass
    in streamed form: begin, one zero_shard_step_out_ctl per bucket as it
    arrives (from the current copy into the other), then decide and commit.
    The CPU oracle runs buckets 0, 11 and 22 in full; its rate is quoted as
    such, and the whole-shard time it implies is labelled extrapolated.
    Before timing, the lean placement search (place_streamed) re-places the
    arrays, one group per trial; `--no-placement` skips it.  Prints one
    JSON line."""
    import torch

    import sharded_mixed_precision_step_amd as zs
    import workloads as wl

    w = wl.LLAMA70B_SHARD
    n, N = w.n, w.n_replicas
    stream = torch.cuda.current_stream()
    log(f"bench: workload={w.name} n={n} N={N} buckets={len(w.buckets)} "
        f"steps={args.steps} warmup={args.warmup}")
    t0 = time.perf_counter()
    st = wl.device_state(w, dev)
    cur = (st["master"], st["m"], st["v"], st["p16"])
    del st
    nxt = tuple(torch.empty_like(t) for t in cur)
    bmax = max(w.buckets)
    bufs = [wl.device_chunks(w, dev, n=bmax, offset_seed=100 + j) for j in range(2)]
    items, off = [], 0
    for b, nb in enumerate(w.buckets):
        items.append(([c[:nb] for c in bufs[b % 2]], off))
        off += nb
    assert off == n
    torch.cuda.synchronize()
    log(f"bench: inputs drawn on device in {time.perf_counter() - t0:.1f} s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_buckets(w, items, cur, (0, 11, 22))
        log(f"bench: cpu oracle {cpu['value']:.3e} params/s on {cpu['cores']} threads "
            f"({cpu['seconds']:.1f} s for {cpu['params']} params)")

    placed = "allocation as made (--no-placement)"
    if not args.no_placement:
        n_buf = len(bufs[0])
        arrays = list(cur) + list(nxt) + list(bufs[0]) + list(bufs[1])
        del cur, nxt, bufs, items       # the search takes the only references
        arrays, placed = place_streamed(zs, w, arrays, n_buf, stream, args)
        cur, nxt = tuple(arrays[0:4]), tuple(arrays[4:8])
        bufs = [arrays[8:8 + n_buf], arrays[8 + n_buf:8 + 2 * n_buf]]
        del arrays
        items, off = [], 0
        for b, nb in enumerate(w.buckets):
            items.append(([c[:nb] for c in bufs[b % 2]], off))
            off += nb
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
    stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
    events = []

    def arrivals(record: bool):
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
        yield from items
        if record:
            e[1].record(stream)
            events.append(e)

    for _ in range(args.warmup):
        stepper.single_pass_streamed(arrivals(False), (cur, nxt), stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        stepper.single_pass_streamed(arrivals(True), (cur, nxt), stream=stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    upd_ms = sum(a.elapsed_time(b) for a, b in events) / max(len(events), 1)
    c = zs.control_read(ctl)
    if c.error:
        raise RuntimeError(f"step control reported error {c.error}")
    # the same steps with the bucket updates alternating over two side streams
    sides = [torch.cuda.Stream() for _ in range(2)]
    resident = [(ch, off, None) for ch, off in items]     # chunks already in place
    ms_2s = _timed(lambda: stepper.single_pass_streamed(iter(resident), (cur, nxt),
                                                        stream=stream, side_streams=sides,
                                                        track_done=False),
                   args.steps, warmup=1)
    assert zs.control_read(ctl).error == 0
    k1_bytes = w.bytes_per_param_step() * n
    k1_gbps = k1_bytes / (upd_ms * 1e-3) / 1e9
    ceilings = copy_ceiling(dev, stream)
    log("bench: stream ceilings " + ", ".join(f"{k} {v:.0f}" for k, v in ceilings.items()))
    log(f"bench: streamed device single pass {ms_per_step:.3f} ms/step, {len(w.buckets)} "
        f"bucket updates {upd_ms:.3f} ms ({k1_gbps:.0f} GB/s), skipped {c.skipped_steps}; "
        f"over two side streams {ms_2s:.3f} ms/step")
    out = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded device draws; fp16 grads, fp32 state)",
        "config": {"workload": w.name, "shard_params": n, "replicas": N,
                   "buckets": len(w.buckets), "loss_scale": w.loss_scale,
                   "adam_step": w.hyper.step,
                   "bytes_per_param_fused_step": w.bytes_per_param_step()},
        "roofline": {"bound": "hbm", "achieved": k1_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": k1_gbps / HBM_PEAK_GBPS, "traffic": None},
        "cpu_baseline": cpu,
        "extra": {
            "placement": placed,
            "path": "single pass under the device control block, streamed: "
                    "zero_control_begin, one zero_shard_step_out_ctl per arriving bucket, "
                    "zero_control_decide",
            "two_side_streams_ms_per_step": ms_2s,
            "two_side_streams_params_per_s": n / (ms_2s * 1e-3),
            "bucket_updates_ms": upd_ms,
            "bucket_updates_gbps": k1_gbps,
            "bucket_updates_pct_peak": 100 * k1_gbps / HBM_PEAK_GBPS,
            "step_gbps": k1_bytes / (ms_per_step * 1e-3) / 1e9,
            "skipped_steps": c.skipped_steps,
            **ceilings,
            "bucket_updates_pct_fma_ceiling": 100 * k1_gbps / ceilings["fma_ceiling_gbps"],
        },
    }
    if args.calibrate_copy:
        calibration_copy(dev)
    print(json.dumps(out), flush=True)


def place_streamed(zs, w, arrays, n_buf, stream, args):
    """The lean placement search for a shard whose two state copies leave no
    room for a second set: trials alternate between re-placing the copy the
    first timing step writes together with the two chunk buffers, and the
    copy it reads (contents copied over in both).  Each trial is timed as one
    streamed step in each direction between the copies; the state's copy 0
    is saved to host memory before the search and written back after."""
    import torch

    from sharded_mixed_precision_step_amd import placement

    hp = zs.adamw_params(w.hyper)

    def timed(arrs):
        c0, c1 = tuple(arrs[0:4]), tuple(arrs[4:8])
        b = (arrs[8:8 + n_buf], arrs[8 + n_buf:8 + 2 * n_buf])
        its, off = [], 0
        for k, nb in enumerate(w.buckets):
            its.append(([c[:nb] for c in b[k % 2]], off))
            off += nb
        ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step,
                             c0[0].device)
        st = zs.DeviceStepper(ctl, hp)
        times = ([], [])
        for r in range(3):                    # the first round is a warm-up
            for d in (0, 1):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
                st.single_pass_streamed(iter(its), (c0, c1), stream=stream)
                e[1].record(stream)
                if r:
                    times[d].append(e)
        torch.cuda.synchronize()
        assert zs.control_read(ctl).error == 0
        return sum(sorted(a.elapsed_time(b) for a, b in t)[len(t) // 2] for t in times)

    # the chunk buffers' contents are the seeded gradients and are copied
    # over; the spare copy's are overwritten before they are read
    groups = [(list(range(4, 8 + 2 * n_buf)), True), (list(range(0, 4)), True)]
    # spacers of up to 1 GiB: a trial of the first group allocates 36 arrays
    # (and a spacer before each) beside the 137 GB already resident
    arrays, rep = placement.place_groups(
        arrays, groups, timed, restore=range(0, 4), trials=args.placement_trials,
        budget_s=max(60.0, 5.0 * args.placement_trials), max_spacer=1 << 30, stream=stream)
    log(f"bench: lean placement search {rep.seconds:.1f} s, {rep.trials} trials, kept "
        f"{rep.kept}: two steps {rep.initial_ms:.3f} -> {rep.final_ms:.3f} ms")
    placed = {"search": "lean (one group per trial: the written copy with the chunk buffers, "
                        "then the read copy)",
              "initial_ms_two_steps": rep.initial_ms, "final_ms_two_steps": rep.final_ms,
              "gain": rep.gain, "trials": rep.trials, "kept_trials": rep.kept,
              "seconds": rep.seconds}
    return arrays, placed


def bench_overflow(args, dev):
    """Overflow workload (125,468,750 params, N = 8, S = 65536, 100,375 of
    the N * n gradient entries set to +inf, -inf, NaN).  Times, per step:
    the device-controlled single pass over the overflowing gradients (the
    update is written to the spare copy and not committed: skip, scale
    backs off); the device-controlled two-pass form over the same gradients
    (check, decide; the update kernel sees the skip and returns at once);
    and, after the gradients are drawn again clean at the halved scale
    32768, the clean single pass.  Asserts that the skipped steps leave t,
    the current copy and the state bit-identical.  Prints one JSON line."""
    import torch

    import sharded_mixed_precision_step_amd as zs
    import workloads as wl

    w = wl.OVERFLOW
    n, N = w.n, w.n_replicas
    stream = torch.cuda.current_stream()
    log(f"bench: workload={w.name} n={n} N={N} injected={w.n_inject} "
        f"steps={args.steps} warmup={args.warmup}")
    d = wl.device_shard(w, dev)
    wl.device_inject(d["chunks"], wl.injection_sites(w))
    cur = (d["master"], d["m"], d["v"], d["p16"])
    spare = tuple(torch.empty_like(t) for t in cur)
    before = [t.clone() for t in cur]
    hp = zs.adamw_params(w.hyper)
    torch.cuda.synchronize()

    def timed_single(ctl, steps, events):
        for k in range(steps):
            zs.zero_control_begin(ctl, hp, stream=stream)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            zs.zero_shard_step_out_ctl(d["chunks"], (cur, spare), hp, ctl, stream=stream)
            e[1].record(stream)
            zs.zero_control_decide(ctl, 0.0, True, stream=stream)
            if events is not None:
                events.append(e)

    def run(fn, ctl):
        ev = []
        fn(ctl, args.warmup, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn(ctl, args.steps, ev)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        return ms, sum(a.elapsed_time(b) for a, b in ev) / max(len(ev), 1)

    def timed_two_pass(ctl, steps, events):
        for k in range(steps):
            zs.zero_control_begin(ctl, hp, stream=stream)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            zs.zero_overflow_check_ctl(d["chunks"], ctl, stream=stream)
            e[1].record(stream)
            zs.zero_control_decide(ctl, 0.0, False, stream=stream)
            zs.zero_shard_step_ctl(d["chunks"], *cur, hp, ctl, stream=stream)
            if events is not None:
                events.append(e)

    # every step is skipped; the scale backs off to min_scale (1) and stays
    scaler = zs.LossScaler.create(scale=w.loss_scale)
    ctl = zs.control_new(scaler, w.hyper.step, dev)
    skip_ms, skip_upd_ms = run(timed_single, ctl)
    c = zs.control_read(ctl)
    total = args.warmup + args.steps
    assert c.skipped_steps == total and c.step == w.hyper.step and c.cur == 0 and c.error == 0
    ctl2 = zs.control_new(scaler, w.hyper.step, dev)
    two_ms, check_ms = run(timed_two_pass, ctl2)
    c2 = zs.control_read(ctl2)
    assert c2.skipped_steps == total and c2.step == w.hyper.step and c2.error == 0
    for a, b in zip(before, cur):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "a skipped step wrote"
    del before
    # the retry: clean gradients at the halved scale, one clean step each
    S2 = w.loss_scale * 0.5
    wl.device_chunks(w, dev, loss_scale=S2, out=d["chunks"])
    ctl3 = zs.control_new(zs.LossScaler.create(scale=S2), w.hyper.step, dev)

    stepper3 = zs.DeviceStepper(ctl3, hp)

    def timed_clean(ctl, steps, events):
        for k in range(steps):
            stepper3._rebase()
            zs.zero_control_begin(ctl, stepper3.hp, stream=stream)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            zs.zero_shard_step_out_ctl(d["chunks"], (cur, spare), stepper3.hp, ctl,
                                       stream=stream)
            e[1].record(stream)
            zs.zero_control_decide(ctl, 0.0, True, stream=stream)
            stepper3.since_base += 1
            if events is not None:
                events.append(e)

    clean_ms, clean_upd_ms = run(timed_clean, ctl3)
    c3 = zs.control_read(ctl3)
    assert c3.skipped_steps == 0 and c3.error == 0 and c3.step == w.hyper.step + total
    step_bytes = w.bytes_per_param_step() * n
    check_bytes = 2 * N * n
    upd_gbps = step_bytes / (skip_upd_ms * 1e-3) / 1e9
    log(f"bench: overflowing single pass {skip_ms:.3f} ms/step (update {skip_upd_ms:.3f} ms), "
        f"two-pass {two_ms:.3f} ms/step (check {check_ms:.3f} ms), clean retry "
        f"{clean_ms:.3f} ms/step")
    out = {
        "metric": METRIC,
        "value": n / (skip_ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": skip_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded device draws; fp16 grads with injected inf/NaN, fp32 state)",
        "config": {"workload": w.name, "shard_params": n, "replicas": N,
                   "injected": w.n_inject, "loss_scale": w.loss_scale,
                   "adam_step": w.hyper.step,
                   "bytes_per_param_fused_step": w.bytes_per_param_step()},
        "roofline": {"bound": "hbm", "achieved": upd_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": upd_gbps / HBM_PEAK_GBPS, "traffic": None},
        "cpu_baseline": None,
        "extra": {
            "path": "device single pass over overflowing gradients: the update goes to the "
                    "spare copy, the decision skips it and backs the scale off",
            "skipped_single_pass_ms": skip_ms, "skipped_update_ms": skip_upd_ms,
            "skipped_update_gbps": upd_gbps,
            "skipped_two_pass_ms": two_ms, "check_ms": check_ms,
            "check_gbps": check_bytes / (check_ms * 1e-3) / 1e9,
            "clean_retry_single_pass_ms": clean_ms, "clean_retry_update_ms": clean_upd_ms,
            "clean_retry_update_gbps": step_bytes / (clean_upd_ms * 1e-3) / 1e9,
            "final_scale_after_skips": c.scale,
        },
    }
    print(json.dumps(out), flush=True)


def bench_replica_sweep(args, dev):
    """The fused step under the control block, and its traffic twin on the
    same arrays, at N = 1, 2, 4, 8, 16, 32 replicas over a 250,000,000-param
    shard (the Llama-3-8B shard's distributions): how the attainable rate
    moves with the read share, 2N + 12 read against 14 written per param,
    and how close the step stays to it.  Prints one JSON line."""
    import torch

    import sharded_mixed_precision_step_amd as zs
    import workloads as wl
    from sharded_mixed_precision_step_amd import twin as zt

    base = wl.LLAMA3_8B_SHARD
    n = 250_000_000
    stream = torch.cuda.current_stream()
    rows = []
    for N in (1, 2, 4, 8, 16, 32):
        w = wl.ShardWorkload(name=f"sweep_n{N}", wid=base.wid, n=n, n_replicas=N,
                             grad_sigma=base.grad_sigma, loss_scale=base.loss_scale,
                             hyper=base.hyper, m_sigma=base.m_sigma, v_sigma=base.v_sigma)
        d = wl.device_shard(w, dev)
        cur = (d["master"], d["m"], d["v"], d["p16"])
        nxt = tuple(torch.empty_like(t) for t in cur)
        ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
        stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))
        ev_step, ev_twin = [], []
        for k in range(args.warmup + args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            stepper._rebase()
            zs.zero_control_begin(ctl, stepper.hp, stream=stream)
            e[0].record(stream)
            zs.zero_shard_step_out_ctl(d["chunks"], (cur, nxt), stepper.hp, ctl, stream=stream)
            e[1].record(stream)
            zs.zero_control_decide(ctl, 0.0, False, stream=stream)   # keep reading cur
            stepper.since_base += 1
            e[2].record(stream)
            zt.zero_traffic_twin(d["chunks"], *cur[:3], *nxt, stream=stream)
            e[3].record(stream)
            if k >= args.warmup:
                ev_step.append((e[0], e[1]))
                ev_twin.append((e[2], e[3]))
        torch.cuda.synchronize()
        assert zs.control_read(ctl).error == 0
        step_ms = sorted(a.elapsed_time(b) for a, b in ev_step)[len(ev_step) // 2]
        twin_ms = sorted(a.elapsed_time(b) for a, b in ev_twin)[len(ev_twin) // 2]
        nbytes = w.bytes_per_param_step() * n
        rows.append({"replicas": N, "bytes_per_param": w.bytes_per_param_step(),
                     "step_ms": step_ms, "step_gbps": nbytes / (step_ms * 1e-3) / 1e9,
                     "twin_ms": twin_ms, "twin_gbps": nbytes / (twin_ms * 1e-3) / 1e9,
                     "step_pct_twin": 100 * twin_ms / step_ms})
        log(f"bench: N={N:2d} step {step_ms:.3f} ms ({rows[-1]['step_gbps']:.0f} GB/s), "
            f"twin {twin_ms:.3f} ms ({rows[-1]['twin_gbps']:.0f} GB/s)")
        del d, cur, nxt
        torch.cuda.empty_cache()
    ref = next(r for r in rows if r["replicas"] == 8)
    out = {
        "metric": METRIC,
        "value": n / (ref["step_ms"] * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ref["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded device draws; fp16 grads, fp32 state)",
        "config": {"workload": "replica_sweep", "shard_params": n,
                   "replicas": [r["replicas"] for r in rows]},
        "roofline": {"bound": "hbm", "achieved": ref["step_gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ref["step_gbps"] / HBM_PEAK_GBPS,
                     "traffic": None},
        "cpu_baseline": None,
        "extra": {"sweep": rows,
                  "note": "value, ms_per_step and roofline are the N = 8 row (fused step only)"},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_buckets(w, items, state, sampled, piece: int = 1 << 22):
    """The CPU oracle as it stands on whole buckets of a shard (host copies of
    their device chunks and state slices), in slices of `piece` params over
    one thread pool for all the sampled buckets together."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle.zero_step as ozs

    threads = oracle_threads()
    work, params = [], 0
    for b in sampled:
        chunks, off = items[b]
        nb = chunks[0].numel()
        ch = [c.cpu().numpy() for c in chunks]
        stt = [t[off:off + nb].cpu().numpy() for t in state]
        work += [(ch, stt, slice(k, min(k + piece, nb))) for k in range(0, nb, piece)]
        params += nb

    def run(item):
        ch, stt, sl = item
        return ozs.shard_step([c[sl] for c in ch], *(t[sl] for t in stt), w.hyper, w.loss_scale)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        results = list(ex.map(run, work))
    seconds = time.perf_counter() - t0
    assert not any(r.overflow for r in results)
    del work, results
    rate = params / seconds
    return {"value": rate, "unit": "params/s", "cores": threads, "kind": "oracle",
            **host_cpus(), "seconds": seconds, "params": params,
            "extrapolated_whole_shard_seconds": w.n / rate,
            "sample": (f"buckets {', '.join(map(str, sampled))} of the {w.name} shard "
                       f"({params} params, N={w.n_replicas} replicas, slices of {piece} "
                       f"params over one thread pool): overflow check and AdamW update; the "
                       f"whole-shard time is extrapolated at this rate")}


def fused_step_median(zs, chunks, cur, nxt, w, stream, reps: int = 9) -> float:
    """Median over `reps` launches (after two untimed) of the fused update
    under a control block of its own, from `cur` into `nxt`, on the arrays as
    given: the decision never flips the copy, so `cur` is only read."""
    import torch
    ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, cur[0].device)
    hp = zs.adamw_params(w.hyper)
    ev = []
    for k in range(reps + 2):
        zs.zero_control_begin(ctl, hp, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        zs.zero_shard_step_out_ctl(chunks, (cur, nxt), hp, ctl, stream=stream)
        e[1].record(stream)
        zs.zero_control_decide(ctl, 0.0, False, stream=stream)
        if k >= 2:
            ev.append(e)
    torch.cuda.synchronize()
    c = zs.control_read(ctl)
    assert c.error == 0 and c.skip == 0
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


def traffic_twin(zs, d, shard, w, stream, reps: int = 20):
    """zero_traffic_twin on the fused step's own arrays (current copy in,
    other copy out): the same loads and stores with XORs for arithmetic, so
    its rate is what the step's access pattern reaches on this device.
    Average and median of HIP-event timings of single launches."""
    import torch

    from sharded_mixed_precision_step_amd import twin as zt
    src, dst = shard.current, shard.other
    for _ in range(3):
        zt.zero_traffic_twin(d["chunks"], *src[:3], *dst, stream=stream)
    ev = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        zt.zero_traffic_twin(d["chunks"], *src[:3], *dst, stream=stream)
        e[1].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    ms = sum(t) / len(t)
    nbytes = w.bytes_per_param_step() * w.n
    return {"twin_ms": ms, "twin_median_ms": t[len(t) // 2],
            "twin_gbps": nbytes / (ms * 1e-3) / 1e9}


def host_single_pass(zs, d, shard, scaler, hp, flag, sq, stream, steps: int, n: int):
    """The single pass with the decision on the host: fused out-of-place
    update, flag read-back, zero_update_loss_scale, commit by swapping."""
    import torch
    t0 = None
    for k in range(steps + 1):           # the first step is an untimed warm-up
        if k == 1:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        zs.committed_step(d["chunks"], shard, hp, scaler, flag, sq, stream=stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"host_single_pass_ms_per_step": ms,
            "host_single_pass_params_per_s": n / (ms * 1e-3)}


def tiny_graph(dev, steps: int = 200):
    """The tiny workload (1,000,003 params, N = 3), launch-bound: one
    device-controlled single-pass step as eager launches (arguments
    marshalled once by DeviceStepper.prepare_single_pass, and per call by
    DeviceStepper.single_pass) versus the same step captured once in a HIP
    graph and replayed; and the fused update alone, warm in the MALL and
    flushed from it (medians of HIP-event timings)."""
    import torch

    import sharded_mixed_precision_step_amd as zs
    import workloads as wl

    w = wl.TINY
    d = wl.device_shard(w, dev)
    copies = ((d["master"], d["m"], d["v"], d["p16"]),
              tuple(torch.empty_like(t) for t in (d["master"], d["m"], d["v"], d["p16"])))

    def fresh():
        ctl = zs.control_new(zs.LossScaler.create(scale=w.loss_scale), w.hyper.step, dev)
        return ctl, zs.DeviceStepper(ctl, zs.adamw_params(w.hyper))

    def eager(prepared: bool) -> float:
        ctl, st = fresh()
        step = (st.prepare_single_pass(d["chunks"], copies) if prepared
                else lambda: st.single_pass(d["chunks"], copies))
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        assert zs.control_read(ctl).error == 0
        return (time.perf_counter() - t0) * 1e6 / steps

    eager_us = eager(True)
    unprepared_us = eager(False)
    ctl, st = fresh()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.single_pass(d["chunks"], copies)
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    reps = min(steps, zs.ZERO_CTL_STEPS - 4)   # t stays inside the captured table
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / reps
    assert zs.control_read(ctl).error == 0
    raw = hip_graph_replays(zs, d, copies, w, fresh)
    # The fused update alone, timed with HIP events: warm (its 32 MB of
    # inputs are in the 256 MB MALL from the step before) and flushed (a
    # 1 GiB fill between steps, outside the events, evicts them).  Warm and
    # flushed steps alternate.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    ctl, st = fresh()
    stream = torch.cuda.current_stream()
    times = {False: [], True: []}
    for k in range(2 * reps + 4):
        flushed = k % 2 == 1
        if flushed:
            flush.fill_(float(k))
        st._rebase()
        zs.zero_control_begin(ctl, st.hp, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        zs.zero_shard_step_out_ctl(d["chunks"], copies, st.hp, ctl, stream=stream)
        e[1].record(stream)
        zs.zero_control_decide(ctl, 0.0, True, stream=stream)
        st.since_base += 1
        if k >= 4:
            times[flushed].append(e)
    torch.cuda.synchronize()
    assert zs.control_read(ctl).error == 0
    med = {f: sorted(a.elapsed_time(b) for a, b in ev)[len(ev) // 2] * 1e3
           for f, ev in times.items()}
    step_bytes = w.bytes_per_param_step() * w.n
    return {"tiny_eager_us_per_step": eager_us, "tiny_eager_unprepared_us_per_step": unprepared_us,
            "tiny_graph_us_per_step": graph_us, **raw,
            "tiny_graph_params_per_s": w.n / (graph_us * 1e-6),
            "tiny_update_warm_us": med[False], "tiny_update_flushed_us": med[True],
            "tiny_update_warm_gbps": step_bytes / (med[False] * 1e-6) / 1e9,
            "tiny_update_flushed_gbps": step_bytes / (med[True] * 1e-6) / 1e9}


def hip_graph_replays(zs, d, copies, w, fresh, per_graph=(1, 8)) -> dict:
    """The tiny workload's device-controlled single pass captured straight
    through the HIP runtime (hipStreamBeginCapture on a stream of its own,
    hipGraphInstantiate once, hipGraphLaunch per replay), with K = 1 and 8
    steps per graph: per-step wall time over back-to-back replays, and the
    device time of one replay by HIP events on the replay stream.  K steps
    share one launch, so the per-launch cost of a graph shows as the
    difference between K = 1 and K = 8."""
    import ctypes

    import torch
    hip = ctypes.CDLL("libamdhip64.so.7")    # the runtime torch already holds
    vp = ctypes.c_void_p
    for name, args in (("hipStreamBeginCapture", [vp, ctypes.c_int]),
                       ("hipStreamEndCapture", [vp, ctypes.POINTER(vp)]),
                       ("hipGraphInstantiate", [ctypes.POINTER(vp), vp, vp, vp, ctypes.c_size_t]),
                       ("hipGraphLaunch", [vp, vp]), ("hipGraphExecDestroy", [vp]),
                       ("hipGraphDestroy", [vp])):
        getattr(hip, name).argtypes = args
        getattr(hip, name).restype = ctypes.c_int

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} returned HIP error {rc}")

    out = {}
    stream = torch.cuda.Stream()
    sp = vp(stream.cuda_stream)
    for k in per_graph:
        ctl, st = fresh()
        torch.cuda.synchronize()
        ok(hip.hipStreamBeginCapture(sp, 0), "hipStreamBeginCapture")   # global mode
        for _ in range(k):
            st.single_pass(d["chunks"], copies, stream=stream)
        graph, exe = vp(), vp()
        ok(hip.hipStreamEndCapture(sp, ctypes.byref(graph)), "hipStreamEndCapture")
        ok(hip.hipGraphInstantiate(ctypes.byref(exe), graph, None, None, 0), "hipGraphInstantiate")
        reps = (zs.ZERO_CTL_STEPS - 8) // k       # every step's t inside the captured table
        ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
        stream.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
        ev[1].record(stream)
        stream.synchronize()
        one_ms = ev[0].elapsed_time(ev[1])
        t0 = time.perf_counter()
        for _ in range(reps - 2):
            ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
        stream.synchronize()
        wall_us = (time.perf_counter() - t0) * 1e6 / ((reps - 2) * k)
        c = zs.control_read(ctl)
        assert c.error == 0 and c.step == w.hyper.step + reps * k, (c.error, c.step)
        ok(hip.hipGraphExecDestroy(exe), "hipGraphExecDestroy")
        ok(hip.hipGraphDestroy(graph), "hipGraphDestroy")
        out[f"tiny_hip_graph_{k}_steps_us_per_step"] = wall_us
        out[f"tiny_hip_graph_{k}_steps_replay_device_us"] = one_ms * 1e3
    return out


def two_pass(zs, d, shard, w, scaler, hp, flag, sq, stream, steps: int):
    """The two-pass step on the same state, for comparison: overflow check,
    flag read-back, loss-scale update, in-place fused update if clean."""
    import torch
    n, N = w.n, w.n_replicas
    master, m, v, p16 = shard.current
    ev_check, ev_step = [], []
    t0 = None
    for k in range(steps + 1):           # the first step is an untimed warm-up
        if k == 1:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        flag.zero_()
        sq.zero_()
        scale = scaler.scale
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        zs.zero_overflow_check(d["chunks"], scale, flag, sq, stream=stream)
        e[1].record(stream)
        if zs.zero_update_loss_scale(scaler, int(flag.item())):
            continue
        e[2].record(stream)
        zs.zero_shard_step(d["chunks"], scale, master, m, v, p16, hp, stream=stream)
        e[3].record(stream)
        hp.step += 1
        if k >= 1:
            ev_check.append((e[0], e[1]))
            ev_step.append((e[2], e[3]))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    check_ms = sum(a.elapsed_time(b) for a, b in ev_check) / max(len(ev_check), 1)
    step_ms = sum(a.elapsed_time(b) for a, b in ev_step) / max(len(ev_step), 1)
    return {"two_pass_ms_per_step": ms, "two_pass_params_per_s": n / (ms * 1e-3),
            "check_ms": check_ms, "check_gbps": 2 * N * n / (check_ms * 1e-3) / 1e9,
            "inplace_step_ms": step_ms,
            "inplace_step_gbps": w.bytes_per_param_step() * n / (step_ms * 1e-3) / 1e9}


def device_two_pass(zs, d, shard, w, scaler, hp, stream, steps: int):
    """The two-pass step under the device control block, on the current copy
    in place: begin, the check (its norm partials on a fixed grid), the
    decision, the in-place update; with no clipping, and with clipping to
    half the gradient's norm (every step clipped).  No read-back inside the
    loop."""
    import torch
    master, m, v, p16 = shard.current
    out = {}
    for label, clip in (("device_two_pass", 0.0), ("device_two_pass_clipped", None)):
        ctl = zs.control_new(zs.LossScaler.create(scale=scaler.scale), int(hp.step),
                             master.device)
        stepper = zs.DeviceStepper(ctl, zs.adamw_params(w.hyper.replace(step=int(hp.step))))
        if clip is None:
            stepper.two_pass(d["chunks"], master, m, v, p16)       # measures the norm
            clip = 0.5 * zs.control_read(ctl).sqnorm ** 0.5
        ms = _timed(lambda: stepper.two_pass(d["chunks"], master, m, v, p16,
                                             max_grad_norm=clip, stream=stream), steps)
        c = zs.control_read(ctl)
        assert c.error == 0 and c.skipped_steps == 0
        if label.endswith("clipped"):
            assert c.clip_coef < 1.0
        hp.step = int(c.step)
        out[f"{label}_ms_per_step"] = ms
        out[f"{label}_params_per_s"] = w.n / (ms * 1e-3)
    return out


def page_literal(zs, d, shard, w, scaler, hp, flag, sq, stream, steps: int):
    """The page-literal split on the same state, for comparison: the owner's
    gradient mean stored as fp16, then the single-pass update from it as a
    one-chunk step (flag, read-back, loss scale, commit).  Also the fp16 mean
    built arrival by arrival (one zero_accumulate_chunk per replica chunk),
    and in groups of 2 and 4 arrivals (one zero_accumulate_chunks each)."""
    import torch
    n, N = w.n, w.n_replicas
    mean16 = torch.empty(n, dtype=torch.float16, device=d["master"].device)
    ev_mean, ev_step = [], []
    t0 = None
    for k in range(steps + 1):           # the first step is an untimed warm-up
        if k == 1:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        flag.zero_()
        sq.zero_()
        scale = scaler.scale
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        zs.zero_reduce_mean_fp16(d["chunks"], mean16, stream=stream)
        e[1].record(stream)
        m_in, a_in, v_in, _ = shard.current
        m_out, a_out, v_out, p_out = shard.other
        zs.zero_shard_step_out([mean16], scale, m_in, a_in, v_in, m_out, a_out, v_out, p_out,
                               hp, flag, sq, stream=stream)
        e[2].record(stream)
        if not zs.zero_update_loss_scale(scaler, int(flag.item())):
            shard.cur = 1 - shard.cur
            hp.step += 1
        if k >= 1:
            ev_mean.append((e[0], e[1]))
            ev_step.append((e[1], e[2]))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    mean_ms = sum(a.elapsed_time(b) for a, b in ev_mean) / max(len(ev_mean), 1)
    step_ms = sum(a.elapsed_time(b) for a, b in ev_step) / max(len(ev_step), 1)
    # the same fp16 mean built by folding the chunks in as they arrive: the
    # first arrival writes the fp32 accumulator (2 + 4 B/param), the middle
    # ones read and write it (2 + 4 + 4), the last writes the mean (2 + 4 + 2)
    acc = torch.empty(n, dtype=torch.float32, device=mean16.device)
    ev_acc = []
    for k in range(steps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(N + 1)]
        for i, c in enumerate(d["chunks"]):
            e[i].record(stream)
            zs.zero_accumulate_chunk(c, i, N, acc, mean16, stream=stream)
        e[N].record(stream)
        if k >= 1:
            ev_acc.append(e)
    torch.cuda.synchronize()
    acc_ms = sum(e[0].elapsed_time(e[N]) for e in ev_acc) / len(ev_acc)
    mid_ms = (sum(e[1].elapsed_time(e[N - 1]) for e in ev_acc) / len(ev_acc) / (N - 2)
              if N > 2 else None)
    acc_bytes = (6 + 10 * (N - 2) + 8) * n if N > 1 else 4 * n
    # the same fold with the chunks arriving in groups (one
    # zero_accumulate_chunks call per group): pairs and quads
    groups = {}
    for g in (2, 4):
        if N % g or N == g:
            continue
        ev_g = []
        for k in range(steps + 1):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for first in range(0, N, g):
                zs.zero_accumulate_chunks(d["chunks"][first:first + g], first, N, acc,
                                          mean16 if first + g == N else None, stream=stream)
            e[1].record(stream)
            if k >= 1:
                ev_g.append(e)
        torch.cuda.synchronize()
        g_ms = sum(a.elapsed_time(b) for a, b in ev_g) / len(ev_g)
        calls = N // g
        g_bytes = (2 * N + 4 * (calls - 1) + 4 * (calls - 1) + 2) * n
        groups[f"accumulate_groups_of_{g}_ms"] = g_ms
        groups[f"accumulate_groups_of_{g}_gbps"] = g_bytes / (g_ms * 1e-3) / 1e9
    del mean16, acc
    out = {"split_ms_per_step": ms, "split_params_per_s": n / (ms * 1e-3),
           "mean_fp16_ms": mean_ms, "mean_fp16_gbps": (2 * N + 2) * n / (mean_ms * 1e-3) / 1e9,
           "split_step_ms": step_ms, "split_step_gbps": 28 * n / (step_ms * 1e-3) / 1e9,
           "accumulate_all_ms": acc_ms,
           "accumulate_all_gbps": acc_bytes / (acc_ms * 1e-3) / 1e9}
    if mid_ms is not None:
        out["accumulate_middle_ms"] = mid_ms
        out["accumulate_middle_gbps"] = 10 * n / (mid_ms * 1e-3) / 1e9
    out.update(groups)
    return out


def copy_ceiling(dev, stream, reps: int = 5):
    """Plain streams on 4 GiB fp32 arrays, each timed over `reps` launches
    with HIP events on the launch stream: the bandwidth this device reaches
    for a given read/write mix, beside which the step's rate is read.
      read only   zero_stream_read (16-byte non-temporal loads, resident grid)
      write only  torch's fill
      copy 1:1    torch's elementwise dst = -src
      add 2:1     torch's elementwise c = a + b (two arrays read, one written:
                  the step's mix at N = 8 is 28 bytes read to 14 written)
      fma 3:1     torch's elementwise c = a + b * d (three read, one written:
                  the step's mix at N = 16 is 44 bytes read to 14 written)
    Each figure is bytes moved over time."""
    import torch

    from sharded_mixed_precision_step_amd import twin as zt
    a = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    c = torch.empty_like(a)
    d = torch.empty_like(a)
    a.fill_(1.0)
    b.fill_(2.0)
    d.fill_(0.5)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nb = a.numel() * 4

    def timed(fn, nbytes):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return nbytes / (ev[0].elapsed_time(ev[1]) / reps * 1e-3) / 1e9

    out = {
        "read_ceiling_gbps": timed(lambda: zt.zero_stream_read(a, sink, stream=stream), nb),
        "write_ceiling_gbps": timed(lambda: c.fill_(3.0), nb),
        "copy_ceiling_gbps": timed(lambda: torch.neg(a, out=c), 2 * nb),
        "add_ceiling_gbps": timed(lambda: torch.add(a, b, out=c), 3 * nb),
        "fma_ceiling_gbps": timed(lambda: torch.addcmul(a, b, d, out=c), 4 * nb),
    }
    del a, b, c, d
    return out


def bench_flatten(zs, wl, dev, stream, reps: int = 10):
    """Bucket flatten of the largest ZeRO-2 bucket (one 4096 x 14336 grad)."""
    import torch
    numel = wl.ZERO2_HIDDEN * wl.ZERO2_FFN
    src = torch.empty(numel, dtype=torch.float16, device=dev)
    wl.device_fill_normal(src, wl.seed_of(wl.ZERO2_WID, 0), 1e-4 * 65536.0)
    pad = wl.ZERO2_ALIGN * wl.ZERO2_REPLICAS
    L = (numel + pad - 1) // pad * pad
    bucket = torch.empty(L, dtype=torch.float16, device=dev)
    zs.zero_bucket_flatten([src], bucket, wl.ZERO2_ALIGN, pad, stream=stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        zs.zero_bucket_flatten([src], bucket, wl.ZERO2_ALIGN, pad, stream=stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    return {"flatten_ms": ms, "flatten_gbps": (2 * numel + 2 * L) / (ms * 1e-3) / 1e9}


if __name__ == "__main__":
    main()
