"""HIP shard step against the CPU oracle, element by element, through the C
ABI: the tiny workload in full, ragged and edge sizes, special values, the
overflow flag, hyperparameter variants, multi-step runs and determinism."""
import numpy as np
import pytest
import torch

import oracle.zero_step as ozs
import sharded_mixed_precision_step_amd as zs
import workloads as wl
from gpu_util import (assert_fp16_close, assert_fp32_close, assert_matches_oracle, device,
                      flags, run_check_then_step, to_dev)

pytestmark = pytest.mark.gpu


def _oracle(h, hyper, S):
    return ozs.shard_step(h["chunks"], h["master"], h["m"], h["v"], h["p16"], hyper, S)


def _shard(w, n, N=None, seed=0, S=None):
    if N is not None or S is not None:
        w = wl.ShardWorkload(name=w.name, wid=w.wid, n=n, n_replicas=N or w.n_replicas,
                             grad_sigma=w.grad_sigma, loss_scale=S or w.loss_scale,
                             hyper=w.hyper, m_sigma=w.m_sigma, v_sigma=w.v_sigma)
    return w, wl.host_shard(w, n=n, offset_seed=seed)


def test_tiny_workload_in_full():
    """psi = 1,000,003, N = 3, S = 1024, first step, m = v = 0: every element."""
    dev = device()
    w = wl.TINY
    h = wl.host_shard(w)
    print(f"case: tiny n={w.n} N={w.n_replicas}", flush=True)
    d = to_dev(h, dev)
    flag, sq = run_check_then_step(d, w.hyper, w.loss_scale)
    want = _oracle(h, w.hyper, w.loss_scale)
    assert flag == int(want.overflow) == 0
    assert abs(sq - want.sqnorm) <= 1e-6 * want.sqnorm
    ulps = assert_matches_oracle(d, want)
    print("max ulp distance vs oracle:", ulps, flush=True)


def test_bit_exact_with_oracle():
    """Every fp32 operation is a separate, correctly rounded IEEE operation on
    both sides, so the state matches the oracle bit for bit (Llama-shard
    distributions, t = 1000, N = 8 and N = 3)."""
    dev = device()
    for N, S in ((8, 65536.0), (3, 1024.0), (5, 1000.0)):
        w, h = _shard(wl.LLAMA3_8B_SHARD, 100_003, N=N, S=S, seed=N)
        print(f"case: bit-exact N={N} S={S}", flush=True)
        d = to_dev(h, dev)
        run_check_then_step(d, w.hyper, S)
        want = _oracle(h, w.hyper, S)
        for k, ref in (("master", want.master), ("m", want.m), ("v", want.v)):
            got = d[k].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (N, k)
        assert np.array_equal(d["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))


@pytest.mark.parametrize("N", [1, 3, 8, 16, 17, 64])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 255, 2047, 2049, 4099])
def test_ragged_sizes(n, N):
    dev = device()
    w, h = _shard(wl.LLAMA3_8B_SHARD, n, N=N, seed=1000 + N)
    print(f"case: ragged n={n} N={N}", flush=True)
    d = to_dev(h, dev)
    flag, sq = run_check_then_step(d, w.hyper, w.loss_scale)
    want = _oracle(h, w.hyper, w.loss_scale)
    assert flag == 0 and abs(sq - want.sqnorm) <= 1e-6 * want.sqnorm
    assert_matches_oracle(d, want)


def test_empty_shard_is_a_noop():
    dev = device()
    fl, sq = flags(dev)
    z16 = torch.zeros(0, dtype=torch.float16, device=dev)
    z32 = [torch.zeros(0, dtype=torch.float32, device=dev) for _ in range(3)]
    zs.zero_overflow_check([z16, z16], 4.0, fl, sq)
    zs.zero_shard_step([z16, z16], 4.0, *z32, z16, zs.adamw_params(wl.TINY.hyper), fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == 0 and float(sq.item()) == 0.0


def test_special_values():
    """fp16 subnormals, +-65504 and -0 in the replicas: a clean step that
    matches the oracle; fp16 params that round to +-inf or to subnormals."""
    dev = device()
    n = 4099
    rng = np.random.default_rng(5)
    chunks = []
    for i in range(3):
        c = rng.standard_normal(n).astype(np.float32).astype(np.float16)
        c[:64] = np.float16(2.0 ** -24) * rng.integers(-1023, 1024, 64)   # subnormals
        c[64:80] = np.float16(65504.0) * np.where(np.arange(16) % 2, 1, -1)
        c[80:96] = np.float16(-0.0)
        chunks.append(c)
    master = rng.standard_normal(n).astype(np.float32) * np.float32(0.02)
    master[100:110] = np.float32(65519.0)      # writes back as 65504 or +inf
    master[110:120] = np.float32(-70000.0)     # writes back as -inf
    master[120:130] = np.float32(3e-6)         # an fp16 subnormal
    with np.errstate(over="ignore"):     # the +-inf params are intended
        p16 = master.astype(np.float16)
    h = dict(chunks=chunks, master=master, m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
             p16=p16)
    hyper = wl.AdamWHyper(step=1)
    for S in (1.0, 1024.0):
        print(f"case: special values S={S}", flush=True)
        d = to_dev(h, dev)
        flag, sq = run_check_then_step(d, hyper, S)
        want = _oracle(h, hyper, S)
        assert flag == int(want.overflow) == 0
        assert abs(sq - want.sqnorm) <= 1e-6 * want.sqnorm
        assert_matches_oracle(d, want)
        assert np.array_equal(d["p16"].cpu().numpy().view(np.uint16), want.p16.view(np.uint16))


@pytest.mark.parametrize("plant", ["nan_last_tail", "pinf_first", "ninf_mid", "pinf_ninf_same",
                                   "none", "huge_unscale", "big_but_finite"])
def test_overflow_flag(plant):
    """The flag is bit-exact with the oracle's decision (made in fp32 on g)."""
    dev = device()
    N, n = 8, 2049            # 2049 = 256 packs of 8 + a one-element tail
    _, h = _shard(wl.LLAMA3_8B_SHARD, n, N=N, seed=77)
    S = 65536.0
    ch = [c.copy() for c in h["chunks"]]
    if plant == "nan_last_tail":
        ch[N - 1][n - 1] = np.nan
    elif plant == "pinf_first":
        ch[0][0] = np.inf
    elif plant == "ninf_mid":
        ch[3][1000] = -np.inf
    elif plant == "pinf_ninf_same":
        ch[1][500], ch[6][500] = np.inf, -np.inf
    elif plant == "huge_unscale":
        ch[2][17] = np.float16(60000.0)
        S = 2.0 ** -120
    elif plant == "big_but_finite":
        ch = [np.full(n, 65504.0, np.float16) for _ in range(N)]
        S = 2.0 ** -100
    print(f"case: overflow flag plant={plant}", flush=True)
    want_flag, want_sq = ozs.check_only(ch, S)
    d = to_dev(dict(h, chunks=ch), dev)
    fl, sq = flags(dev)
    zs.zero_overflow_check(d["chunks"], S, fl, sq)
    fl2, sq2 = flags(dev)
    zs.zero_shard_step(d["chunks"], S, d["master"], d["m"], d["v"], d["p16"],
                       zs.adamw_params(wl.LLAMA3_8B_SHARD.hyper), fl2, sq2)
    torch.cuda.synchronize()
    assert int(fl.item()) == int(want_flag)
    assert int(fl2.item()) == int(want_flag)     # the fused step reports the same flag
    if not want_flag:
        assert abs(float(sq.item()) - want_sq) <= 1e-6 * want_sq
        assert abs(float(sq2.item()) - want_sq) <= 1e-6 * want_sq


@pytest.mark.parametrize("variant", [
    dict(decoupled_wd=False), dict(bias_correction=False), dict(step=1), dict(step=2),
    dict(step=5000), dict(lr=0.0), dict(weight_decay=0.0), dict(eps=0.0, step=3),
    dict(beta1=0.0, beta2=0.5, step=4),
])
@pytest.mark.parametrize("S", [65536.0, 1000.0])
def test_hyperparameter_variants(variant, S):
    dev = device()
    w, h = _shard(wl.LLAMA3_8B_SHARD, 20_011, N=6, S=S, seed=3)
    hyper = w.hyper.replace(**variant)
    print(f"case: hyper {variant} S={S}", flush=True)
    d = to_dev(h, dev)
    run_check_then_step(d, hyper, S)
    assert_matches_oracle(d, _oracle(h, hyper, S))


def test_reductions_accumulate_across_buckets():
    """Two calls on two halves of a shard share one flag and one squared norm."""
    dev = device()
    w, h = _shard(wl.LLAMA3_8B_SHARD, 30_000, N=8, seed=9)
    half = 15_000
    fl, sq = flags(dev)
    d = to_dev(h, dev)
    zs.zero_overflow_check([c[:half] for c in d["chunks"]], w.loss_scale, fl, sq)
    zs.zero_overflow_check([c[half:] for c in d["chunks"]], w.loss_scale, fl, sq)
    torch.cuda.synchronize()
    want_flag, want_sq = ozs.check_only(h["chunks"], w.loss_scale)
    assert int(fl.item()) == 0 == int(want_flag)
    assert abs(float(sq.item()) - want_sq) <= 1e-6 * want_sq
    d["chunks"][5][half + 3] = float("nan")
    zs.zero_overflow_check([c[:half] for c in d["chunks"]], w.loss_scale, fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == 0
    zs.zero_overflow_check([c[half:] for c in d["chunks"]], w.loss_scale, fl, sq)
    torch.cuda.synchronize()
    assert int(fl.item()) == 1


def test_checked_step_skips_and_recovers():
    """Overflow: the step is skipped, the scale halves and master, m, v and
    the fp16 params stay bit-identical; the next clean step (at the halved
    scale, same t) matches the oracle."""
    dev = device()
    w, h = _shard(wl.LLAMA3_8B_SHARD, 50_001, N=8, seed=21)
    d = to_dev(h, dev)
    d["chunks"][7][50_000] = float("nan")
    snap = {k: d[k].clone() for k in ("master", "m", "v", "p16")}
    scaler = zs.LossScaler.create(scale=w.loss_scale)
    hp = zs.adamw_params(w.hyper)
    fl, sq = flags(dev)
    r = zs.checked_step(d["chunks"], d["master"], d["m"], d["v"], d["p16"], hp, scaler, fl, sq)
    torch.cuda.synchronize()
    assert r.overflow and r.skipped and scaler.scale == w.loss_scale / 2 and hp.step == w.hyper.step
    for k, t in snap.items():
        assert torch.equal(d[k].view(torch.uint8), t.view(torch.uint8)), k
    S2 = scaler.scale
    h2 = wl.host_shard(wl.ShardWorkload(name="retry", wid=w.wid, n=w.n, n_replicas=8,
                                        grad_sigma=w.grad_sigma, loss_scale=S2, hyper=w.hyper),
                       offset_seed=22)
    for c, src in zip(d["chunks"], h2["chunks"]):
        c.copy_(torch.from_numpy(src))
    r2 = zs.checked_step(d["chunks"], d["master"], d["m"], d["v"], d["p16"], hp, scaler, fl, sq)
    torch.cuda.synchronize()
    assert not r2.overflow and not r2.skipped and hp.step == w.hyper.step + 1
    want = ozs.shard_step(h2["chunks"], h["master"], h["m"], h["v"], h["p16"], w.hyper, S2)
    assert abs(r2.sqnorm - want.sqnorm) <= 1e-6 * want.sqnorm
    assert_matches_oracle(d, want)


def test_multi_step_run_matches_oracle():
    """Five steps with fresh replica gradients each step, t = 1..5."""
    dev = device()
    w = wl.TINY
    n = 30_001
    h = wl.host_shard(w, n=n, offset_seed=40)
    d = to_dev(h, dev)
    state = (h["master"], h["m"], h["v"], h["p16"])
    for t in range(1, 6):
        g = wl.host_shard(w, n=n, offset_seed=40 + t)["chunks"]
        for c, src in zip(d["chunks"], g):
            c.copy_(torch.from_numpy(src))
        hyper = w.hyper.replace(step=t)
        run_check_then_step(d, hyper, w.loss_scale)
        r = ozs.shard_step(g, *state, hyper, w.loss_scale)
        state = (r.master, r.m, r.v, r.p16)
        assert_matches_oracle(d, r, label=f"t={t} ")


def test_deterministic():
    dev = device()
    w, h = _shard(wl.LLAMA3_8B_SHARD, 1 << 20, N=8, seed=50)
    outs = []
    for _ in range(2):
        d = to_dev(h, dev)
        fl, sq = flags(dev)
        zs.zero_shard_step(d["chunks"], w.loss_scale, d["master"], d["m"], d["v"], d["p16"],
                           zs.adamw_params(w.hyper), fl, sq)
        torch.cuda.synchronize()
        outs.append((d, float(sq.item())))
    (a, sa), (b, sb) = outs
    for k in ("master", "m", "v", "p16"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k
    assert abs(sa - sb) <= 1e-12 * sa


def test_runs_on_the_given_stream():
    dev = device()
    w, h = _shard(wl.LLAMA3_8B_SHARD, 100_000, N=4, seed=60)
    d = to_dev(h, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        fl, sq = flags(dev)
        zs.zero_overflow_check(d["chunks"], w.loss_scale, fl, sq, stream=s)
        zs.zero_shard_step(d["chunks"], w.loss_scale, d["master"], d["m"], d["v"], d["p16"],
                           zs.adamw_params(w.hyper), stream=s)
    s.synchronize()
    assert_matches_oracle(d, _oracle(h, w.hyper, w.loss_scale))
