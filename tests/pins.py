"""Pins: checks that tie the CPU oracle to facts outside itself.

Each ``pin_*`` raises AssertionError when the oracle disagrees with what the
pages, the mathematics or an independent library fix.  The oracle is looked
up through its modules at call time, so a test can plant a mistake in it and
show that some pin catches the mistake.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.accounting as acc
import oracle.flatten as fl
import oracle.loss_scale as ls
import oracle.ring as ring
import oracle.zero_step as zs
from workloads import (LLAMA3_8B_SHARD, TINY, AdamWHyper, exactly_summable_fp16,
                       host_fp16_grad, host_normal_f32, seed_of)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits32(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _terms(s):
    return sorted(s.split("+"))


# --------------------------------------------------------------------------
# Replica sum: the pages' ring.
# --------------------------------------------------------------------------

def pin_ring_worked_example():
    """The simulated 3-GPU ring reproduces the walkthrough's rounds."""
    g = _golden("ring_3gpu_worked_example.json")
    init = [[(lbl,) for lbl in row] for row in g["initial"]]
    final, after_sr, log = ring.ring_allreduce(init, add=lambda a, b: a + b)
    letters = g["chunks"]
    for k, page_round in enumerate(g["scatter_reduce"]):
        msgs = [e for e in log if e["phase"] == "scatter_reduce" and e["round"] == k]
        assert len(msgs) == len(page_round)
        for pm in page_round:
            hit = [e for e in msgs if e["src"] == pm["src"] and e["dst"] == pm["dst"]]
            assert len(hit) == 1, pm
            e = hit[0]
            assert sorted(e["sent"]) == _terms(pm["sent"]), (e, pm)
            assert sorted(e["holds"]) == _terms(pm["holds"]), (e, pm)
            assert letters[e["chunk"]] == pm["sent"][0]
    rounds = {e["round"] for e in log if e["phase"] == "scatter_reduce"}
    assert len(rounds) == len(g["scatter_reduce"])
    for r, want in g["complete_after_scatter_reduce"].items():
        c = letters.index(want[0])
        assert sorted(after_sr[int(r)][c]) == _terms(want)
    for pm in g["all_gather_first_round"]:
        e = [e for e in log if e["phase"] == "all_gather" and e["round"] == 0
             and e["src"] == pm["src"]][0]
        assert e["dst"] == pm["dst"] and sorted(e["sent"]) == _terms(pm["sent"])
    for row in final:
        assert [sorted(v) for v in row] == [_terms(s) for s in g["final_every_gpu"]]


def _ring_sum(chunks):
    """Run the simulated ring on numeric chunks; every rank's full vector."""
    n_rep = len(chunks)
    n = chunks[0].size
    parts = np.array_split(np.arange(n), n_rep)
    holdings = [[chunks[r][p].astype(np.float32) for p in parts] for r in range(n_rep)]
    final, _, log = ring.ring_allreduce(holdings, add=np.add, size=lambda x: x.size)
    return [np.concatenate(row) for row in final], log


def pin_replica_sum_matches_ring():
    """On exactly summable fp16 inputs the oracle's sum equals, bit for bit,
    what every rank holds after the brute-force ring all-reduce."""
    for n_rep in range(2, 10):
        for n in (1, n_rep - 1, n_rep, 37, 1001):
            chunks = [exactly_summable_fp16(seed_of(90, n_rep, n, i), n)
                      for i in range(n_rep)]
            want = zs.replica_sum(chunks)
            assert want.dtype == np.float32 and want.shape == (n,)
            rows, _ = _ring_sum(chunks)
            for row in rows:
                assert np.array_equal(_bits32(row), _bits32(want)), (n_rep, n)


def pin_replica_sum_error_bound():
    """On inexact inputs (fp16 values of mixed magnitudes whose fp32 partial
    sums round), the oracle's sum lies within the error bound of recursive
    summation (Higham, Accuracy and Stability of Numerical Algorithms,
    section 4.2): |s - S| <= (N - 1) u sum |x_i|, u = 2^-24, where S is the
    exact sum.  For N <= 16 fp16 terms S is exact in float64 (the terms span
    at most 2^-24..2^16).  The ring's rotating order, the pages' own, meets
    the same bound, so the two orders differ by at most twice it; the
    order itself is a reading, the value is not."""
    rng = np.random.default_rng(seed_of(97))
    u = 2.0 ** -24
    for n_rep in (2, 3, 5, 8, 16):
        n = 4096
        chunks = []
        for _ in range(n_rep):
            mag = np.exp2(rng.integers(-20, 12, n)).astype(np.float64)
            x = (rng.standard_normal(n) * mag).astype(np.float16)
            chunks.append(x)
        exact = np.sum([c.astype(np.float64) for c in chunks], axis=0)
        bound = (n_rep - 1) * u * np.sum([np.abs(c.astype(np.float64)) for c in chunks], axis=0)
        s = zs.replica_sum(chunks).astype(np.float64)
        assert np.all(np.abs(s - exact) <= bound), n_rep
        rows, _ = _ring_sum(chunks)
        for row in rows:
            assert np.all(np.abs(row.astype(np.float64) - exact) <= bound), n_rep
        # the inputs are inexact: some partial sums do round
        assert np.any(s != exact), n_rep


def pin_ring_traffic():
    """Each rank sends 2 (N - 1) messages of psi / N elements (about 2 psi)."""
    for n_rep in (2, 3, 4, 8):
        n = 96
        chunks = [np.ones(n, np.float16) for _ in range(n_rep)]
        _, log = _ring_sum(chunks)
        for r in range(n_rep):
            mine = [e for e in log if e["src"] == r]
            assert len(mine) == 2 * (n_rep - 1)
            sent = sum(e["elements"] for e in mine)
            assert sent == acc.ring_allreduce_elements_sent_per_rank(n, n_rep)
    assert acc.ring_allreduce_elements_sent_per_rank(10 ** 9, 10 ** 4) / 10 ** 9 > 1.999


# --------------------------------------------------------------------------
# Mean and unscale.
# --------------------------------------------------------------------------

def pin_identical_replicas():
    """N identical replicas x give g = x / S exactly (power-of-two S): the
    sum is N x exactly, the mean x exactly, the unscale an exponent shift."""
    x = host_fp16_grad(seed_of(91), 4099, 1e-3, 1024.0)
    for n_rep in (1, 2, 3, 5, 7, 8, 16, 64):
        for log2s in (0, 10, 16, -3):
            g = zs.unscaled_grad([x] * n_rep, float(2.0 ** log2s))
            want = np.ldexp(x.astype(np.float64), -log2s).astype(np.float32)
            assert np.array_equal(_bits32(g), _bits32(want)), (n_rep, log2s)


def pin_mean_of_distinct_replicas():
    """Distinct exactly summable replicas: g is the exact sum divided by N S,
    rounded once (for N = 8 an exponent shift; for N = 3 a single rounding
    of s / 3, which never lands on an fp32 tie)."""
    for n_rep, log2s in ((8, 10), (3, 0), (3, 16), (5, 4)):
        chunks = [exactly_summable_fp16(seed_of(92, n_rep, i), 5003) for i in range(n_rep)]
        exact = np.sum([c.astype(np.float64) for c in chunks], axis=0)
        want = (exact / n_rep).astype(np.float32)
        want = np.ldexp(want.astype(np.float64), -log2s).astype(np.float32)
        g = zs.unscaled_grad(chunks, float(2.0 ** log2s))
        assert np.array_equal(_bits32(g), _bits32(want)), (n_rep, log2s)


# --------------------------------------------------------------------------
# Gradient-norm clipping.
# --------------------------------------------------------------------------

def pin_clip_matches_torch():
    """With fp64 gradients, torch.nn.utils.clip_grad_norm_ scales them by
    min(1, max_norm / (norm + 1e-6)); the oracle's fp32 clipped gradient
    agrees to within 2 fp32 roundings, and is left exactly unchanged when the
    norm is below the limit."""
    import torch
    chunks = [host_fp16_grad(seed_of(99, i), 30011, 1e-2, 1024.0) for i in range(4)]
    g = zs.unscaled_grad(chunks, 1024.0)
    sq = zs.grad_sqnorm(g)
    norm = math.sqrt(sq)
    for max_norm in (0.25 * norm, 0.999 * norm, 2.0 * norm, 0.0, -1.0):
        t = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
        t.grad = torch.from_numpy(g.astype(np.float64))
        if max_norm > 0:
            torch.nn.utils.clip_grad_norm_([t], max_norm)
        want = t.grad.numpy()
        got = (g * zs.clip_coefficient(sq, max_norm)).astype(np.float64)
        assert np.all(np.abs(got - want) <= 2 * 2.0 ** -24 * np.abs(want)), max_norm
        if not (0 < max_norm < norm):
            assert zs.clip_coefficient(sq, max_norm) == 1.0
            assert np.array_equal(_bits32(g * zs.clip_coefficient(sq, max_norm)), _bits32(g))


def pin_clip_closed_form():
    """Constant gradient c over n elements: the norm is |c| sqrt(n), so the
    factor is max_norm / (|c| sqrt(n) + 1e-6)."""
    n, c = 4096, 0.5                     # sum of squares 1024 exactly, norm 32
    ch = [np.full(n, c, np.float16)]
    r = zs.shard_step_clipped(ch, *(_zeros_state(n)), AdamWHyper(step=1, lr=1.0,
                                                               weight_decay=0.0), 1.0, 8.0)
    assert r.sqnorm == n * c * c
    assert zs.clip_coefficient(r.sqnorm, 8.0) == np.float32(8.0 / (32.0 + 1e-6))
    # first step, m = v = 0: m' = (1 - b1) * g_clipped
    gc = np.float32(c) * np.float32(8.0 / (32.0 + 1e-6))
    assert np.all(r.m == np.float32(1 - np.float32(0.9)) * gc)


def _zeros_state(n):
    master = np.zeros(n, np.float32)
    return master, np.zeros(n, np.float32), np.zeros(n, np.float32), master.astype(np.float16)


# --------------------------------------------------------------------------
# The page-literal split: the owner's mean stored as fp16.
# --------------------------------------------------------------------------

def _round_rne(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round the rational x to the nearest binary floating-point value with
    `mant_bits` significand bits (hidden bit included), exponents down to
    emin (subnormals below) and up to emax, ties to even; past the largest
    finite value it becomes +-inf (returned as None with the sign lost: the
    callers here never overflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)                      # subnormals share emin's quantum
    q = Fraction(2) ** (e - mant_bits + 1)  # value of one unit in the last place
    k, rem = divmod(a, q)
    k = int(k)
    if rem * 2 > q or (rem * 2 == q and k % 2 == 1):
        k += 1
    r = k * q
    assert r < Fraction(2) ** (emax + 1), "overflow not expected here"
    return sign * r


def pin_fp16_mean_is_rounded_exact_mean():
    """On exactly summable replicas the fp32 sum is exact, so the fp16 mean is
    the exact rational s / N rounded to binary32 (the division), then to
    binary16, both to nearest even: checked element by element with exact
    rational arithmetic, for both ways of forming it (all chunks at once,
    and one chunk arriving at a time)."""
    for n_rep in (3, 5, 7, 9):
        chunks = [exactly_summable_fp16(seed_of(97, n_rep, i), 257, bound_log2=4)
                  for i in range(n_rep)]
        for form in (zs.replica_mean_fp16, zs.accumulate_chunks):
            got = form(chunks)
            for j in range(got.size):
                s = sum(Fraction(float(c[j])) for c in chunks)
                want = _round_rne(_round_rne(s / n_rep, 24, -126, 127), 11, -14, 15)
                assert Fraction(float(got[j])) == want, (form.__name__, n_rep, j)


def pin_fp16_split_with_identical_replicas():
    """Identical replicas x: the mean is x, exactly representable in fp16, so
    the split (fp16 mean, then the update from it) equals the fused step bit
    for bit."""
    x = host_fp16_grad(seed_of(98), 2053, 1e-3, 1024.0)
    master = host_normal_f32(seed_of(98, 1), 2053, 0.02)
    m = np.abs(host_normal_f32(seed_of(98, 2), 2053, 1e-4))
    v = np.abs(host_normal_f32(seed_of(98, 3), 2053, 1e-8))
    p16 = master.astype(np.float16)
    hyp = AdamWHyper(step=17)
    for n_rep in (1, 3, 8):
        mean16 = zs.replica_mean_fp16([x] * n_rep)
        assert np.array_equal(mean16.view(np.uint16), x.view(np.uint16))
        a = zs.shard_step_from_fp16_mean(mean16, master, m, v, p16, hyp, 1024.0)
        b = zs.shard_step([x] * n_rep, master, m, v, p16, hyp, 1024.0)
        for u, w in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
            assert np.array_equal(_bits32(u), _bits32(w))
        assert np.array_equal(a.p16.view(np.uint16), b.p16.view(np.uint16))
        assert a.sqnorm == b.sqnorm and a.overflow == b.overflow is False


# --------------------------------------------------------------------------
# Overflow flag and squared norm.
# --------------------------------------------------------------------------

def pin_nonfinite_flag():
    base = [host_fp16_grad(seed_of(93, i), 1000, 1e-3, 1024.0) for i in range(3)]
    assert zs.check_only(base, 1024.0)[0] is False
    for chunk, idx, vals in ((2, 999, [np.inf]), (0, 0, [-np.inf]), (1, 500, [np.nan])):
        ch = [c.copy() for c in base]
        ch[chunk][idx] = vals[0]
        assert zs.check_only(ch, 1024.0)[0] is True
    ch = [c.copy() for c in base]
    ch[0][7], ch[1][7] = np.inf, -np.inf
    assert zs.check_only(ch, 1024.0)[0] is True
    big = [np.full(16, 65504.0, np.float16) for _ in range(64)]
    assert zs.check_only(big, 1.0)[0] is False
    x = [np.full(4, 60000.0, np.float16)]
    assert zs.check_only(x, 2.0 ** -120)[0] is True      # 60000 * 2^120 > FLT_MAX
    assert zs.check_only(x, 2.0 ** -100)[0] is False     # 60000 * 2^100 < FLT_MAX


def pin_sqnorm():
    c = [np.full(1000, 0.125, np.float16)] * 4
    assert zs.check_only(c, 1.0)[1] == 1000 / 64
    chunks = [host_fp16_grad(seed_of(94, i), 3001, 1e-3, 1024.0) for i in range(3)]
    g = zs.unscaled_grad(chunks, 1024.0)
    exact = math.fsum(float(v) * float(v) for v in g)
    got = zs.grad_sqnorm(g)
    assert abs(got - exact) <= 1e-13 * exact
    assert zs.grad_sqnorm(g[1234:], zs.grad_sqnorm(g[:1234])) == got


# --------------------------------------------------------------------------
# Adam / AdamW.
# --------------------------------------------------------------------------

def _tiny_inputs(n=20011, key=95):
    chunks = [host_fp16_grad(seed_of(key, i), n, TINY.grad_sigma, TINY.loss_scale)
              for i in range(TINY.n_replicas)]
    master = host_normal_f32(seed_of(key, 10), n, 0.02)
    zero = np.zeros(n, np.float32)
    return chunks, master, zero


def pin_first_step_closed_form():
    """t = 1, m = v = 0: m' = (1-b1) g, v' = (1-b2) g^2, the bias corrections
    cancel, so master' = p - lr wd p - lr g / (|g| + eps), i.e. about
    p - lr wd p - lr sign(g) when eps << |g|."""
    chunks, master, zero = _tiny_inputs()
    hyp = TINY.hyper
    r = zs.shard_step(chunks, master, zero, zero, master.astype(np.float16), hyp,
                      TINY.loss_scale)
    assert not r.overflow
    g = zs.unscaled_grad(chunks, TINY.loss_scale).astype(np.float64)
    b1, b2 = float(F32(hyp.beta1)), float(F32(hyp.beta2))
    lr, wd, eps = float(F32(hyp.lr)), float(F32(hyp.weight_decay)), float(F32(hyp.eps))
    p = master.astype(np.float64)
    np.testing.assert_allclose(r.m, (1 - b1) * g, rtol=2e-7, atol=0)
    np.testing.assert_allclose(r.v, (1 - b2) * g * g, rtol=4e-7, atol=0)
    want = p - lr * wd * p - lr * g / (np.abs(g) + eps)
    ulp = np.spacing(np.abs(r.master)).astype(np.float64)
    # u carries a few fp32 roundings (|u| ~ 1, error ~ 8 * 2^-24 at most)
    assert np.all(np.abs(r.master - want) <= 2 * ulp + lr * 8 * 2.0 ** -24)
    nz = g != 0
    approx = p - lr * wd * p - lr * np.sign(g)
    bound = lr * eps / np.abs(g[nz]) + 2 * ulp[nz] + lr * 8 * 2.0 ** -24
    assert np.all(np.abs(r.master[nz] - approx[nz]) <= bound)


def pin_zero_gradient():
    """g = 0: m' = b1 m and v' = b2 v, each one fp32 product."""
    n = 4097
    m = host_normal_f32(seed_of(96, 1), n, 1e-4)
    v = np.abs(host_normal_f32(seed_of(96, 2), n, 1e-8))
    master = host_normal_f32(seed_of(96, 3), n, 0.02)
    hyp = LLAMA3_8B_SHARD.hyper
    zero = [np.zeros(n, np.float16)] * 8
    r = zs.shard_step(zero, master, m, v, master.astype(np.float16), hyp, 65536.0)
    b1, b2 = float(F32(hyp.beta1)), float(F32(hyp.beta2))
    assert np.array_equal(_bits32(r.m), _bits32((b1 * m.astype(np.float64)).astype(np.float32)))
    assert np.array_equal(_bits32(r.v), _bits32((b2 * v.astype(np.float64)).astype(np.float32)))
    assert r.sqnorm == 0.0 and not r.overflow


def pin_lr_zero():
    """lr = 0 leaves the master weights unchanged, whatever wd and g are, and
    the fp16 params are the master rounded by torch's own fp16 conversion."""
    import torch
    chunks, master, zero = _tiny_inputs(5003, 97)
    hyp = AdamWHyper(lr=0.0, weight_decay=0.01, step=7)
    m = host_normal_f32(seed_of(97, 20), 5003, 1e-4)
    v = np.abs(host_normal_f32(seed_of(97, 21), 5003, 1e-8))
    r = zs.shard_step(chunks, master, m, v, master.astype(np.float16), hyp, 1024.0)
    assert np.array_equal(_bits32(r.master), _bits32(master))
    want = torch.from_numpy(master).half().numpy()
    assert np.array_equal(r.p16.view(np.uint16), want.view(np.uint16))


def _torch_adamw_step(g, master, m, v, hyp, adam_l2=False):
    import torch
    p = torch.nn.Parameter(torch.from_numpy(master.copy()))
    p.grad = torch.from_numpy(g.copy())
    cls = torch.optim.Adam if adam_l2 else torch.optim.AdamW
    f = lambda x: float(np.float32(x))     # the fp32 values the step holds
    opt = cls([p], lr=f(hyp.lr), betas=(f(hyp.beta1), f(hyp.beta2)), eps=f(hyp.eps),
              weight_decay=f(hyp.weight_decay), foreach=False, fused=False)
    opt.state[p] = {"step": torch.tensor(float(hyp.step - 1)),
                    "exp_avg": torch.from_numpy(m.copy()),
                    "exp_avg_sq": torch.from_numpy(v.copy())}
    opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def _within(got, want, scale, units):
    """|got - want| <= units * 2^-24 * scale, elementwise."""
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    return bool(np.all(err <= units * 2.0 ** -24 * scale))


def pin_torch_adamw():
    """N = 1 and S = 1 reduce the step to one plain fp32 AdamW (or L2 Adam)
    update of torch.optim on the CPU.  The two evaluate the same formula in
    different operation orders, so each result is compared within 16 fp32
    roundings of the magnitude of its own terms (beta1 |m| + (1-beta1) |g| for
    m, and so on).  torch receives the hyperparameters as the fp32 values the
    step holds, so both sides use the same betas, lr, eps and wd."""
    n = 6007
    dyadic = AdamWHyper(lr=2.0 ** -10, beta1=0.875, beta2=1 - 2.0 ** -9,
                        eps=2.0 ** -27, weight_decay=2.0 ** -6)
    cases = [(dyadic.replace(step=t), l2, (1e-1, 1e-2, 1e-3))
             for t in (1, 2, 17, 1000) for l2 in (False, True)]
    cases += [(LLAMA3_8B_SHARD.hyper.replace(step=t), l2, (3.5e-5, 1e-4, 1e-8))
              for t in (1000, 5000) for l2 in (False, True)]
    for hyp, l2, (gs, ms, vs) in cases:
        key = seed_of(98, hyp.step, int(l2), int(gs * 1e6))
        x = host_fp16_grad(seed_of(key, 0), n, gs, 1.0)
        g = x.astype(np.float64)
        master = host_normal_f32(seed_of(key, 1), n, 0.02)
        m = host_normal_f32(seed_of(key, 2), n, ms)
        v = np.abs(host_normal_f32(seed_of(key, 3), n, vs))
        if hyp.step == 1:
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
        hyp = hyp.replace(decoupled_wd=not l2)
        r = zs.shard_step([x], master, m, v, master.astype(np.float16), hyp, 1.0)
        tp, tm, tv = _torch_adamw_step(x.astype(np.float32), master, m, v, hyp, adam_l2=l2)
        b1, b2 = float(F32(hyp.beta1)), float(F32(hyp.beta2))
        if l2:
            g = g + hyp.weight_decay * master.astype(np.float64)
        assert _within(r.m, tm, b1 * np.abs(m) + (1 - b1) * np.abs(g), 16), (hyp, "m")
        assert _within(r.v, tv, b2 * v + (1 - b2) * g * g, 16), (hyp, "v")
        step = np.abs(tp.astype(np.float64) - master)
        assert _within(r.master, tp, np.abs(master) + step, 16), (hyp, "master")


def pin_fp16_writeback():
    """With lr = wd = 0 the fp16 params are the (unchanged) master rounded to
    binary16; golden IEEE cases fix ties, overflow and subnormals.  L2 mode
    with wd = 0 keeps -0 (the decoupled decay p - 0*p would give +0), and
    infinite masters are left out (0 * inf is NaN in either mode)."""
    g = _golden("fp16_rne_cases.json")
    cases = [c for c in g["cases"] if c[0] not in ("7f800000", "ff800000")]
    master = np.array([int(a, 16) for a, _, _ in cases], np.uint32).view(np.float32)
    want = np.array([int(b, 16) for _, b, _ in cases], np.uint16)
    n = master.size
    zero = np.zeros(n, np.float32)
    hyp = AdamWHyper(lr=0.0, weight_decay=0.0, step=3, decoupled_wd=False)
    r = zs.shard_step([np.zeros(n, np.float16)], master, zero, zero,
                      np.zeros(n, np.float16), hyp, 1.0)
    assert np.array_equal(r.p16.view(np.uint16), want)


def pin_update_order():
    """The fp16 params come from the new master, not the old one."""
    import torch
    chunks, master, zero = _tiny_inputs(4001, 99)
    hyp = AdamWHyper(lr=0.05, step=1)
    r = zs.shard_step(chunks, master, zero, zero, master.astype(np.float16), hyp, 1024.0)
    new16 = torch.from_numpy(r.master).half().numpy().view(np.uint16)
    old16 = torch.from_numpy(master).half().numpy().view(np.uint16)
    assert np.array_equal(r.p16.view(np.uint16), new16)
    assert np.mean(new16 != old16) > 0.9


def pin_skip_leaves_state():
    chunks, master, zero = _tiny_inputs(2003, 100)
    chunks[1][77] = np.nan
    m = host_normal_f32(seed_of(100, 5), 2003, 1e-4)
    p16 = master.astype(np.float16)
    r = zs.shard_step(chunks, master, m, zero, p16, TINY.hyper, 1024.0)
    assert r.overflow
    assert np.array_equal(_bits32(r.master), _bits32(master))
    assert np.array_equal(_bits32(r.m), _bits32(m))
    assert np.array_equal(_bits32(r.v), _bits32(zero))
    assert np.array_equal(r.p16.view(np.uint16), p16.view(np.uint16))


# --------------------------------------------------------------------------
# Byte accounting, loss scaler and bucket layout.
# --------------------------------------------------------------------------

def pin_accounting():
    """16 B per parameter under DDP (2 fp16 param + 2 fp16 grad + 12 fp32
    optimizer state: 4 m, 4 v, 4 master); ZeRO-1 ~4x and ZeRO-2 ~8x savings
    as N grows; ZeRO-3 N-fold."""
    assert acc.ddp_bytes_per_param() == 16
    assert acc.zero_bytes_per_param(0, 8) == 16
    big = 10 ** 9
    assert abs(16 / acc.zero_bytes_per_param(1, big) - 4) < 1e-6
    assert abs(16 / acc.zero_bytes_per_param(2, big) - 8) < 1e-6
    assert 16 / acc.zero_bytes_per_param(3, 64) == 64
    assert [acc.step_bytes_per_param(n) for n in (3, 8, 16)] == [32, 42, 58]
    assert acc.check_bytes_per_param(8) == 16


def pin_scaler():
    s = ls.ScalerState(scale=65536.0, growth_interval=3)
    seen = []
    for flag in (1, 0, 0, 0):
        skip = ls.update_loss_scale(s, bool(flag))
        seen.append((skip, s.scale))
    assert seen == [(True, 32768.0), (False, 32768.0), (False, 32768.0), (False, 65536.0)]
    assert s.skipped_steps == 1 and s.good_steps == 0
    s = ls.ScalerState(scale=1.0, min_scale=1.0)
    assert ls.update_loss_scale(s, True) and s.scale == 1.0
    s = ls.ScalerState(scale=2.0 ** 24, growth_interval=1)
    assert not ls.update_loss_scale(s, False) and s.scale == 2.0 ** 24
    s = ls.ScalerState(scale=4.0, growth_interval=2)
    for flag in (0, 1, 0):      # an overflow restarts the run of clean steps
        ls.update_loss_scale(s, bool(flag))
    assert s.scale == 2.0 and s.good_steps == 1


def pin_scaler_grad_scaler():
    """The reading of the scaler is the usual dynamic loss scaling, which
    torch's GradScaler (torch.amp, on the CPU) implements: driven by the same
    forced sequences of clean and overflowing steps (an inf gradient forces
    the overflow), it skips the same steps and walks the same scales and
    clean-step counts, for growth intervals 1, 2, 3 and 7, with the floor and
    ceiling out of reach."""
    import torch
    rng = np.random.default_rng(7)
    for interval in (1, 2, 3, 7):
        flags = rng.random(60) < 0.3
        ref = torch.amp.GradScaler("cpu", init_scale=1024.0, growth_factor=2.0,
                                   backoff_factor=0.5, growth_interval=interval)
        p = torch.nn.Parameter(torch.zeros(4))
        opt = torch.optim.SGD([p], lr=1.0)
        s = ls.ScalerState(scale=1024.0, growth_interval=interval, min_scale=2.0 ** -100,
                           max_scale=2.0 ** 100)
        for k, flag in enumerate(flags):
            ref.scale(torch.ones(()))
            before = p.detach().clone()
            p.grad = torch.full((4,), float("inf") if flag else 1.0)
            ref.step(opt)
            ref.update()
            skipped = torch.equal(before, p.detach())
            assert ls.update_loss_scale(s, bool(flag)) == skipped, (interval, k)
            assert s.scale == ref.get_scale(), (interval, k, s.scale, ref.get_scale())
            assert s.good_steps == ref._get_growth_tracker(), (interval, k)


def pin_flatten_layouts():
    for case in _golden("flatten_layouts.json")["cases"]:
        got = fl.bucket_layout(case["numels"], case["align"], case["pad_multiple"])
        assert got == case["offsets"], case
        tensors = [np.arange(1, k + 1, dtype=np.float16) for k in case["numels"]
                   if k <= 5000]
        if len(tensors) != len(case["numels"]):
            continue
        bucket, offs = fl.flatten(tensors, case["align"], case["pad_multiple"])
        mask = np.zeros(bucket.size, bool)
        for t, o in zip(tensors, offs):
            assert np.array_equal(bucket[o:o + t.size], t)
            mask[o:o + t.size] = True
        assert not np.any(bucket[~mask])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
