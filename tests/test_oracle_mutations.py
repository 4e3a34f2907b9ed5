"""Plant plausible mistakes in the CPU oracle and check that a pin catches
each one.  The mistakes live only in this file and only on the CPU; the
oracle itself is restored after every case by monkeypatch."""
import dataclasses

import numpy as np
import pytest

import oracle.flatten as fl
import oracle.loss_scale as ls
import oracle.zero_step as zs
import pins

pytestmark = pytest.mark.cpu

F32 = np.float32


def _adamw_variant(kind):
    """adamw_update with one planted mistake."""
    def update(g, master, m, v, hyper):
        k = zs.adam_constants(hyper)
        with np.errstate(all="ignore"):
            if not k.decoupled_wd:
                g = g - k.wd * master if kind == "l2_sign" else g + k.wd * master
            m1 = k.beta1 * m + k.c1 * g
            if kind == "v_linear":
                v1 = k.beta2 * v + k.c2 * g
            else:
                v1 = k.beta2 * v + (k.c2 * g) * g
            m_hat, v_hat = m1 / k.bc1, v1 / k.bc2
            if kind == "eps_inside_sqrt":
                u = m_hat / np.sqrt(v_hat + k.eps)
            elif kind == "m_v_transposed":
                u = v_hat / (np.sqrt(np.abs(m_hat)) + k.eps)
            else:
                u = m_hat / (np.sqrt(v_hat) + k.eps)
            if k.decoupled_wd:
                p = master + k.lrwd * master if kind == "wd_sign" else master - k.lrwd * master
            else:
                p = master
            master1 = p - k.lr * u
            src = master if kind == "p16_from_old_master" else master1
            return master1, m1, v1, src.astype(np.float16)
    return update


def _constants_variant(kind):
    orig = zs.adam_constants

    def constants(hyper):
        k = orig(hyper)
        if kind == "no_bias_correction":
            return dataclasses.replace(k, bc1=F32(1), bc2=F32(1))
        if kind == "bias_correction_t_minus_1":
            t = max(int(hyper.step) - 1, 1)
            return dataclasses.replace(k, bc1=F32(1 - float(k.beta1) ** t),
                                       bc2=F32(1 - float(k.beta2) ** t))
        if kind == "betas_swapped":
            return dataclasses.replace(k, beta1=k.beta2, beta2=k.beta1, c1=k.c2, c2=k.c1)
        if kind == "c2_from_beta1":
            return dataclasses.replace(k, c2=k.c1)
        if kind == "wd_ignored_in_decay":
            return dataclasses.replace(k, lrwd=k.lr)
        raise AssertionError(kind)
    return constants


def _sum_drop_last(chunks):
    s = zs.widen(chunks[0])
    for x in chunks[1:-1]:
        s = s + zs.widen(x)
    return s


def _sum_repeat_first(chunks):
    s = zs.widen(chunks[0])
    for x in chunks[:-1]:
        s = s + zs.widen(x)
    return s


def _scaler_grow_on_overflow(s, overflow):
    if overflow:
        s.scale = float(F32(s.scale) * F32(s.growth_factor))
        s.good_steps = 0
        s.skipped_steps += 1
        return True
    return _orig_scaler(s, overflow)


_orig_scaler = ls.update_loss_scale


def _scaler_no_reset(s, overflow):
    if overflow:
        s.scale = float(max(F32(s.scale) * F32(s.backoff_factor), F32(s.min_scale)))
        s.skipped_steps += 1
        return True
    return _orig_scaler(s, overflow)


def _scaler_grows_late(s, overflow):
    if overflow:
        return _orig_scaler(s, overflow)
    s.good_steps += 1
    if s.good_steps > s.growth_interval:
        s.scale = float(min(F32(s.scale) * F32(s.growth_factor), F32(s.max_scale)))
        s.good_steps = 0
    return False


def _layout_unaligned(numels, align, pad_multiple):
    offs, end = [], 0
    for k in numels:
        offs.append(end)
        end += int(k)
    offs.append(fl.round_up(end, pad_multiple))
    return offs


def _layout_no_pad(numels, align, pad_multiple):
    offs, end = [], 0
    for k in numels:
        start = fl.round_up(end, align)
        offs.append(start)
        end = start + int(k)
    offs.append(end)
    return offs


MUTATIONS = {
    "sum_drops_last_replica": (zs, "replica_sum", _sum_drop_last),
    "sum_repeats_first_replica": (zs, "replica_sum", _sum_repeat_first),
    "mean_divides_by_n_minus_1": (zs, "replica_mean", lambda s, n: s / F32(max(n - 1, 1))),
    "mean_not_divided": (zs, "replica_mean", lambda s, n: s),
    "unscale_multiplies": (zs, "unscale", lambda mean, S: mean * F32(S)),
    "flag_inverted": (zs, "nonfinite", lambda g: bool(np.all(np.isfinite(g)))),
    "flag_misses_inf": (zs, "nonfinite", lambda g: bool(np.any(np.isnan(g)))),
    "sqnorm_of_abs": (zs, "grad_sqnorm",
                      lambda g, start=0.0: float(start + np.sum(np.abs(g.astype(np.float64))))),
    "sqnorm_drops_start": (zs, "grad_sqnorm",
                           lambda g, start=0.0: float(np.sum(np.square(g.astype(np.float64))))),
    "scaler_grows_on_overflow": (ls, "update_loss_scale", _scaler_grow_on_overflow),
    "scaler_keeps_clean_run": (ls, "update_loss_scale", _scaler_no_reset),
    "scaler_grows_one_step_late": (ls, "update_loss_scale", _scaler_grows_late),
    "layout_unaligned_starts": (fl, "bucket_layout", _layout_unaligned),
    "layout_no_padding": (fl, "bucket_layout", _layout_no_pad),
}
for _k in ("no_bias_correction", "bias_correction_t_minus_1", "betas_swapped",
           "c2_from_beta1", "wd_ignored_in_decay"):
    MUTATIONS[_k] = (zs, "adam_constants", _constants_variant(_k))
for _k in ("eps_inside_sqrt", "m_v_transposed", "wd_sign", "p16_from_old_master",
           "v_linear", "l2_sign"):
    MUTATIONS[_k] = (zs, "adamw_update", _adamw_variant(_k))


def _mean16_toward_zero(chunks):
    """The fp16 mean rounded toward zero instead of to nearest even."""
    x = zs.replica_mean(zs.replica_sum(chunks), len(chunks))
    h = x.astype(np.float16)
    away = np.abs(h.astype(np.float32)) > np.abs(x)
    return np.where(away, np.nextafter(h, np.float16(0)), h).astype(np.float16)


def _accumulate_drops_last(chunks):
    acc = zs.widen(chunks[0])
    for c in chunks[1:-1]:
        acc = acc + zs.widen(c)
    return (acc / F32(len(chunks))).astype(np.float16)


def _split_unscale_multiplies(mean16, master, m, v, p16, hyper, loss_scale, sqnorm_start=0.0):
    g = zs.widen(mean16) * F32(loss_scale)
    return zs.step_from_grad(g, master, m, v, p16, hyper, sqnorm_start)


def _clip_variant(kind):
    def coef(sqnorm, max_norm):
        if not max_norm > 0.0:
            return F32(1.0)
        if kind == "no_clamp":
            return F32(max_norm / (np.sqrt(sqnorm) + 1e-6))
        if kind == "squared_norm":
            return F32(min(1.0, max_norm / (sqnorm + 1e-6)))
        if kind == "inverted":
            return F32(min(1.0, (np.sqrt(sqnorm) + 1e-6) / max_norm))
        raise ValueError(kind)
    return coef


def _clipped_step_variant(kind):
    def step(chunks, master, m, v, p16, hyper, loss_scale, max_norm):
        g = zs.unscaled_grad(chunks, loss_scale)
        flag = zs.nonfinite(g)
        sq = zs.grad_sqnorm(g)
        if flag:
            return zs.StepResult(True, sq, master.copy(), m.copy(), v.copy(), p16.copy())
        gc = g * zs.clip_coefficient(sq, max_norm)
        if kind == "norm_after_clip":
            sq = zs.grad_sqnorm(gc)
        elif kind == "update_unclipped":
            gc = g
        master1, m1, v1, p161 = zs.adamw_update(gc, master, m, v, hyper)
        return zs.StepResult(False, sq, master1, m1, v1, p161)
    return step


MUTATIONS.update({
    "clipped_step_norm_after_clip": (zs, "shard_step_clipped",
                                     _clipped_step_variant("norm_after_clip")),
    "clipped_step_updates_unclipped": (zs, "shard_step_clipped",
                                       _clipped_step_variant("update_unclipped")),
    "clip_not_clamped_to_one": (zs, "clip_coefficient", _clip_variant("no_clamp")),
    "clip_by_squared_norm": (zs, "clip_coefficient", _clip_variant("squared_norm")),
    "clip_inverted": (zs, "clip_coefficient", _clip_variant("inverted")),
    "mean16_rounds_toward_zero": (zs, "replica_mean_fp16", _mean16_toward_zero),
    "mean16_not_divided": (zs, "replica_mean_fp16",
                           lambda chunks: zs.replica_sum(chunks).astype(np.float16)),
    "accumulate_drops_last_arrival": (zs, "accumulate_chunks", _accumulate_drops_last),
    "split_unscale_multiplies": (zs, "shard_step_from_fp16_mean", _split_unscale_multiplies),
})


def test_unmutated_variants_pass(monkeypatch):
    """The variant machinery itself, with no mistake planted, passes every pin."""
    monkeypatch.setattr(zs, "adamw_update", _adamw_variant("none"))
    for pin in pins.ALL_PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
