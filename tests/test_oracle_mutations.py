"""Plant plausible mistakes in copies of the oracle (CPU only) and require that at least
one pin rejects each.  This shows the pins are strong enough to trust the oracle."""
import types

import numpy as np
import pytest

import oracle as O
from oracle import mixllm_oracle as core
from tests import pins


def _ns(**over):
    ns = types.SimpleNamespace(**{k: getattr(core, k) for k in dir(core) if not k.startswith("__")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _act_round_half_up(a16, group=128):
    a = np.asarray(a16, np.float16).astype(np.float32)
    ag = a.reshape(a.shape[0], -1, group)
    amax = np.abs(ag).max(axis=2)
    sa = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(amax > 0, sa, np.float32(1))
    q = np.clip(np.floor(ag / safe[:, :, None] + np.float32(0.5)), -127, 127)
    q = np.where((amax > 0)[:, :, None], q, 0)
    return q.astype(np.int8).reshape(a.shape), sa, q.sum(axis=2).astype(np.int32)


def _act_per_token(a16, group=128):
    a = np.asarray(a16, np.float16).astype(np.float32)
    ag = a.reshape(a.shape[0], -1, group)
    amax = np.abs(a).max(axis=1, keepdims=True).repeat(ag.shape[1], axis=1)
    sa = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(amax > 0, sa, np.float32(1))
    q = np.clip(np.rint(ag / safe[:, :, None]), -127, 127)
    q = np.where((amax > 0)[:, :, None], q, 0)
    return q.astype(np.int8).reshape(a.shape), sa, q.sum(axis=2).astype(np.int32)


def _w8_div128(w16, group=128):
    w = np.asarray(w16, np.float16).astype(np.float32)
    wg = w.reshape(w.shape[0], -1, group)
    amax = np.abs(wg).max(axis=2)
    s16 = (amax / np.float32(128)).astype(np.float16)
    safe = np.where(amax > 0, s16.astype(np.float32), np.float32(1))
    q = np.clip(np.rint(wg / safe[:, :, None]), -127, 127)
    return q.astype(np.int8).reshape(w.shape), s16


def _w4_zero_sign(w16, group=128):
    q, z, s = core.quant_w4_asym(w16, group)
    w = np.asarray(w16, np.float16).astype(np.float32)
    wg = w.reshape(w.shape[0], -1, group)
    lo = np.minimum(wg.min(axis=2), 0)
    safe = np.where(s > 0, s.astype(np.float32), np.float32(1))
    z2 = np.clip(np.rint(lo / safe), 0, 15)
    q2 = np.clip(np.rint(wg / safe[:, :, None]) + z2[:, :, None], 0, 15)
    return q2.astype(np.uint8).reshape(w.shape), z2.astype(np.uint8), s


def _w4_plain_minmax(w16, group=128):
    """Range not widened to include 0."""
    w = np.asarray(w16, np.float16).astype(np.float32)
    wg = w.reshape(w.shape[0], -1, group)
    lo, hi = wg.min(axis=2), wg.max(axis=2)
    s16 = ((hi - lo) / np.float32(15)).astype(np.float16)
    safe = np.where(s16 > 0, s16.astype(np.float32), np.float32(1))
    z = np.clip(np.rint(-lo / safe), 0, 15)
    q = np.clip(np.rint(wg / safe[:, :, None]) + z[:, :, None], 0, 15)
    return q.astype(np.uint8).reshape(w.shape), z.astype(np.uint8), s16


def _gemm_drop_zero(aq, sa, q, z, s16, group=128):
    return core.gemm_mixed(aq, sa, q, np.zeros_like(z), s16, group)


def _gemm_first_group_scale(aq, sa, q, z, s16, group=128):
    s = np.repeat(s16[:, :1], s16.shape[1], axis=1)
    return core.gemm_mixed(aq, sa, q, z, s, group)


def _gemm_sa_wrong_group(aq, sa, q, z, s16, group=128):
    return core.gemm_mixed(aq, np.roll(sa, 1, axis=1), q, z, s16, group)


def _gemm_neg(aq, sa, q, z, s16, group=128):
    y = core.gemm_mixed(aq, sa, q, z, s16, group)
    y[:, 1::3] *= -1
    return y


def _partials_plus_z(aq, q, z, group=128):
    return core.partials(aq, q, (2 * z.astype(np.int64)) % 16, group)


def _mixed_swap_subsets(w16, idx8, group=128):
    n = np.asarray(w16).shape[0]
    other = np.setdiff1d(np.arange(n), np.asarray(idx8))
    return core.quant_weights_mixed(w16, other, group)


def _i2f_wrong_bias(i):
    i = np.asarray(i, np.int64)
    return ((np.int64(0x4B000000) + i).astype(np.uint32).view(np.float32) - np.float32(8388608.0))


def _eff_bits_wrong(p):
    return 4.0 + 4.4 * p


def _footprint_fp16_zero(bits, group=128):
    return 0.5 + 4.0 / group if bits == 4 else 1.0 + 2.0 / group


def _to_fp16_trunc(y64):
    """Round toward zero instead of to nearest even."""
    y = np.asarray(y64, np.float64)
    y16 = y.astype(np.float16)
    over = np.abs(y16.astype(np.float64)) > np.abs(y)
    y16[over] = np.nextafter(y16[over], np.float16(0))
    return y16


def _layer_with(**over):
    ns = _ns(**over)

    def layer_forward(a16, w16, idx8, group=128):
        aq, sa, ssum = ns.quant_act(a16, group)
        q, z, s16, is8 = ns.quant_weights_mixed(w16, idx8, group)
        y64 = ns.gemm_mixed(aq, sa, q, z, s16, group)
        return dict(aq=aq, sa=sa, s_sum=ssum, q=q, z=z, s16=s16, is8=is8, y64=y64,
                    y16=ns.to_fp16(y64))

    ns.layer_forward = layer_forward
    return ns


def _mixed_with(w4=None, w8=None):
    def quant_weights_mixed(w16, idx8, group=128):
        w16 = np.asarray(w16, np.float16)
        n, k = w16.shape
        is8 = np.zeros(n, bool)
        is8[np.asarray(idx8, np.int64)] = True
        q = np.zeros((n, k), np.int16)
        z = np.zeros((n, k // group), np.uint8)
        s = np.zeros((n, k // group), np.float16)
        if is8.any():
            q8, s8 = (w8 or core.quant_w8_sym)(w16[is8], group)
            q[is8], s[is8] = q8, s8
        if (~is8).any():
            q4, z4, s4 = (w4 or core.quant_w4_asym)(w16[~is8], group)
            q[~is8], z[~is8], s[~is8] = q4, z4, s4
        return q, z, s, is8
    return quant_weights_mixed


def _sal_with(form):
    def channel_salience(w16, grads, group=128):
        d = core.w4_perturbation(w16, group)
        t = np.einsum("dnk,nk->dn", np.asarray(grads, np.float64), d)
        return form(t)
    return channel_salience


def _assign_ascending(scores, total):
    return core.assign_channels([-np.asarray(s, np.float64) for s in scores], total)


def _assign_per_layer(scores, total):
    n = sum(len(s) for s in scores)
    out = []
    for s in scores:
        k = int(round(total * len(s) / n))
        out.append(np.sort(np.argsort(-np.asarray(s))[:k]).astype(np.int32))
    return out


def _ulp_doubled(y16):
    """The tolerance's ulp one binade too coarse."""
    y = np.abs(np.asarray(y16, dtype=np.float64))
    out = np.full(y.shape, 2.0 ** -24)
    normal = y >= 2.0 ** -14
    out[normal] = 2.0 ** (np.floor(np.log2(y[normal])) - 9)
    return out


def _ulp_no_subnormal_floor(y16):
    """Subnormal and zero outputs given a zero tolerance."""
    y = np.abs(np.asarray(y16, dtype=np.float64))
    out = np.zeros(y.shape)
    normal = y >= 2.0 ** -14
    out[normal] = 2.0 ** (np.floor(np.log2(y[normal])) - 10)
    return out


def _mlp_gate_up_swapped(x16, w_gate, w_up, w_down, idx8_gate, idx8_up, idx8_down, group=128):
    """SiLU applied to the up projection instead of the gate."""
    return core.mlp_block_forward(x16, w_up, w_gate, w_down, idx8_up, idx8_gate, idx8_down, group)


MUTANTS = {
    "act_round_half_up": _layer_with(quant_act=_act_round_half_up),
    "act_per_token_scale": _layer_with(quant_act=_act_per_token),
    "w8_divisor_128": _layer_with(quant_w8_sym=_w8_div128,
                                  quant_weights_mixed=_mixed_with(w8=_w8_div128)),
    "w4_zero_point_sign": _layer_with(quant_w4_asym=_w4_zero_sign,
                                      quant_weights_mixed=_mixed_with(w4=_w4_zero_sign)),
    "w4_range_not_widened": _layer_with(quant_w4_asym=_w4_plain_minmax,
                                        quant_weights_mixed=_mixed_with(w4=_w4_plain_minmax)),
    "gemm_drops_zero_point": _layer_with(gemm_mixed=_gemm_drop_zero),
    "gemm_one_weight_scale": _layer_with(gemm_mixed=_gemm_first_group_scale),
    "gemm_act_scale_off_by_one_group": _layer_with(gemm_mixed=_gemm_sa_wrong_group),
    "gemm_sign_error": _layer_with(gemm_mixed=_gemm_neg),
    "partials_wrong_zero": _layer_with(partials=_partials_plus_z),
    "subsets_swapped": _layer_with(quant_weights_mixed=_mixed_swap_subsets),
    "i2f_wrong_bias": _ns(i2f_bias=_i2f_wrong_bias),
    "effective_bits_wrong": _ns(effective_bits=_eff_bits_wrong),
    "w4_zero_as_fp16": _ns(weight_footprint=_footprint_fp16_zero),
    "fp16_truncation": _layer_with(to_fp16=_to_fp16_trunc),
    "salience_first_order_dropped": _ns(channel_salience=_sal_with(lambda t: np.mean(np.abs(0.5 * t * t), axis=0))),
    "salience_abs_outside": _ns(channel_salience=_sal_with(lambda t: np.mean(np.abs(t) + 0.5 * t * t, axis=0))),
    "salience_no_half": _ns(channel_salience=_sal_with(lambda t: np.mean(np.abs(t + t * t), axis=0))),
    "salience_sum_not_mean": _ns(channel_salience=_sal_with(lambda t: np.sum(np.abs(t + 0.5 * t * t), axis=0))),
    "salience_perturbation_sign": _ns(channel_salience=_sal_with(lambda t: np.mean(np.abs(-t + 0.5 * t * t), axis=0))),
    "assign_lowest": _ns(assign_channels=_assign_ascending),
    "assign_per_layer": _ns(assign_channels=_assign_per_layer),
    "silu_sign": _ns(silu=lambda x: np.asarray(x, np.float64) / (1.0 + np.exp(np.asarray(x, np.float64)))),
    "silu_sigmoid_only": _ns(silu=lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))),
    "ulp_doubled": _ns(ulp_fp16=_ulp_doubled),
    "ulp_no_subnormal_floor": _ns(ulp_fp16=_ulp_no_subnormal_floor),
    "mlp_gate_up_swapped": _ns(mlp_block_forward=_mlp_gate_up_swapped),
}


def _caught(ns):
    for pin in pins.ALL_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError, IndexError, OverflowError):
            return pin.__name__
    return None


def test_real_oracle_passes_every_pin():
    assert _caught(_ns()) is None
    assert _caught(O) is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _caught(MUTANTS[name]) is not None, f"no pin catches mutant {name}"
