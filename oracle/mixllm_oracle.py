"""Plain CPU oracle of the MixLLM W4.4A8 output-channel mixed-precision linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code, tables or helpers with the HIP
library under ``weight_activation_quantized_amd/``.

Sources (the pages this follows; section names are given as printed on them):

* "MixLLM talk notes" -- the MLSys 2026 talk-notes page "MixLLM: LLM Quantization
  with Global Mixed-precision between Output-features and Highly-efficient System
  Design" on notes.yuuk.io.  Sections used: 設計判断の概要 (design decisions),
  量子化構成の選択 (quantization configurations), 二段階逆量子化による int8 Tensor
  Core 活用 (two-step dequantization), 高速 I2F 変換 (fast I2F),
  ルーフラインモデルによる性能分析 (roofline model).
* "MixLLM summary page" -- the awesome-system-papers page "MixLLM: LLM
  Quantization with Global Mixed-precision between Output-features and
  Highly-efficient System Design (MLSys 2026)".  Sections used: 核心方法 (core
  method), 关键观察 / 隐含假设 (observation 3: arithmetic intensity).

What the method computes (core method; two-step dequantization):

* activations: 8-bit symmetric, round-to-nearest, one scale per token and per
  128-wide group of input features;
* weights: each output channel is either 8-bit symmetric (the ~10% salient
  channels) or 4-bit asymmetric (value, zero point, scale), group size 128;
* output: Y[m, n] = sum_g s_w[n, g] * s_a[m, g] * sum_{k in g} (W_q[n, k] - z[n, g]) * A_q[m, k],
  i.e. an exact integer dot product inside each group, then one scale per group.

Readings of points the pages leave open (each is also listed in the design notes):

* RTN ties round half to even (numpy ``rint``).
* Symmetric codes use the range [-127, 127] and the scale amax / 127.
* The asymmetric range is the group's [min, max] widened to include 0, the scale
  is (max - min) / 15, the zero point is a 4-bit integer round(-min / s), and the
  code is clamp(round(w / s) + z, 0, 15).
* Weight scales are stored as fp16 (round to nearest even from the fp32 value);
  the codes are computed with the stored fp16 scale.  A scale that underflows to
  zero for a non-zero group becomes 2**-24, the smallest fp16 subnormal.
* Activation scales are fp32.
* Divisions are IEEE fp32 divisions x / s (never x * (1/s)).
* The contraction is exact integer arithmetic; the group fold is done in fp64 and
  rounded once to fp16 (round to nearest even).  No bias term (the pages never
  mention one).

Precision: integer work is exact.  The oracle evaluates each group's integer
contraction as an fp64 BLAS matmul of small integers; every operand and every
partial sum is an integer below 2**22, far inside fp64's exact-integer range, so
the result is exact.
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# --------------------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------------------

_F16_MIN_SUBNORMAL = np.float16(2.0 ** -24)


def _groups(x32: np.ndarray, group: int) -> np.ndarray:
    rows, k = x32.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    return x32.reshape(rows, k // group, group)


def _fp16_scale(s32: np.ndarray, nonzero: np.ndarray) -> np.ndarray:
    """fp32 scale -> stored fp16 scale (round to nearest even), with the underflow rule."""
    s16 = s32.astype(np.float16)
    s16 = np.where(nonzero & (s16 == 0), _F16_MIN_SUBNORMAL, s16)
    return np.where(nonzero, s16, np.float16(0)).astype(np.float16)


def quant_w8_sym(w16: np.ndarray, group: int = GROUP):
    """8-bit symmetric group-wise RTN weight quantizer.

    MixLLM talk notes, 設計判断の概要: salient output channels are promoted to 8-bit
    *symmetric* quantization; roofline section: footprint 1 + 2/G bytes per element
    (int8 code + fp16 scale per group).

    Returns (q int8 [N, K] in [-127, 127], s16 fp16 [N, G]).  Dequantized value is q * s16.
    """
    w = np.asarray(w16, dtype=np.float16).astype(np.float32)
    wg = _groups(w, group)
    amax = np.abs(wg).max(axis=2)
    nonzero = amax > 0
    s32 = amax / np.float32(127.0)
    s16 = _fp16_scale(s32, nonzero)
    sdiv = s16.astype(np.float32)
    safe = np.where(nonzero, sdiv, np.float32(1.0))
    q = np.clip(np.rint(wg / safe[:, :, None]), -127, 127)
    q = np.where(nonzero[:, :, None], q, 0)
    return q.astype(np.int8).reshape(w.shape), s16


def quant_w4_asym(w16: np.ndarray, group: int = GROUP):
    """4-bit asymmetric group-wise RTN weight quantizer.

    MixLLM talk notes, 二段階逆量子化: the dequantized weight is (W_q - z) * s_w with a
    4-bit W_q and a zero point z whose subtraction stays in int8 range; roofline
    section: footprint 0.5 + 2.5/G bytes per element (4-bit code, 4-bit zero point,
    fp16 scale).

    Returns (q uint8 [N, K] in [0, 15], z uint8 [N, G] in [0, 15], s16 fp16 [N, G]).
    """
    w = np.asarray(w16, dtype=np.float16).astype(np.float32)
    wg = _groups(w, group)
    lo = np.minimum(wg.min(axis=2), np.float32(0.0))
    hi = np.maximum(wg.max(axis=2), np.float32(0.0))
    rng = hi - lo  # fp32 subtraction
    nonzero = rng > 0
    s32 = rng / np.float32(15.0)
    s16 = _fp16_scale(s32, nonzero)
    sdiv = s16.astype(np.float32)
    safe = np.where(nonzero, sdiv, np.float32(1.0))
    z = np.clip(np.rint(-lo / safe), 0, 15)
    q = np.clip(np.rint(wg / safe[:, :, None]) + z[:, :, None], 0, 15)
    z = np.where(nonzero, z, 0)
    q = np.where(nonzero[:, :, None], q, 0)
    return q.astype(np.uint8).reshape(w.shape), z.astype(np.uint8), s16


def quant_act(a16: np.ndarray, group: int = GROUP):
    """8-bit symmetric per-token, group-wise RTN activation quantizer.

    MixLLM talk notes, 設計判断の概要 (activations: 8-bit symmetric, group-wise RTN)
    and アブレーション研究 (activation groups of 128).

    Returns (q int8 [M, K], s_a fp32 [M, G], S_A int32 [M, G] = per-group code sums).
    """
    a = np.asarray(a16, dtype=np.float16).astype(np.float32)
    ag = _groups(a, group)
    amax = np.abs(ag).max(axis=2)
    nonzero = amax > 0
    sa = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(nonzero, sa, np.float32(1.0))
    q = np.clip(np.rint(ag / safe[:, :, None]), -127, 127)
    q = np.where(nonzero[:, :, None], q, 0)
    s_sum = q.astype(np.int64).sum(axis=2).astype(np.int32)
    return q.astype(np.int8).reshape(a.shape), sa, s_sum


def quant_weights_mixed(w16: np.ndarray, idx8, group: int = GROUP):
    """Quantize the two disjoint channel subsets (MixLLM summary page, 核心方法: global
    top channels 8-bit symmetric, the rest 4-bit asymmetric).

    Returns, in original channel order: q int16 [N, K] (uint4 codes for 4-bit
    channels, int8 codes for 8-bit channels), z uint8 [N, G] (0 for 8-bit channels),
    s16 fp16 [N, G], is8 bool [N].
    """
    w16 = np.asarray(w16, dtype=np.float16)
    n, k = w16.shape
    g = k // group
    is8 = np.zeros(n, dtype=bool)
    idx8 = np.asarray(idx8, dtype=np.int64)
    if idx8.size:
        if idx8.min() < 0 or idx8.max() >= n or np.unique(idx8).size != idx8.size:
            raise ValueError("idx8 must hold distinct channel indices in [0, N)")
        is8[idx8] = True
    q = np.zeros((n, k), dtype=np.int16)
    z = np.zeros((n, g), dtype=np.uint8)
    s16 = np.zeros((n, g), dtype=np.float16)
    if is8.any():
        q8, s8 = quant_w8_sym(w16[is8], group)
        q[is8] = q8
        s16[is8] = s8
    if (~is8).any():
        q4, z4, s4 = quant_w4_asym(w16[~is8], group)
        q[~is8] = q4
        z[~is8] = z4
        s16[~is8] = s4
    return q, z, s16, is8


# --------------------------------------------------------------------------------------
# Two-step dequantized GEMM
# --------------------------------------------------------------------------------------

def partials(aq: np.ndarray, q: np.ndarray, z: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Step 1-2 of the two-step dequantization (MixLLM talk notes, 二段階逆量子化):
    P[m, n, g] = sum_{k in group g} (q[n, k] - z[n, g]) * aq[m, k], exact integers.

    Each group is one fp64 BLAS matmul of small integers (exact, see module doc).
    Returns int64 [M, N, G].
    """
    m, k = aq.shape
    n = q.shape[0]
    g_count = k // group
    out = np.empty((m, n, g_count), dtype=np.int64)
    a64 = aq.astype(np.float64)
    for g in range(g_count):
        sl = slice(g * group, (g + 1) * group)
        wd = q[:, sl].astype(np.float64) - z[:, g].astype(np.float64)[:, None]
        out[:, :, g] = np.rint(a64[:, sl] @ wd.T).astype(np.int64)
    return out


def gemm_mixed(aq: np.ndarray, sa: np.ndarray, q: np.ndarray, z: np.ndarray,
               s16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Step 3 of the two-step dequantization: Y64[m, n] = sum_g s_w[n,g] * s_a[m,g] * P[m,n,g].

    MixLLM talk notes, 二段階逆量子化 (scale s_w * s_a applied per group after the
    integer MatMul) and 並列実行 (each output channel is written at its own index:
    the result is in original channel order).  Accumulated in fp64.
    Returns float64 [M, N]; ``to_fp16`` gives the layer output.
    """
    m, k = aq.shape
    n = q.shape[0]
    g_count = k // group
    y = np.zeros((m, n), dtype=np.float64)
    a64 = aq.astype(np.float64)
    for g in range(g_count):
        sl = slice(g * group, (g + 1) * group)
        wd = q[:, sl].astype(np.float64) - z[:, g].astype(np.float64)[:, None]
        p = a64[:, sl] @ wd.T  # exact integers
        y += (sa[:, g].astype(np.float64)[:, None] * s16[:, g].astype(np.float64)[None, :]) * p
    return y


def to_fp16(y64: np.ndarray) -> np.ndarray:
    """Round the fp64 result once to fp16 (round to nearest even)."""
    y16 = np.asarray(y64, dtype=np.float64).astype(np.float16)
    if not np.all(np.isfinite(y16)):
        raise OverflowError("layer output overflows fp16")
    return y16


def layer_forward(a16: np.ndarray, w16: np.ndarray, idx8, group: int = GROUP):
    """The whole layer: quantize activations, quantize both weight subsets, two-step
    dequantized GEMM, fp16 output in original channel order.  Returns a dict."""
    aq, sa, s_sum = quant_act(a16, group)
    q, z, s16, is8 = quant_weights_mixed(w16, idx8, group)
    y64 = gemm_mixed(aq, sa, q, z, s16, group)
    return dict(aq=aq, sa=sa, s_sum=s_sum, q=q, z=z, s16=s16, is8=is8, y64=y64, y16=to_fp16(y64))


# --------------------------------------------------------------------------------------
# The Llama MLP block around the layer (the gate/up and down projections whose shapes
# the talk notes time, A100 GPU でのシステム性能; the activation between them is the
# standard Llama one, SiLU(gate) * up, which the pages do not describe)
# --------------------------------------------------------------------------------------

def silu(x64: np.ndarray) -> np.ndarray:
    """SiLU(x) = x / (1 + e^-x) in fp64."""
    x = np.asarray(x64, np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def silu_mul_fp16(g16: np.ndarray, u16: np.ndarray) -> np.ndarray:
    """h = SiLU(gate) * up from fp16 inputs, in fp64, rounded once to fp16."""
    return to_fp16(silu(np.asarray(g16, np.float16).astype(np.float64))
                   * np.asarray(u16, np.float16).astype(np.float64))


def mlp_block_forward(x16, w_gate, w_up, w_down, idx8_gate, idx8_up, idx8_down, group: int = GROUP):
    """quantize x -> gate and up projections (one layer over the gate and up channels;
    columns are independent, so this equals the two layers) -> h = SiLU(gate) * up in
    fp16 -> quantize h -> down projection.  Returns a dict with the fp16 gate/up output,
    h and the block output."""
    inter = np.asarray(w_gate).shape[0]
    w_gu = np.concatenate([np.asarray(w_gate, np.float16), np.asarray(w_up, np.float16)])
    idx_gu = np.concatenate([np.asarray(idx8_gate, np.int64), np.asarray(idx8_up, np.int64) + inter])
    gu = layer_forward(x16, w_gu, idx_gu, group)
    h16 = silu_mul_fp16(gu["y16"][:, :inter], gu["y16"][:, inter:])
    dn = layer_forward(h16, w_down, idx8_down, group)
    return dict(gu16=gu["y16"], h16=h16, y16=dn["y16"], y64=dn["y64"], down=dn)


# --------------------------------------------------------------------------------------
# Uniform-precision layers, written separately (p0 = pure W4A8, p100 = pure W8A8)
# --------------------------------------------------------------------------------------

def _fold_int_partials(aq, sa, wd_int, s16, group):
    """Shared fold order for the pure routines; partials via exact int64 matmul."""
    m, k = aq.shape
    n = wd_int.shape[0]
    y = np.zeros((m, n), dtype=np.float64)
    a_int = aq.astype(np.int64)
    for g in range(k // group):
        sl = slice(g * group, (g + 1) * group)
        p = (a_int[:, sl] @ wd_int[:, sl].T).astype(np.float64)
        y += (sa[:, g].astype(np.float64)[:, None] * s16[:, g].astype(np.float64)[None, :]) * p
    return y


def gemm_w4a8_pure(a16: np.ndarray, w16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """All channels 4-bit asymmetric (the p0 configuration of 量子化構成の選択)."""
    aq, sa, _ = quant_act(a16, group)
    q, z, s16 = quant_w4_asym(w16, group)
    wd = q.astype(np.int64) - np.repeat(z.astype(np.int64), group, axis=1)
    return _fold_int_partials(aq, sa, wd, s16, group)


def gemm_w8a8_pure(a16: np.ndarray, w16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """All channels 8-bit symmetric (the p100 configuration of 量子化構成の選択)."""
    aq, sa, _ = quant_act(a16, group)
    q, s16 = quant_w8_sym(w16, group)
    return _fold_int_partials(aq, sa, q.astype(np.int64), s16, group)


# --------------------------------------------------------------------------------------
# Global output-channel precision search (MixLLM talk notes, グローバル混合精度探索;
# summary page, 核心方法)
# --------------------------------------------------------------------------------------

def w4_perturbation(w16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """c_q - c_0 for every output channel: the channel as the 4-bit asymmetric path stores
    it, dequantized ((q - z) * s16), minus the original fp16 weights.  fp64, exact."""
    q, z, s16 = quant_w4_asym(w16, group)
    n, k = q.shape
    g = k // group
    deq = (q.reshape(n, g, group).astype(np.float64) - z[:, :, None].astype(np.float64)) \
        * s16[:, :, None].astype(np.float64)
    return deq.reshape(n, k) - np.asarray(w16, np.float16).astype(np.float64)


def channel_salience(w16: np.ndarray, grads: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Salience of each output channel c of one layer: the loss change if only c is
    quantized, from a second-order Taylor expansion with the Hessian replaced by the
    empirical Fisher matrix (1/|D|) sum_d g_d g_d^T, which leaves one dot product per
    calibration sample d and keeps the first-order term:

        S_c = (1/|D|) sum_d | t_d + t_d^2 / 2 |,   t_d = g_d . (c_q - c_0)

    grads: [D, N, K] per-sample gradients of the loss w.r.t. the layer's weights.
    Returns fp64 [N]."""
    grads = np.asarray(grads, dtype=np.float32)
    delta = w4_perturbation(w16, group)
    t = np.einsum("dnk,nk->dn", grads.astype(np.float64), delta)
    return np.mean(np.abs(t + 0.5 * t * t), axis=0)


def assign_channels(scores, total_8bit: int):
    """The global assignment: every channel of every layer in one list, ranked by
    salience descending (ties: lower layer index, then lower channel index, first -- a
    reading; the pages do not order ties), the first ``total_8bit`` get 8 bits.
    scores: list of per-layer fp64 arrays.  Returns the per-layer sorted idx8 arrays."""
    layer = np.concatenate([np.full(len(s), i, np.int64) for i, s in enumerate(scores)])
    chan = np.concatenate([np.arange(len(s), dtype=np.int64) for s in scores])
    val = np.concatenate([np.asarray(s, np.float64) for s in scores])
    if total_8bit < 0 or total_8bit > len(val):
        raise ValueError("total_8bit out of range")
    order = np.lexsort((chan, layer, -val))  # last key is the primary one
    top = order[:total_8bit]
    return [np.sort(chan[top][layer[top] == i]).astype(np.int32) for i in range(len(scores))]


# --------------------------------------------------------------------------------------
# Fast int-to-float (MixLLM talk notes, 高速 I2F 変換)
# --------------------------------------------------------------------------------------

I2F_BIAS_BITS = 0x4B400000          # fp32 bit pattern of 1.5 * 2**23
I2F_BIAS_VALUE = np.float32(12582912.0)


def i2f_bias(i) -> np.ndarray:
    """Convert int32 values through the bias trick: add the bias bit pattern, reinterpret
    as fp32, subtract the bias value.  Exact for i in [-2**22, 2**22)."""
    i = np.asarray(i, dtype=np.int64)
    bits = (np.int64(I2F_BIAS_BITS) + i).astype(np.uint32)
    return bits.view(np.float32) - I2F_BIAS_VALUE


# --------------------------------------------------------------------------------------
# Byte and intensity model (MixLLM talk notes, ルーフラインモデル; summary page, 关键观察 3)
# --------------------------------------------------------------------------------------

def weight_footprint(bits: int, group: int = GROUP) -> float:
    """Bytes per weight element including group metadata: 8-bit symmetric 1 + 2/G
    (fp16 scale), 4-bit asymmetric 0.5 + 2.5/G (fp16 scale + 4-bit zero point)."""
    if bits == 8:
        return 1.0 + 2.0 / group
    if bits == 4:
        return 0.5 + 2.5 / group
    raise ValueError(bits)


def effective_bits(p8: float) -> float:
    """Average weight bit width when a fraction p8 of output channels is 8-bit and the
    rest 4-bit (量子化構成の選択)."""
    return 4.0 * (1.0 - p8) + 8.0 * p8


def operand_intensity(m: int, n: int, k: int, w_bits: int, a_bits: int) -> float:
    """ops / byte with bytes = weights + activations only (the model behind the
    summary page's observation 3 figures)."""
    return 2.0 * m * n * k / (n * k * w_bits / 8.0 + m * k * a_bits / 8.0)


def algorithmic_bytes(m: int, n: int, k: int, n8: int, group: int = GROUP,
                      with_act_sums: bool = False) -> float:
    """Bytes the mixed GEMM must move: packed 4-bit weights + zero points + scales,
    8-bit weights + scales, 4-byte channel index per output channel, int8
    activations + fp32 activation scales (+ int32 group sums if used), fp16 output."""
    g = k // group
    n4 = n - n8
    b = n4 * k / 2 + n4 * g * 2.5 + n8 * k + n8 * g * 2 + 4 * n
    b += m * k + 4 * m * g + (4 * m * g if with_act_sums else 0) + 2 * m * n
    return float(b)


def ulp_fp16(y16: np.ndarray) -> np.ndarray:
    """Spacing of fp16 numbers at |y|: 2**(floor(log2|y|) - 10) for normal values,
    2**-24 for subnormal values and zero."""
    y = np.abs(np.asarray(y16, dtype=np.float64))
    out = np.full(y.shape, 2.0 ** -24)
    normal = y >= 2.0 ** -14
    out[normal] = 2.0 ** (np.floor(np.log2(y[normal])) - 10)
    return out
