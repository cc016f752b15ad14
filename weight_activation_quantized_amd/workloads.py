"""Seeded synthetic inputs for the W4.4A8 mixed linear layer.

This module only draws random numbers and picks shapes; it holds none of the
method's arithmetic (no quantization, no contraction).  Both the HIP path's tests
and the CPU oracle take their inputs from here.

Distributions (the pages measure single linear layers with synthetic shapes,
K = 4096 and N in {4096, 14336}, tokens 1..1024: MixLLM talk notes, section
A100 GPU でのシステム性能; no dataset is involved):

* weights: N(0, 0.02) in float64, 4 seeded output channels scaled x8 (outliers),
  cast once to fp16;
* 8-bit channel set: a seeded permutation of the channels, independent of the
  outliers, first n8 sorted ascending;
* activations: N(0, 1) in float64 with ceil(0.02 K) seeded input columns scaled
  x20, cast once to fp16; or Student-t(3) values (heavy tails) cast to fp16.

Per-layer 8-bit counts for the Llama-3.1-8B-shaped block follow the per-layer
fractions the talk notes report (探索の特性 / 核心的洞察: v_proj 71.22%,
down_proj 53.82%, gate_proj 0.73%), with the remaining budget of the global 10%
split over the other layers by largest remainder.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GROUP = 128


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def make_weights(n: int, k: int, seed) -> np.ndarray:
    """fp16 [N, K] weights ~ N(0, 0.02), 4 channels x8."""
    rng = _rng(*seed, 1)
    w = rng.normal(0.0, 0.02, size=(n, k))
    out = rng.permutation(n)[: min(4, n)]
    w[out] *= 8.0
    return w.astype(np.float16)


def make_idx8(n: int, n8: int, seed) -> np.ndarray:
    """Sorted int32 indices of the n8 8-bit channels."""
    rng = _rng(*seed, 2)
    return np.sort(rng.permutation(n)[:n8]).astype(np.int32)


def make_acts(m: int, k: int, seed, dist: str = "normal") -> np.ndarray:
    """fp16 [M, K] activations."""
    rng = _rng(*seed, 3)
    if dist == "normal":
        a = rng.standard_normal(size=(m, k))
        cols = rng.permutation(k)[: int(math.ceil(0.02 * k))]
        a[:, cols] *= 20.0
    elif dist == "t3":
        a = rng.standard_t(3, size=(m, k))
    else:
        raise ValueError(dist)
    return a.astype(np.float16)


@dataclass(frozen=True)
class Shape:
    cfg: int
    layer: str
    m: int
    n: int
    k: int
    n8: int
    dist: str = "normal"

    @property
    def seed(self):
        """Seed of the activations (one batch per token count)."""
        return (self.cfg, _LAYER_IDS[self.layer], self.m)

    @property
    def wseed(self):
        """Seed of the weights and of the 8-bit channel set (shared by all token counts)."""
        return (self.cfg, _LAYER_IDS[self.layer], 0, self.n, self.k)

    @property
    def name(self) -> str:
        return f"cfg{self.cfg}-{self.layer}-M{self.m}-N{self.n}-K{self.k}-n8_{self.n8}"


_LAYER_IDS = {name: i for i, name in enumerate(
    ["tiny", "p0", "p10", "p20", "p50", "p100", "q", "k", "v", "o", "gate", "up", "down",
     "qo", "kv", "edge"])}


def n8_fraction(n: int, p: float) -> int:
    """ceil(p * N) 8-bit channels."""
    return int(math.ceil(round(p * n, 9)))


# Llama-3.1-8B block: (layer, N, K)
LLAMA8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
           ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LLAMA8B_FIXED = {"v": 0.7122, "down": 0.5382, "gate": 0.0073}


def llama8b_n8() -> dict:
    """Per-layer 8-bit channel counts for one Llama-3.1-8B-shaped block: 10% of the
    block's 43008 output channels, v/down/gate at the reported fractions, the rest
    spread over q/k/o/up in proportion to N by largest remainder."""
    total_n = sum(n for _, n, _ in LLAMA8B)
    budget = n8_fraction(total_n, 0.10)
    fixed = {name: int(round(LLAMA8B_FIXED[name] * n)) for name, n, _ in LLAMA8B
             if name in LLAMA8B_FIXED}
    rest = budget - sum(fixed.values())
    others = [(name, n) for name, n, _ in LLAMA8B if name not in LLAMA8B_FIXED]
    n_other = sum(n for _, n in others)
    quotas = [(name, rest * n / n_other) for name, n in others]
    base = {name: int(math.floor(x)) for name, x in quotas}
    left = rest - sum(base.values())
    pos = {name: i for i, (name, _, _) in enumerate(LLAMA8B)}
    order = sorted(quotas, key=lambda t: (-(t[1] - math.floor(t[1])), pos[t[0]]))
    for name, _ in order[:left]:
        base[name] += 1
    out = dict(fixed)
    out.update(base)
    return out


def config_shapes(cfg: int):
    """Every (layer, M) shape of one of the five workloads."""
    if cfg == 0:
        return [Shape(0, "tiny", 16, 512, 1024, n8_fraction(512, 0.10))]
    if cfg == 1:
        return [Shape(1, name, 512, 4096, 4096, n8_fraction(4096, p))
                for name, p in (("p0", 0.0), ("p10", 0.10), ("p20", 0.20), ("p50", 0.50),
                                ("p100", 1.0))]
    if cfg == 2:
        n8 = llama8b_n8()
        return [Shape(2, name, m, n, k, n8[name]) for name, n, k in LLAMA8B
                for m in (1, 16, 128, 512, 1024)]
    if cfg == 3:
        layers = [("qo", 8192, 8192), ("kv", 1024, 8192), ("gate", 28672, 8192),
                  ("down", 8192, 28672)]
        return [Shape(3, name, m, n, k, n8_fraction(n, 0.10)) for name, n, k in layers
                for m in (512, 1024)]
    if cfg == 4:
        layers = [("gate", 28672, 8192), ("down", 8192, 28672)]
        return [Shape(4, name, m, n, k, n8_fraction(n, 0.10), "t3") for name, n, k in layers
                for m in (1, 4, 8, 32, 256, 2048)]
    raise ValueError(cfg)


HEADLINE = Shape(1, "p10", 512, 4096, 4096, 410)


def make_layer_inputs(shape: Shape):
    """(A fp16 [M, K], W fp16 [N, K], idx8 int32 [n8]) for a shape."""
    return make_acts(shape.m, shape.k, shape.seed, shape.dist), *make_layer_weights(shape)


def make_layer_weights(shape: Shape):
    """(W fp16 [N, K], idx8 int32 [n8]) for a shape; independent of the token count."""
    return make_weights(shape.n, shape.k, shape.wseed), make_idx8(shape.n, shape.n8, shape.wseed)


# Llama-3.1-8B MLP block (hidden 4096, intermediate 14336), 8-bit counts as in llama8b_n8().
MLP8B = dict(hidden=4096, inter=14336)


def mlp_block_inputs(m: int, hidden: int, inter: int, n8: dict, seed=(9,), dist: str = "normal"):
    """(x fp16 [M, hidden], w_gate, w_up [inter, hidden], w_down [hidden, inter] fp16,
    idx8_gate, idx8_up, idx8_down) for an MLP block."""
    key = tuple(seed) + (hidden, inter)
    x = make_acts(m, hidden, key + (m,), dist)
    wg = make_weights(inter, hidden, key + (1,))
    wu = make_weights(inter, hidden, key + (2,))
    wd = make_weights(hidden, inter, key + (3,))
    return (x, wg, wu, wd, make_idx8(inter, n8["gate"], key + (1,)), make_idx8(inter, n8["up"], key + (2,)),
            make_idx8(hidden, n8["down"], key + (3,)))


# Llama-3.1-8B attention input projections: q (4096 channels), k and v (1024 each, grouped
# query attention), all over the 4096-wide hidden state; 8-bit counts as in llama8b_n8().
QKV8B = dict(hidden=4096, q=4096, kv=1024)


def qkv_inputs(m: int, hidden: int, nq: int, nkv: int, n8: dict, seed=(11,), dist: str = "normal"):
    """(x fp16 [M, hidden], w_q [nq, hidden], w_k, w_v [nkv, hidden] fp16, idx8_q, idx8_k,
    idx8_v) for the three projections that read one hidden state."""
    key = tuple(seed) + (hidden, nq, nkv)
    x = make_acts(m, hidden, key + (m,), dist)
    wq = make_weights(nq, hidden, key + (1,))
    wk = make_weights(nkv, hidden, key + (2,))
    wv = make_weights(nkv, hidden, key + (3,))
    return (x, wq, wk, wv, make_idx8(nq, n8["q"], key + (1,)), make_idx8(nkv, n8["k"], key + (2,)),
            make_idx8(nkv, n8["v"], key + (3,)))
