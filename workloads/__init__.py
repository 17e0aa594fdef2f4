"""Seeded synthetic inputs for the INT4 weight-only linear layer.

This module is shared by the tests, the smoke check and the benchmark, and by both sides of every
parity check.  It draws random numbers and lays out shapes; it holds none of the quantization
arithmetic (no scales, codes, packing or products).  bf16 inputs are produced by torch's own
fp32 -> bf16 conversion (round to nearest even) and travel as uint16 bit patterns.

Shapes follow the 7B-class decoder the Orin page measures ("模型尺寸和 decode 的真实瓶颈":
28 layers, hidden 3584, KV dim 512, intermediate 18944) and the Gemma MLP of the Lab 5 page
("Linear形状采样").  Weights stand in for trained checkpoints: fp32 N(0, 0.02^2); activations
stand in for live hidden states: fp32 N(0, 1) rounded to bf16.  No dataset is imitated.

Random streams: numpy PCG64, ``default_rng([seed, tensor_id])``; tensor ids are laid out as
``10 * linear_index + {0: W, 1: outlier positions, 2: outlier signs, 3: x, 4: bias,
5: activation-outlier channels}``.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

SYM, ASYM = 0, 1

W_SIGMA = 0.02

TID_W, TID_OUT_POS, TID_OUT_SIGN, TID_X, TID_BIAS, TID_ACT_CH = 0, 1, 2, 3, 4, 5


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor_id])


def tid(linear_index: int, what: int) -> int:
    return 10 * linear_index + what


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16) using torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight(seed: int, lin: int, d_out: int, d_in: int, sigma: float = W_SIGMA) -> np.ndarray:
    """fp32 [d_out][d_in] ~ N(0, sigma^2)."""
    return rng(seed, tid(lin, TID_W)).normal(0.0, sigma, size=(d_out, d_in)).astype(np.float32)


def qat_grid_weight(seed: int, lin: int, d_out: int, d_in: int,
                    off_grid_frac: float = 0.0) -> np.ndarray:
    """bf16 bit patterns [d_out][d_in] standing in for a weight trained on the 4-bit grid (a QAT
    export stored in bf16): per row and 32-column group, a step drawn log-uniformly in
    [2^-10, 2^-6] and rounded to bf16, times integer levels rint(N(0, 2.5^2)) clipped to [-8, 7],
    the product rounded to bf16.  A fraction off_grid_frac of the groups holds N(0, 0.02^2) values
    instead (off the grid).  Nothing here is derived from a weight: the grid is drawn, not found."""
    r = rng(seed, tid(lin, TID_W))
    n_groups = (d_in + 31) // 32
    steps = np.exp2(r.uniform(-10.0, -6.0, size=(d_out, n_groups))).astype(np.float32)
    steps = (to_bf16_bits(steps).astype(np.uint32) << 16).view(np.float32)
    levels = np.clip(np.rint(r.normal(0.0, 2.5, size=(d_out, n_groups, 32))), -8, 7)
    vals = (levels.astype(np.float32) * steps[:, :, None]).reshape(d_out, n_groups * 32)
    if off_grid_frac > 0.0:
        off = r.random((d_out, n_groups)) < off_grid_frac
        noise = r.normal(0.0, W_SIGMA, size=(d_out, n_groups, 32)).astype(np.float32)
        vals = np.where(np.repeat(off, 32, axis=1), noise.reshape(d_out, -1), vals)
    return to_bf16_bits(np.ascontiguousarray(vals[:, :d_in]))


def add_weight_outliers(w: np.ndarray, seed: int, lin: int, frac: float,
                        value: float) -> np.ndarray:
    """Replace round(frac * size) distinct uniformly chosen entries with +-value (fair sign)."""
    n = int(round(frac * w.size))
    pos = rng(seed, tid(lin, TID_OUT_POS)).choice(w.size, size=n, replace=False)
    sign = np.where(rng(seed, tid(lin, TID_OUT_SIGN)).random(n) < 0.5, -1.0, 1.0)
    flat = w.reshape(-1)
    flat[pos] = (sign * value).astype(np.float32)
    return w


def activations(seed: int, lin: int, M: int, K: int, outlier_frac: float = 0.0,
                outlier_scale: float = 1.0) -> np.ndarray:
    """bf16 bits [M][K]; x ~ N(0,1), with round(outlier_frac*K) fixed channels scaled before
    the bf16 rounding (the same channels for every token)."""
    x = rng(seed, tid(lin, TID_X)).normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    if outlier_frac > 0.0:
        n = int(round(outlier_frac * K))
        ch = rng(seed, tid(lin, TID_ACT_CH)).choice(K, size=n, replace=False)
        x[:, ch] *= np.float32(outlier_scale)
    return to_bf16_bits(x)


def bias(seed: int, lin: int, d_out: int) -> np.ndarray:
    """bf16 bits [d_out]; b ~ N(0, 1)."""
    return to_bf16_bits(rng(seed, tid(lin, TID_BIAS)).normal(0.0, 1.0, size=d_out))


@dataclass
class Linear:
    name: str
    d_out: int
    d_in: int
    group_size: int
    mode: int
    weight_outlier_frac: float = 0.0
    weight_outlier_value: float = 0.0
    act_outlier_frac: float = 0.0
    act_outlier_scale: float = 1.0
    with_bias: bool = False


@dataclass
class Config:
    key: str
    seed: int
    description: str
    linears: List[Linear]
    tokens: Tuple[int, ...]
    path: str  # "w4a16" or "w4a8"
    repeat_layers: int = 1  # the decoder step repeats the layer's linear set this many times
    extra: List[Linear] = field(default_factory=list)


HIDDEN, KV_DIM, INTER, N_LAYERS = 3584, 512, 18944, 28

C1 = Config("C1", 101, "tiny single W4A16 linear, g32 symmetric",
            [Linear("tiny", 128, 256, 32, SYM)], (1, 4), "w4a16")

C2 = Config("C2", 202, "decode GEMV, 7B-class MLP, g128 symmetric, 0.1% weight outliers",
            [Linear("gate_up", 2 * INTER, HIDDEN, 128, SYM, 1e-3, 0.5),
             Linear("down", HIDDEN, INTER, 128, SYM, 1e-3, 0.5)], (1,), "w4a16")

C3 = Config("C3", 303, "28-layer decoder-step linear set, g128 asymmetric",
            [Linear("qkv", HIDDEN + 2 * KV_DIM, HIDDEN, 128, ASYM),
             Linear("o", HIDDEN, HIDDEN, 128, ASYM),
             Linear("gate_up", 2 * INTER, HIDDEN, 128, ASYM),
             Linear("down", HIDDEN, INTER, 128, ASYM)], (1, 8, 16), "w4a16",
            repeat_layers=N_LAYERS,
            extra=[Linear("pad3600", HIDDEN, 3600, 128, ASYM)])

C4 = Config("C4", 404, "prefill GEMM, M=2048, g32 symmetric",
            [Linear("qkv", HIDDEN + 2 * KV_DIM, HIDDEN, 32, SYM),
             Linear("gate_up", 2 * INTER, HIDDEN, 32, SYM),
             Linear("down", HIDDEN, INTER, 32, SYM)], (2048,), "w4a16")

C5 = Config("C5", 505, "W4A8 decode GEMV, per-row symmetric weights, 1% activation channels x20",
            [Linear("up", INTER, HIDDEN, 0, SYM, act_outlier_frac=0.01, act_outlier_scale=20.0,
                    with_bias=True),
             Linear("down", HIDDEN, INTER, 0, SYM, act_outlier_frac=0.01,
                    act_outlier_scale=20.0, with_bias=True)], (1,), "w4a8")

CONFIGS = {c.key: c for c in (C1, C2, C3, C4, C5)}


def linear_weight(cfg: Config, lin_index: int, layer: int = 0,
                  lin: Optional[Linear] = None) -> np.ndarray:
    """fp32 weight of linear ``lin_index`` (of layer ``layer`` for the repeated decoder step)."""
    lin = lin if lin is not None else cfg.linears[lin_index]
    index = layer * 100 + lin_index
    w = weight(cfg.seed, index, lin.d_out, lin.d_in)
    if lin.weight_outlier_frac > 0.0:
        add_weight_outliers(w, cfg.seed, index, lin.weight_outlier_frac,
                            lin.weight_outlier_value)
    return w


def linear_x(cfg: Config, lin_index: int, M: int, lin: Optional[Linear] = None,
             layer: int = 0) -> np.ndarray:
    lin = lin if lin is not None else cfg.linears[lin_index]
    return activations(cfg.seed, layer * 100 + lin_index, M, lin.d_in, lin.act_outlier_frac,
                       lin.act_outlier_scale)


def linear_bias(cfg: Config, lin_index: int, lin: Optional[Linear] = None,
                layer: int = 0) -> Optional[np.ndarray]:
    lin = lin if lin is not None else cfg.linears[lin_index]
    if not lin.with_bias:
        return None
    return bias(cfg.seed, layer * 100 + lin_index, lin.d_out)
