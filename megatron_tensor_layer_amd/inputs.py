"""Seeded synthetic inputs for the tensor-parallel GPT layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the HIP path (through the tests and the benchmark)
and the oracle consume exactly the values produced here.

Recipe
------
* Activations X and the upstream gradient dY: N(0, 1); weights and biases:
  N(0, 0.02^2).  The pages give no distribution; 0.02 is the usual GPT init
  standard deviation, and biases are drawn like weights so that every bias
  path is exercised.
* Draws come from numpy's PCG64 (``default_rng``) in float32, then are
  rounded to bfloat16 by round-to-nearest-even for bf16 configs (kept as
  float32 for the fp32 config).  Returned arrays are float32 holding exactly
  representable values, so the oracle (fp64) and the GPU (bf16 / fp32) see
  identical numbers.
* Seeds are derived from (config name, tensor name, part index) with
  blake2b, so the part of a tensor that one tensor-parallel rank owns can be
  drawn without drawing the rest.  A tensor split along an axis is the
  concatenation of its parts along that axis.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class LayerConfig:
    name: str
    h: int
    a: int
    s: int
    b: int
    t: int
    dtype: str  # "bf16" | "fp32"

    @property
    def d(self) -> int:
        return self.h // self.a

    @property
    def tokens(self) -> int:
        return self.s * self.b

    @property
    def heads_per_rank(self) -> int:
        return self.a // self.t

    @property
    def ffn(self) -> int:
        return 4 * self.h


# The five workloads: a CPU-seconds fp32 check and four GPT shapes
# (1.7B, 18B, 175B and 1T parameters) at sequence length 2048.
CONFIGS = {
    "check_fp32": LayerConfig("check_fp32", h=64, a=4, s=32, b=2, t=4, dtype="fp32"),
    "gpt_1.7b": LayerConfig("gpt_1.7b", h=2304, a=24, s=2048, b=4, t=1, dtype="bf16"),
    "gpt_18b": LayerConfig("gpt_18b", h=6144, a=48, s=2048, b=2, t=8, dtype="bf16"),
    "gpt_175b": LayerConfig("gpt_175b", h=12288, a=96, s=2048, b=1, t=8, dtype="bf16"),
    "gpt_1t": LayerConfig("gpt_1t", h=25600, a=160, s=2048, b=1, t=8, dtype="bf16"),
}


def make_config(name, h, a, s, b, t, dtype) -> LayerConfig:
    return LayerConfig(name, h, a, s, b, t, dtype)


def seed_for(config_name: str, tensor: str, part: int = 0) -> int:
    key = f"{config_name}/{tensor}/{part}".encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(), "little")


def round_to_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 arrays whose low 16 bits are zero."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + rounding) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """The uint16 bit patterns of bf16-exact float32 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def draw(config_name: str, tensor: str, shape, std: float, dtype: str, part: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed_for(config_name, tensor, part))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return round_to_bf16(x) if dtype == "bf16" else x


# --- tensors of the layer ---------------------------------------------------

# name -> (rows, cols, split axis or None) in units of (h, ffn)
def _param_shape(cfg: LayerConfig, name: str):
    h, f = cfg.h, cfg.ffn
    return {
        "Wq": ((h, h), 1), "Wk": ((h, h), 1), "Wv": ((h, h), 1),
        "bq": ((h,), 0), "bk": ((h,), 0), "bv": ((h,), 0),
        "Wo": ((h, h), 0), "bo": ((h,), None),
        "W1": ((h, f), 1), "b1": ((f,), 0),
        "W2": ((f, h), 0), "b2": ((h,), None),
    }[name]


PARAM_NAMES = ("Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo", "bo", "W1", "b1", "W2", "b2")


def param_part(cfg: LayerConfig, name: str, part: int, parts: int | None = None) -> np.ndarray:
    """Part `part` of `parts` (default cfg.t) of a parameter along its split
    axis; replicated parameters (bo, b2) are returned whole."""
    parts = cfg.t if parts is None else parts
    shape, axis = _param_shape(cfg, name)
    if axis is None:
        return draw(cfg.name, name, shape, WEIGHT_STD, cfg.dtype, 0)
    shp = list(shape)
    assert shp[axis] % parts == 0
    shp[axis] //= parts
    return draw(cfg.name, name, tuple(shp), WEIGHT_STD, cfg.dtype, part)


def param_full(cfg: LayerConfig, name: str) -> np.ndarray:
    shape, axis = _param_shape(cfg, name)
    if axis is None:
        return param_part(cfg, name, 0)
    return np.concatenate([param_part(cfg, name, r) for r in range(cfg.t)], axis=axis)


def params_full(cfg: LayerConfig) -> dict:
    return {n: param_full(cfg, n) for n in PARAM_NAMES}


def params_rank(cfg: LayerConfig, r: int) -> dict:
    """The parts of every parameter that rank r owns (replicas whole)."""
    return {n: param_part(cfg, n, r) for n in PARAM_NAMES}


# LayerNorm weights (g1, g2) ~ 1 + N(0, 0.1^2) and biases (be1, be2) ~
# N(0, 0.02^2), each [h] and replicated on every rank.  The pages give no
# initialisation; the spread of the weights around 1 makes a transposed or
# misindexed weight visible in the tests.
LN_WEIGHT_STD = 0.1
LN_NAMES = ("g1", "be1", "g2", "be2")


def ln_param(cfg: LayerConfig, name: str) -> np.ndarray:
    if name in ("g1", "g2"):
        x = draw(cfg.name, name, (cfg.h,), LN_WEIGHT_STD, "fp32") + np.float32(1.0)
        return round_to_bf16(x) if cfg.dtype == "bf16" else x.astype(np.float32)
    return draw(cfg.name, name, (cfg.h,), WEIGHT_STD, cfg.dtype)


def ln_params(cfg: LayerConfig) -> dict:
    return {n: ln_param(cfg, n) for n in LN_NAMES}


def activation(cfg: LayerConfig, name: str = "X", tokens: int | None = None) -> np.ndarray:
    """[tokens, h] token-major activation or gradient, N(0, 1)."""
    T = cfg.tokens if tokens is None else tokens
    return draw(cfg.name, name, (T, cfg.h), 1.0, cfg.dtype)
